"""The allocation-free E2E-TV entry point (specopd_e2etv_fwd_bwd_noalloc)
against the workspace entry point (specopd_e2etv_fwd_bwd) through the C ABI:
the same outputs bitwise, on two calls in a row with the second one smaller
(the static scratch keeps the first call's contents, so whatever must start
at zero has to be cleared by the call itself), on the on-chip bf16 kernel and
the streaming fp32 kernel, and a call too large for the scratch refused."""

import pytest
import torch

import oracle
import speculative_decoding_drafter_amd as sd
from parity import ALPHA_ATOL, check_loss
from synthetic import WORKLOADS, gen_loss, shrink_loss

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _outs(R, Wn, V, dev):
    return {
        "alpha": torch.full((R, Wn), float("nan"), dtype=torch.float32, device=dev),
        "prefix": torch.full((R, Wn), float("nan"), dtype=torch.float32, device=dev),
        "loss": torch.full((3,), float("nan"), dtype=torch.float64, device=dev),
        "grad": torch.full((R, Wn, V), float("nan"), dtype=torch.float32, device=dev),
    }


def _noalloc(inp):
    R, Wn, V = inp["draft"].shape
    desc = sd.e2etv_desc(R, Wn, V, inp["draft"].dtype, torch.float32)
    o = _outs(R, Wn, V, inp["draft"].device)
    sd.specopd_e2etv_fwd_bwd_noalloc(desc, inp["draft"], inp["target"], inp["parent"], o["alpha"],
                                     o["prefix"], o["loss"], o["grad"])
    return o


@pytest.mark.parametrize("dtype,cid,sizes", [
    ("bf16", 3, [(24, 151936), (5, 151936)]),   # resident kernel; fewer rows the second time
    ("f32", 2, [(12, 20000), (3, 4099)]),       # streaming kernel; fewer rows, shorter rows
])
def test_noalloc_matches_workspace_call_twice(gpu_ok, dtype, cid, sizes):
    for i, (R, V) in enumerate(sizes):
        cfg = shrink_loss(WORKLOADS[cid].loss, R=R, V=V, dtype=dtype)
        inp = gen_loss(cfg, 50 + i, device=DEV, cid=cid)
        print(f"noalloc call {i}: R={R} Wn={cfg.Wn} V={V} {dtype}", flush=True)
        got = _noalloc(inp)
        ref = sd.e2etv(inp["draft"], inp["target"], inp["parent"])
        torch.cuda.synchronize()
        assert sd.specopd_e2etv_device_status(ref["desc"], ref["ws"]) == 0
        for key in ("alpha", "prefix", "loss", "grad"):
            assert torch.equal(got[key], ref[key]), (i, key)
        r = oracle.e2etv(inp["draft"].cpu(), inp["target"].cpu(), inp["parent"].cpu(), with_grad=False)
        check_loss(got["loss"][0].item(), r["loss"])
        assert (got["alpha"].cpu().double().numpy() - r["alpha"]).__abs__().max() <= ALPHA_ATOL


def test_noalloc_rejects_a_call_beyond_the_scratch(gpu_ok):
    # 300,000 rows need more than the static scratch holds: refused before
    # anything is enqueued (the pointers are never touched)
    desc = sd.e2etv_desc(100000, 3, 16, torch.bfloat16, torch.float32)
    assert sd.specopd_e2etv_workspace_size(desc) > sd.E2ETV_NOALLOC_SCRATCH_BYTES
    x = torch.zeros(16, dtype=torch.float32, device=DEV)
    st = sd.specopd_e2etv_fwd_bwd_noalloc(desc, x, x[4:], x[8:].view(torch.int32), None, None,
                                          x.view(torch.float64)[4:], None, raw_status=True)
    assert st == sd.SPECOPD_ERR_WORKSPACE
