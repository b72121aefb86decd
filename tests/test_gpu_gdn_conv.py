"""The GDN layer's branch short convolution on the GPU through the C ABI
against the fp64 oracle (jaehun.me review §3.2(c): the convolution history
follows only the branch's ancestors).

Every output element at reduced sizes (chains and the forked tree, head
sizes 64 and 128, widths 1 to 8, with and without the per-head unit
scaling, bf16 and fp32), anchors at the trunk's start (zero history),
malformed parent maps, sampled branches at the full workload sizes, and
run-to-run determinism.

Tolerance.  The kernel sums at most 8 fp32 products per channel in the
oracle's order, applies SiLU with the hardware exponential and an IEEE
division, and for unit heads one fp32 sum of squares over D values; that
is a few fp32 roundings (~1e-7 relative) on values of order one, so fp32
outputs are checked to 1e-5 + 1e-5 |ref|.  bf16 outputs are that fp32
value rounded to bf16, which may land on either neighbour of a value near
a rounding boundary: one bf16 unit, 2^-7 |ref|, plus 1e-5."""

import numpy as np
import pytest
import torch

import oracle
import speculative_decoding_drafter_amd as sd
from synthetic import WORKLOADS, chain, gen_gdn_conv, shrink_gdn

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


def _tol(dtype):
    return (1e-5, 2.0 ** -7) if dtype == "bf16" else (1e-5, 1e-5)


def _check(got, ref, dtype, what=""):
    atol, rtol = _tol(dtype)
    got = got.float().cpu().numpy().astype(np.float64) if torch.is_tensor(got) else got
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bad = err > atol + rtol * np.abs(ref)
    assert not bad.any(), f"{what}: {bad.sum()} elements out of tolerance, max err {err.max():.3e}"


def _ref(inp, D, l2norm, branches=None):
    return oracle.gdn_branch_conv(_np(inp["trunk_x"]), _np(inp["x"]), inp["w"].cpu().numpy().astype(np.float64),
                                  inp["anchors"].cpu().numpy(), inp["parent"].cpu().numpy(), D=D, l2norm=l2norm,
                                  branches=branches)


@pytest.mark.parametrize("cid,kw,K,l2", [
    (3, dict(T=2, L=300, P=64, B=5, H=3, D=128, dtype="bf16"), 4, True),    # chains of 16, q/k style
    (3, dict(T=2, L=300, P=64, B=5, H=3, D=128, dtype="bf16"), 4, False),   # v style
    (5, dict(T=1, L=200, P=30, B=6, H=2, D=128, dtype="bf16"), 4, True),    # forked tree
    (5, dict(T=1, L=150, P=20, B=4, H=5, D=64, dtype="f32"), 3, True),      # fp32, D=64, odd head count
    (2, dict(T=3, L=130, P=10, B=4, H=4, D=64, dtype="bf16"), 1, False),    # width one
    (2, dict(T=1, L=130, P=10, B=4, H=2, D=128, dtype="f32"), 8, False),    # the widest window
])
def test_reduced_workloads(gpu_ok, cid, kw, K, l2):
    cfg = shrink_gdn(WORKLOADS[cid].gdn, **kw)
    inp = gen_gdn_conv(cfg, 3, device=DEV, cid=cid, K=K)
    out, _ = sd.gdn_conv(inp["trunk_x"], inp["x"], inp["w"], inp["anchors"], inp["parent"], cfg.H, l2norm=l2)
    torch.cuda.synchronize()
    _check(out, _ref(inp, cfg.D, l2), cfg.dtype, f"wl{cid} {kw} K={K} l2={l2}")


def test_anchors_at_the_trunk_start(gpu_ok):
    """Anchors 0, 1 and 2 with K = 4: a root's window runs past token 0 and
    reads zeros there."""
    cfg = shrink_gdn(WORKLOADS[3].gdn, T=1, L=64, P=0, B=4, H=2, D=128, parent=chain(3)[0], dtype="f32")
    inp = gen_gdn_conv(cfg, 4, device=DEV, cid=3, K=4)
    inp["anchors"] = torch.tensor([[0, 1, 2, 63]], dtype=torch.int32, device=DEV)
    out, _ = sd.gdn_conv(inp["trunk_x"], inp["x"], inp["w"], inp["anchors"], inp["parent"], cfg.H)
    torch.cuda.synchronize()
    _check(out, _ref(inp, cfg.D, False), cfg.dtype, "anchors at the start")


def test_malformed_parent_maps_give_nan_where_the_window_meets_them(gpu_ok):
    cfg = shrink_gdn(WORKLOADS[3].gdn, T=1, L=100, P=0, B=3, H=2, D=64, parent=chain(6)[0], dtype="f32")
    inp = gen_gdn_conv(cfg, 5, device=DEV, cid=3, K=3)
    inp["anchors"][0, 0] = 100            # outside the trunk: every node
    inp["parent"][0, 1, 4] = 4            # node 4 its own parent: nodes 4 and 5 read it
    out, _ = sd.gdn_conv(inp["trunk_x"], inp["x"], inp["w"], inp["anchors"], inp["parent"], cfg.H)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.isnan(got[0, 0]).all()
    assert np.isnan(got[0, 1, 4:]).all()
    good = inp["parent"].clone()
    good[0, 1, 4] = 3
    inp_ok = dict(inp, parent=good)
    inp_ok["anchors"] = inp["anchors"].clone()
    inp_ok["anchors"][0, 0] = 10
    ref = _ref(inp_ok, cfg.D, False)
    _check(got[0, 1, :4], ref[0, 1, :4], cfg.dtype, "nodes before the bad link")
    _check(got[0, 2], ref[0, 2], cfg.dtype, "untouched branch")


def _branch_ref(inp, t, b, K, D, l2):
    """One branch's outputs from the oracle, reading only the trunk rows its
    windows can reach (a - K + 1 .. a)."""
    a = int(inp["anchors"][t, b])
    lo = max(0, a - K + 1)
    tx = _np(inp["trunk_x"][t, lo:a + 1])
    return oracle.branch_conv(tx, _np(inp["x"][t, b]), inp["w"].cpu().numpy().astype(np.float64), a - lo,
                              inp["parent"][t, b].cpu().numpy(), D=D, l2norm=l2)


@pytest.mark.parametrize("cid", [2, 3, 5])
def test_full_size_sampled_branches(gpu_ok, cid):
    cfg = WORKLOADS[cid].gdn
    inp = gen_gdn_conv(cfg, 0, device=DEV, cid=cid, K=4)
    for l2 in (True, False):
        out, _ = sd.gdn_conv(inp["trunk_x"], inp["x"], inp["w"], inp["anchors"], inp["parent"], cfg.H, l2norm=l2)
        torch.cuda.synchronize()
        rng = np.random.default_rng(cid)
        picks = sorted({(int(rng.integers(cfg.T)), int(rng.integers(cfg.B))) for _ in range(4)})
        for t, b in picks:
            _check(out[t, b], _branch_ref(inp, t, b, 4, cfg.D, l2), cfg.dtype, f"wl{cid} branch {(t, b)} l2={l2}")


def test_deterministic_and_timed(gpu_ok):
    cfg = shrink_gdn(WORKLOADS[5].gdn, T=1, L=400, P=64, B=32, H=4, D=128)
    inp = gen_gdn_conv(cfg, 6, device=DEV, cid=5)
    a, _ = sd.gdn_conv(inp["trunk_x"], inp["x"], inp["w"], inp["anchors"], inp["parent"], cfg.H, l2norm=True)
    sd.specopd_kernel_timing(True)
    b, _ = sd.gdn_conv(inp["trunk_x"], inp["x"], inp["w"], inp["anchors"], inp["parent"], cfg.H, l2norm=True)
    torch.cuda.synchronize()
    ms, n = sd.specopd_kernel_time(4)
    sd.specopd_kernel_timing(False)
    assert torch.equal(a, b)
    assert n == 1 and ms > 0
