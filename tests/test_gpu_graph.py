"""The calls under HIP graph capture: a graph holding a tree-attention call,
an E2E-TV call and a trunk prefill, replayed several times with the
program's own eager work and synchronisations in between, must give every
time bitwise what the eager calls give (the library records no memset and
allocates nothing, so its kernels are all that a replay runs)."""

import pytest
import torch

import speculative_decoding_drafter_amd as sd
from synthetic import WORKLOADS, gen_attn, gen_loss, gen_prefill, shrink_attn, shrink_loss

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_graph_replays_match_eager_calls(gpu_ok):
    acfg = shrink_attn(WORKLOADS[2].attn, L=900, P=200, B=8)
    ai = gen_attn(acfg, 31, device=DEV, cid=2)
    lcfg = shrink_loss(WORKLOADS[2].loss, R=4)
    li = gen_loss(lcfg, 31, device=DEV, cid=2)
    pcfg = shrink_attn(WORKLOADS[2].attn, L=500)
    pi = gen_prefill(pcfg, 31, device=DEV, cid=2)

    # eager results
    a_ref, adesc, aws = sd.tree_attn(ai)
    l_ref = sd.e2etv(li["draft"], li["target"], li["parent"])
    p_ref = sd.prefill(pi["q"], pi["k"], pi["v"])
    torch.cuda.synchronize()
    a_ref = a_ref.clone()
    l_ref_vals = {k: l_ref[k].clone() for k in ("alpha", "prefix", "loss", "grad")}
    p_ref_vals = [x.clone() for x in p_ref[:3]]

    # buffers the graph writes
    a_out = torch.empty_like(a_ref)
    l_outs = {k: torch.empty_like(v) for k, v in l_ref_vals.items()}
    l_outs["desc"], l_outs["ws"] = l_ref["desc"], torch.empty_like(l_ref["ws"])
    p_outs = tuple(torch.empty_like(x) for x in p_ref_vals)
    p_ws = torch.empty_like(p_ref[4])
    a_ws = torch.empty_like(aws)

    def work():
        sd.tree_attn(ai, ws=a_ws, out=a_out)
        sd.e2etv(li["draft"], li["target"], li["parent"], ws=l_outs["ws"], outs=l_outs)
        sd.prefill(pi["q"], pi["k"], pi["v"], ws=p_ws, outs=p_outs)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work()  # warm up off the default stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    for rep in range(3):
        # the program's own eager work between replays: clobber the outputs
        a_out.fill_(7.0)
        for v in l_outs.values():
            if isinstance(v, torch.Tensor) and v is not l_outs["ws"]:
                v.fill_(7.0)
        for x in p_outs:
            x.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(a_out, a_ref), f"replay {rep}: attention"
        for k in ("alpha", "prefix", "loss", "grad"):
            assert torch.equal(l_outs[k], l_ref_vals[k]), f"replay {rep}: {k}"
        for x, y in zip(p_outs, p_ref_vals):
            assert torch.equal(x, y), f"replay {rep}: prefill"
