"""Calls enqueue on the stream they are given: on a side stream, with the
inputs produced on the default stream before it and the outputs read after
an explicit synchronisation, every call gives bitwise what it gives on the
default stream."""

import pytest
import torch

import speculative_decoding_drafter_amd as sd
from synthetic import WORKLOADS, gen_attn, gen_loss, gen_prefill, shrink_attn, shrink_loss

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_calls_on_a_side_stream_match_the_default_stream(gpu_ok):
    acfg = shrink_attn(WORKLOADS[2].attn, L=700, P=150, B=6)
    ai = gen_attn(acfg, 21, device=DEV, cid=2)
    lcfg = shrink_loss(WORKLOADS[2].loss, R=3)
    li = gen_loss(lcfg, 21, device=DEV, cid=2)
    pcfg = shrink_attn(WORKLOADS[2].attn, L=300)
    pi = gen_prefill(pcfg, 21, device=DEV, cid=2)

    a0, adesc, aws = sd.tree_attn(ai)
    l0 = sd.e2etv(li["draft"], li["target"], li["parent"])
    p0 = sd.prefill(pi["q"], pi["k"], pi["v"])
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    a1 = torch.empty_like(a0)
    aws1 = torch.empty_like(aws)
    l1 = {k: (torch.empty_like(v) if isinstance(v, torch.Tensor) else v) for k, v in l0.items()
          if k in ("alpha", "prefix", "loss", "grad")}
    lws1 = torch.empty_like(l0["ws"])
    pouts = tuple(torch.empty_like(x) for x in p0[:3])
    pws1 = torch.empty_like(p0[4])
    with torch.cuda.stream(side):
        sd.specopd_tree_attn_fwd(adesc, ai["trunk_k"], ai["trunk_v"], ai["q"], ai["k"], ai["v"],
                                 ai["anchors"], ai["parent"], ai["pos"], a1, aws1, stream=side.cuda_stream)
        sd.specopd_e2etv_fwd_bwd(l0["desc"], li["draft"], li["target"], li["parent"], l1["alpha"],
                                 l1["prefix"], l1["loss"], l1["grad"], lws1, stream=side.cuda_stream)
        sd.specopd_prefill_fwd(p0[3], pi["q"], pi["k"], pi["v"], pouts[1], pouts[2], pouts[0], pws1,
                               stream=side.cuda_stream)
    side.synchronize()
    assert torch.equal(a1, a0)
    for key in ("alpha", "prefix", "loss", "grad"):
        assert torch.equal(l1[key], l0[key]), key
    for x, y in zip(pouts, p0[:3]):
        assert torch.equal(x, y)
