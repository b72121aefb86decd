"""Batch-invariant tree scoring (SPECOPD_TREE_BATCH_INVARIANT) on the GPU.

The jaehun.me review (§3.2, "maintaining numerical consistency", Table 4)
states that with deterministic target inference full recomputation, single
and batched cached scoring and merged tree execution give the same logits
exactly.  Here: a branch scored alone, inside the full workload batch and
inside a permuted batch (trunks reversed, branches shuffled) must give
bitwise the same rows, at the full sizes of the 8B-layer, 8-trunk and
long-context workloads; and those rows still match the oracle."""

import numpy as np
import pytest
import torch

import oracle
import speculative_decoding_drafter_amd as sd
from parity import check_attention
from synthetic import WORKLOADS, gen_attn, shrink_attn

pytestmark = pytest.mark.gpu
DEV = "cuda"
BI = sd.SPECOPD_TREE_BATCH_INVARIANT


def _call(inp, flags=BI):
    out, desc, ws = sd.tree_attn(inp, flags=flags)
    torch.cuda.synchronize()
    assert sd.specopd_tree_attn_device_status(desc, ws) == 0
    return out


def _subset(inp, t, bs):
    """Trunk t with branches bs only, as a call of its own (fresh, aligned
    copies)."""
    idx = torch.tensor(bs, device=inp["q"].device)
    return {
        "trunk_k": inp["trunk_k"][t:t + 1].clone(), "trunk_v": inp["trunk_v"][t:t + 1].clone(),
        "q": inp["q"][t:t + 1, idx].clone(), "k": inp["k"][t:t + 1, idx].clone(),
        "v": inp["v"][t:t + 1, idx].clone(), "anchors": inp["anchors"][t:t + 1, idx].clone(),
        "parent": inp["parent"][t:t + 1, idx].clone(), "pos": inp["pos"][t:t + 1, idx].clone(),
    }


def _permuted(inp, tperm, bperm):
    out = {}
    for k, v in inp.items():
        x = v[tperm]
        if k not in ("trunk_k", "trunk_v"):
            x = x[:, bperm]
        out[k] = x.contiguous()
    return out


@pytest.mark.parametrize("cid", [2, 3, 5])
def test_branch_alone_in_batch_and_permuted_bitwise(gpu_ok, cid):
    cfg = WORKLOADS[cid].attn
    print(f"workload {cid}: T={cfg.T} B={cfg.B} Wn={cfg.Wn} Hq={cfg.Hq}/{cfg.Hkv} D={cfg.D}", flush=True)
    inp = gen_attn(cfg, 0, device=DEV, cid=cid)
    full = _call(inp)
    rng = np.random.default_rng(100 + cid)
    tperm = torch.arange(cfg.T - 1, -1, -1, device=DEV)
    bperm = torch.tensor(rng.permutation(cfg.B), device=DEV)
    perm = _call(_permuted(inp, tperm, bperm))
    back = torch.empty_like(perm)
    back[tperm[:, None], bperm[None, :]] = perm
    assert torch.equal(back, full), "permuted batch differs"
    # branches alone and in small groups: every trunk, the longest and the
    # shortest anchors, random ones
    anch = inp["anchors"].cpu().numpy()
    picks = []
    for t in range(cfg.T):
        picks += [(t, int(anch[t].argmax())), (t, int(anch[t].argmin()))]
        picks += [(t, int(b)) for b in rng.choice(cfg.B, size=2, replace=False)]
    for (t, b) in picks:
        alone = _call(_subset(inp, t, [b]))
        assert torch.equal(alone[0, 0], full[t, b]), f"branch ({t},{b}) alone differs"
    t = cfg.T - 1
    group = sorted(int(b) for b in rng.choice(cfg.B, size=min(5, cfg.B), replace=False))
    sub = _call(_subset(inp, t, group))
    for i, b in enumerate(group):
        assert torch.equal(sub[0, i], full[t, b]), f"branch ({t},{b}) in a group of 5 differs"
    # and the rows are still right
    few = sorted(set(picks[:4]))
    c = {k: v.cpu() for k, v in inp.items()}
    ref = oracle.tree_attention(c["trunk_k"], c["trunk_v"], c["q"], c["k"], c["v"], c["anchors"],
                                c["parent"], c["pos"], branches=few)
    got = full.float().cpu().numpy()
    for (t, b) in few:
        check_attention(got[t, b], ref[t, b], what=f"branch ({t},{b})")


def test_flag_changes_nothing_when_the_call_fills_the_gpu(gpu_ok):
    """A call with enough (trunk, kv head, pack) units to fill the GPU is
    scored in one pass per pack with or without the flag: same bits."""
    cfg = WORKLOADS[3].attn
    inp = gen_attn(cfg, 1, device=DEV, cid=3)
    assert torch.equal(_call(inp, flags=0), _call(inp, flags=BI))


@pytest.mark.parametrize("seed", range(6))
def test_random_shapes_subsets_bitwise(gpu_ok, seed):
    """Seeded random shapes (trees of 1..40 nodes, 1..16 query heads per kv
    head, D of 64/128/256): each branch alone equals its rows in the whole
    call, bitwise."""
    rng = np.random.default_rng(4000 + seed)
    Wn = int(rng.integers(1, 41))
    parent = [-1] + [int(rng.integers(-1, j)) for j in range(1, Wn)]
    depth = []
    for j in range(Wn):
        d, k = 0, j
        while parent[k] != -1:
            k = parent[k]
            d += 1
        depth.append(d)
    D = int(rng.choice([64, 128, 256]))
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    B = int(rng.integers(2, 24))
    L = int(rng.integers(B + 40, 3000))
    cfg = shrink_attn(WORKLOADS[2].attn, T=int(rng.integers(1, 3)), L=L, P=int(rng.integers(0, L - B)),
                      B=B, Hq=G * Hkv, Hkv=Hkv, D=D, parent=tuple(parent), depth=tuple(depth))
    print(f"random shape {seed}: {cfg}", flush=True)
    inp = gen_attn(cfg, 60 + seed, device=DEV, cid=2)
    full = _call(inp)
    for t in range(cfg.T):
        for b in rng.choice(B, size=min(3, B), replace=False):
            alone = _call(_subset(inp, t, [int(b)]))
            assert torch.equal(alone[0, 0], full[t, int(b)]), f"branch ({t},{b})"
