"""QSA block selection with branch-consistent indexer groups on the GPU
through the C ABI, against the fp64 oracle (jaehun.me review §3.2(b)).

Covered: the trunk pass's group cache; every node's kept groups, their
scores and the keys of the groups a node completes, at reduced sizes
(chains, the forked tree, random trees, 64-node branches that take two
matrix-core row blocks, index key sizes 64, 128 and 256, every anchor
residue mod 4, fewer candidates than k); the whole pipeline with each side
building its own trunk cache from the raw keys; malformed trees; sampled
branches at the full workload sizes; run-to-run determinism.

Tolerance (derived from the arithmetic).  The kernel rounds the rotated
query and the keys it compresses to bf16 (the matrix cores' operands) and
sums their products in fp32; the oracle keeps both in fp64.  A rounding to
bf16 moves each factor by at most 2^-9 of itself, so a score moves by at
most about 2^-8 sum_i |y_i k_i| (both factors rounded), plus fp32 rounding of
angles and sums (~1e-6 relative): the check allows 1.25 * 2^-8 sum_i
|y_i k_i| + 1e-5 per score, computed from the oracle's own factors.  Which
groups are kept is an integer decision taken on those scores, so where two
candidates' scores lie within that allowance of the k-th the kernel may
keep either: the check is that every kept group's oracle score is at least
the oracle's k-th score minus twice the row's allowance and every group left
out is at most the k-th plus twice it, and the kept sets must agree exactly
on at least 97% of the nodes with the oracle taking the decision in the
kernel's precision (rotated query and compressed keys rounded to bf16 before
exact products: only fp32 summation order and rare one-unit differences in
a rounded operand then separate the two).  Counts of kept groups (the candidates complete
at the node's position) are exact.  Compressed keys are compared with the
bf16 bound: one bf16 unit, 2^-7 |ref|, plus 1e-3."""

import numpy as np
import pytest
import torch

import oracle
import speculative_decoding_drafter_amd as sd
from oracle.rope import rope
from synthetic import WORKLOADS, chain, gen_qsa, shrink_qsa

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


def _host(inp):
    return {k: (_np(v) if v.dtype in (torch.bfloat16, torch.float32) else v.cpu().numpy())
            for k, v in inp.items()}


def _depths(parent):
    d = []
    for j, p in enumerate(parent):
        d.append(0 if p < 0 else d[p] + 1)
    return np.array(d)


def _tree_inputs(cfg, seed, cid, parent=None):
    inp = gen_qsa(cfg, seed, device=DEV, cid=cid)
    if parent is not None:
        T, B, Wn = inp["parent"].shape
        par = np.asarray(parent, np.int32).reshape(T, B, Wn)
        anch = inp["anchors"].cpu().numpy()
        pos = np.zeros_like(par)
        for t in range(T):
            for b in range(B):
                pos[t, b] = anch[t, b] + 1 + _depths(par[t, b])
        inp["parent"] = torch.from_numpy(par).to(DEV)
        inp["pos"] = torch.from_numpy(pos).to(DEV)
    return inp


def _check_branch(h, out, t, b, k, ref, agree, ref_bf=None):
    """Compare one branch's GPU selection with the oracle's result `ref`."""
    sel = out["sel"][t, b].cpu().numpy()
    score = out["score"][t, b].cpu().numpy().astype(np.float64)
    bkey = _np(out["bkey"][t, b]) if out.get("bkey") is not None else None
    pos = h["pos"][t, b]
    y = h["y"][t, b]
    for j in range(sel.shape[0]):
        s_o = ref["scores"][j]
        n = int(ref["ncand"][j])
        kept = sel[j][sel[j] >= 0]
        assert kept.shape[0] == min(n, k), f"({t},{b},{j}): {kept.shape[0]} kept, want {min(n, k)}"
        assert (np.diff(kept) > 0).all() and (kept < n).all(), f"({t},{b},{j}): not increasing or out of range"
        assert (sel[j][kept.shape[0]:] == -1).all() and np.isneginf(score[j][kept.shape[0]:]).all()
        if n == 0:
            agree.append(True)
            continue
        # per-score allowance from the oracle's factors
        yr = rope(y[j], int(pos[j]))
        keys = ref["keys"][j]
        allow = 1.25 * 2.0 ** -8 * (np.abs(keys) @ np.abs(yr)) + 1e-5
        err = np.abs(score[j][:kept.shape[0]] - s_o[kept])
        assert (err <= allow[kept]).all(), f"({t},{b},{j}): score error {err.max():.3e}"
        if n > k:
            tau = np.sort(s_o)[::-1][k - 1]
            slack = 2.0 * allow.max()
            out_set = np.setdiff1d(np.arange(n), kept)
            assert s_o[kept].min() >= tau - slack, f"({t},{b},{j}): a kept group scores below the k-th"
            assert s_o[out_set].max() <= tau + slack, f"({t},{b},{j}): a dropped group scores above the k-th"
        rs = (ref if ref_bf is None else ref_bf)["sel"][j]
        agree.append(np.array_equal(kept, rs[rs >= 0]))
        if bkey is not None:
            if ref["bgroup"][j] >= 0:
                d = np.abs(bkey[j] - ref["bkey"][j])
                assert (d <= 1e-3 + 2.0 ** -7 * np.abs(ref["bkey"][j])).all(), f"({t},{b},{j}): key"
            else:
                assert (bkey[j] == 0).all()


def _oracle_branch(h, t, b, k, gk=None, operands="f64"):
    gk_t = h["trunk_gk"][t] if gk is None else gk[t]
    ref = oracle.qsa_branch_select(gk_t, h["trunk_raw"][t], h["x"][t, b], h["y"][t, b],
                                   int(h["anchors"][t, b]), h["parent"][t, b], h["pos"][t, b],
                                   h["gamma"], k, operands=operands)
    # every candidate key of every node, for the allowance
    a = int(h["anchors"][t, b])
    gt = (a + 1) // 4
    keys = []
    for j in range(h["x"].shape[2]):
        n = int(ref["ncand"][j])
        kk = np.empty((n, gk_t.shape[1]))
        kk[:min(n, gt)] = gk_t[:min(n, gt)]
        for i in oracle.walk_ancestors(h["parent"][t, b], j):
            if ref["bgroup"][i] >= 0:
                kk[ref["bgroup"][i]] = ref["bkey"][i]
        keys.append(kk)
    ref["keys"] = keys
    return ref


def _run_and_check(inp, k, branches=None, min_agree=0.97):
    out = sd.qsa_select(inp, k)
    torch.cuda.synchronize()
    assert sd.specopd_qsa_device_status(out["desc"], out["ws"]) == 0
    h = _host(inp)
    T, B = h["anchors"].shape
    todo = branches if branches is not None else [(t, b) for t in range(T) for b in range(B)]
    agree = []
    for (t, b) in todo:
        _check_branch(h, out, t, b, k, _oracle_branch(h, t, b, k), agree,
                      _oracle_branch(h, t, b, k, operands="bf16"))
    assert np.mean(agree) >= min_agree, f"kept sets agree on {np.mean(agree):.3f} of nodes"
    return out


@pytest.mark.parametrize("Di", [64, 128, 256])
def test_trunk_group_cache(gpu_ok, Di):
    cfg = shrink_qsa(WORKLOADS[2].qsa, T=2, L=203, P=40, B=3, Di=Di)
    inp = gen_qsa(cfg, 11, device=DEV, cid=2)
    gk = sd.qsa_trunk_groups(inp["trunk_raw"], inp["gamma"])
    torch.cuda.synchronize()
    assert gk.shape == (2, 50, Di)
    h = _host(inp)
    for t in range(2):
        ref = oracle.sequence_group_keys(h["trunk_raw"][t], h["gamma"])
        got = _np(gk[t])
        d = np.abs(got - ref)
        assert (d <= 1e-3 + 2.0 ** -7 * np.abs(ref)).all(), f"trunk {t}: max err {d.max():.3e}"
    # far positions: the angle reduction keeps long trunks exact enough
    cfg = shrink_qsa(WORKLOADS[5].qsa, L=32768, B=1, Di=Di)
    inp = gen_qsa(cfg, 12, device=DEV, cid=5)
    gk = sd.qsa_trunk_groups(inp["trunk_raw"], inp["gamma"])
    h = _host(inp)
    for g in (0, 4095, 8191):
        ref = oracle.compress_group(h["trunk_raw"][0, 4 * g:4 * g + 4], h["gamma"], 4 * g)
        d = np.abs(_np(gk[0, g]) - ref)
        assert (d <= 1e-3 + 2.0 ** -7 * np.abs(ref)).all(), f"group {g}: max err {d.max():.3e}"


@pytest.mark.parametrize("cid,kw,k", [
    (1, dict(), 4),                                                         # tiny: chains of 4, Di 64
    (2, dict(L=700, P=100, B=12), 16),                                      # chains of 8, Di 128
    (3, dict(T=2, L=900, P=200, B=9), 40),                                  # chains of 16, two trunks
    (5, dict(L=1200, P=300, B=10), 24),                                     # forked tree
    (5, dict(L=1100, P=300, B=6, Di=256), 32),                              # Di 256
    (2, dict(L=400, P=50, B=5, Di=64), 200),                                # k above most counts
])
def test_selection_matches_oracle(gpu_ok, cid, kw, k):
    cfg = shrink_qsa(WORKLOADS[cid].qsa, **kw)
    inp = gen_qsa(cfg, 21 + cid, device=DEV, cid=cid)
    _run_and_check(inp, k)


@pytest.mark.parametrize("seed", range(3))
def test_random_trees_and_wide_branches(gpu_ok, seed):
    rng = np.random.default_rng(seed)
    Wn = [13, 40, 64][seed]
    cfg = shrink_qsa(WORKLOADS[2].qsa, L=900, P=100, B=5, parent=chain(Wn)[0], Di=[64, 128, 256][seed])
    par = []
    for _ in range(cfg.B):
        par.append([-1] + [int(rng.integers(max(0, j - 6), j)) for j in range(1, Wn)])
    inp = _tree_inputs(cfg, 31 + seed, 2, parent=par)
    _run_and_check(inp, [7, 30, 12][seed])


def test_every_anchor_residue_and_short_histories(gpu_ok):
    cfg = shrink_qsa(WORKLOADS[2].qsa, L=300, P=0, B=12, parent=chain(9)[0], Di=128)
    inp = gen_qsa(cfg, 41, device=DEV, cid=2)
    # anchors 0..11 cover every residue mod 4 and histories with no complete group
    inp["anchors"] = torch.arange(12, dtype=torch.int32, device=DEV).view(1, 12) * 7 % 60
    inp["anchors"][0, :4] = torch.tensor([0, 1, 2, 3], dtype=torch.int32)
    a = inp["anchors"].cpu().numpy()
    inp["pos"] = torch.from_numpy((a[:, :, None] + 1 + np.arange(9)[None, None, :]).astype(np.int32)).to(DEV)
    _run_and_check(inp, 5)


def test_pipeline_with_own_trunk_caches(gpu_ok):
    """Each side builds the trunk cache from the raw keys itself; the kept
    groups then equal the plain-sequence selection of the oracle."""
    cfg = shrink_qsa(WORKLOADS[5].qsa, L=1500, P=300, B=8, Di=128)
    inp = gen_qsa(cfg, 51, device=DEV, cid=5)
    inp["trunk_gk"] = sd.qsa_trunk_groups(inp["trunk_raw"], inp["gamma"])
    out = sd.qsa_select(inp, 20)
    torch.cuda.synchronize()
    h = _host(inp)
    gk_o = np.stack([oracle.sequence_group_keys(h["trunk_raw"][t], h["gamma"]) for t in range(cfg.T)])
    agree = []
    for b in range(cfg.B):
        # the GPU's cache is its own bf16 rounding of these keys: the allowance
        # (both factors of a score rounded) covers it
        ref = _oracle_branch(h, 0, b, 20, gk=gk_o)
        _check_branch(h, out, 0, b, 20, ref, agree)
        for j in range(cfg.Wn):  # the oracle's own exactness statement on this branch
            path = oracle.walk_ancestors(h["parent"][0, b], j)[::-1]
            a = int(h["anchors"][0, b])
            seq = np.concatenate([h["trunk_raw"][0, :a + 1], h["x"][0, b][path]], axis=0)
            sel, _, _ = oracle.plain_row_select(seq, h["y"][0, b, j], h["gamma"], 20)
            assert np.array_equal(sel, ref["sel"][j][:sel.shape[0]])
    assert np.mean(agree) >= 0.97


def test_malformed_branches_are_flagged(gpu_ok):
    cfg = shrink_qsa(WORKLOADS[2].qsa, L=500, P=50, B=6)
    inp = gen_qsa(cfg, 61, device=DEV, cid=2)
    par = inp["parent"].clone()
    pos = inp["pos"].clone()
    anc = inp["anchors"].clone()
    par[0, 1, 3] = 5                  # a parent after its child
    pos[0, 2, 4] += 1                 # position not anchor + 1 + depth
    anc[0, 3] = cfg.L                 # anchor outside the trunk
    par[0, 4, 0] = 0                  # a node its own parent
    bad = dict(inp, parent=par, pos=pos, anchors=anc)
    out = sd.qsa_select(bad, 8)
    torch.cuda.synchronize()
    assert sd.specopd_qsa_device_status(out["desc"], out["ws"]) == 4
    for b in (1, 2, 3, 4):
        assert (out["sel"][0, b] == -1).all()
        assert torch.isnan(out["score"][0, b]).all()
        assert (out["bkey"][0, b].float() == 0).all()
    # the well-formed branches are untouched by their neighbours
    good = sd.qsa_select(inp, 8)
    torch.cuda.synchronize()
    for b in (0, 5):
        assert torch.equal(out["sel"][0, b], good["sel"][0, b])
        assert torch.equal(out["score"][0, b], good["score"][0, b])


def test_deterministic(gpu_ok):
    cfg = shrink_qsa(WORKLOADS[5].qsa, L=4000, P=800, B=16)
    inp = gen_qsa(cfg, 71, device=DEV, cid=5)
    a = sd.qsa_select(inp, 64)
    b = sd.qsa_select(inp, 64)
    torch.cuda.synchronize()
    for key in ("sel", "score", "bkey"):
        assert torch.equal(a[key], b[key]), key


@pytest.mark.parametrize("cid", [2, 3, 5])
def test_full_size_sampled_branches(gpu_ok, cid):
    cfg = WORKLOADS[cid].qsa
    inp = gen_qsa(cfg, 0, device=DEV, cid=cid)
    out = sd.qsa_select(inp, cfg.topk)
    torch.cuda.synchronize()
    assert sd.specopd_qsa_device_status(out["desc"], out["ws"]) == 0
    rng = np.random.default_rng(cid)
    branches = [(int(rng.integers(cfg.T)), int(rng.integers(cfg.B))) for _ in range(6)]
    anch = inp["anchors"].cpu().numpy()
    # the branches with the longest and the shortest history too
    t0 = int(np.unravel_index(anch.argmax(), anch.shape)[0]), int(np.unravel_index(anch.argmax(), anch.shape)[1])
    t1 = int(np.unravel_index(anch.argmin(), anch.shape)[0]), int(np.unravel_index(anch.argmin(), anch.shape)[1])
    branches += [t0, t1]
    h = inp
    hh = {"anchors": anch, "parent": inp["parent"].cpu().numpy(), "pos": inp["pos"].cpu().numpy(),
          "gamma": inp["gamma"].cpu().numpy().astype(np.float64)}
    ts = sorted({t for t, _ in branches})
    hh["trunk_gk"] = {t: _np(h["trunk_gk"][t]) for t in ts}
    hh["trunk_raw"] = {t: _np(h["trunk_raw"][t]) for t in ts}
    hh["x"] = _np(h["x"])
    hh["y"] = _np(h["y"])
    agree = []
    for (t, b) in branches:
        _check_branch(hh, out, t, b, cfg.topk, _oracle_branch(hh, t, b, cfg.topk), agree,
                      _oracle_branch(hh, t, b, cfg.topk, operands="bf16"))
    assert np.mean(agree) >= 0.97
