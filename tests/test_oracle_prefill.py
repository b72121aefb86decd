"""Pins of the trunk-prefill oracle (oracle.trunk_prefill): a library causal
attention over keys rotated by complex arithmetic, closed forms for the
first token and for constant values, the cache contents, and the pages'
consistency claim in its four forms — full recomputation (R), cached
scoring one branch at a time (C1) and in a batch (CB), and the merged tree
(T) — computed by the tree oracle from the prefill's cache ([R] §3.2,
Table 4).  A planted off-by-one in the causal mask fails the library pin."""

import numpy as np
import pytest
import torch

import oracle


def _complex_rope(x, pos, base=10000.0):
    """Rotate-half pairs as complex numbers, an independent statement of the
    rotary convention (x: [L][H][D], pos: [L])."""
    D = x.shape[-1]
    h = D // 2
    z = x[..., :h] + 1j * x[..., h:]
    freqs = base ** (-np.arange(0, D, 2) / D)
    z = z * np.exp(1j * pos[:, None, None] * freqs[None, None, :])
    return np.concatenate([z.real, z.imag], axis=-1)


def _library_causal(q, k, v):
    """torch scaled_dot_product_attention, causal, fp64 CPU, GQA by repeating
    kv heads.  q: [L][Hq][D] (rotated), k, v: [L][Hkv][D]."""
    G = q.shape[1] // k.shape[1]
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(np.repeat(k, G, axis=1)).permute(1, 0, 2)[None]
    vt = torch.from_numpy(np.repeat(v, G, axis=1)).permute(1, 0, 2)[None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    return o[0].permute(1, 0, 2).numpy()


def _inputs(seed, L, Hq, Hkv, D):
    rng = np.random.default_rng(seed)
    return rng.normal(size=(L, Hq, D)), rng.normal(size=(L, Hkv, D)), rng.normal(size=(L, Hkv, D))


@pytest.mark.parametrize("seed,L,Hq,Hkv,D", [(0, 37, 4, 2, 16), (1, 64, 8, 8, 8), (2, 5, 6, 1, 32)])
def test_prefill_is_library_causal_attention(seed, L, Hq, Hkv, D):
    q, k, v = _inputs(seed, L, Hq, Hkv, D)
    out, ck, cv = oracle.trunk_prefill(q, k, v)
    pos = np.arange(L)
    ref = _library_causal(_complex_rope(q, pos), _complex_rope(k, pos), v)
    np.testing.assert_allclose(out, ref, atol=1e-12)
    np.testing.assert_allclose(ck, _complex_rope(k, pos), atol=1e-12)
    np.testing.assert_array_equal(cv, v)


def test_prefill_selected_rows_match_all_rows():
    q, k, v = _inputs(3, 50, 4, 2, 16)
    full, _, _ = oracle.trunk_prefill(q, k, v)
    rows = [0, 7, 49, 23]
    part, _, _ = oracle.trunk_prefill(q, k, v, rows=rows)
    np.testing.assert_allclose(part[rows], full[rows], atol=1e-14)
    others = np.setdiff1d(np.arange(50), rows)
    assert np.all(part[others] == 0.0)


def test_prefill_closed_forms():
    q, k, v = _inputs(4, 20, 4, 2, 8)
    out, _, _ = oracle.trunk_prefill(q, k, v)
    # the first token attends to itself only
    np.testing.assert_allclose(out[0], np.repeat(v[:1], 2, axis=1)[0], atol=1e-14)
    # constant values: every row returns that constant, whatever the scores
    vc = np.broadcast_to(np.array([0.5, -1.25, 2.0, 0.0, 1.0, 3.0, -2.0, 0.25]), v.shape).copy()
    outc, _, _ = oracle.trunk_prefill(q, k, vc)
    np.testing.assert_allclose(outc, np.broadcast_to(vc[:, :1], (20, 1, 8)).repeat(4, axis=1), atol=1e-13)
    # zero queries: uniform weights over the visible prefix
    out0, _, _ = oracle.trunk_prefill(np.zeros_like(q), k, v)
    for s in (0, 5, 19):
        np.testing.assert_allclose(out0[s, 0], v[: s + 1, 0].mean(axis=0), atol=1e-13)


def test_planted_off_by_one_is_caught():
    """A causal mask that lets token s see token s+1 fails the library pin."""
    q, k, v = _inputs(5, 12, 2, 1, 8)
    pos = np.arange(12)
    qr, kr = _complex_rope(q, pos), _complex_rope(k, pos)
    s = (qr[:, 0] @ kr[:, 0].T) / np.sqrt(8)
    s = np.where(np.arange(12)[None, :] <= np.arange(12)[:, None] + 1, s, -np.inf)
    w = np.exp(s - s.max(axis=1, keepdims=True))
    wrong = (w @ v[:, 0]) / w.sum(axis=1, keepdims=True)
    ref = _library_causal(qr, kr, v)[:, 0]
    assert np.abs(wrong - ref).max() > 1e-3


def test_r_c1_cb_t_consistency():
    """[R] §3.2 / Table 4: for branches that continue the reference, full
    recomputation (R: prefill over trunk and continuation), scoring each
    branch alone from the cache (C1), scoring them in one batch (CB) and the
    merged tree (T) give the same rows (fp64, to rounding)."""
    L, Hq, Hkv, D, W = 60, 4, 2, 16, 4
    q, k, v = _inputs(6, L, Hq, Hkv, D)
    R, ck, cv = oracle.trunk_prefill(q, k, v)           # every row of the reference
    anchors = np.array([9, 30, 47])
    parent = np.array([-1, 0, 1, 2])
    B = len(anchors)
    pos = anchors[:, None] + 1 + np.arange(W)[None]
    bq = np.stack([q[a + 1: a + 1 + W] for a in anchors])
    bk = np.stack([k[a + 1: a + 1 + W] for a in anchors])
    bv = np.stack([v[a + 1: a + 1 + W] for a in anchors])
    # C1: one branch per call
    C1 = np.stack([oracle.tree_attention_branch(ck, cv, bq[b], bk[b], bv[b], anchors[b], parent, pos[b])
                   for b in range(B)])
    # CB: one batched call over every branch
    CB = oracle.tree_attention(ck[None], cv[None], bq[None], bk[None], bv[None], anchors[None],
                               np.tile(parent, (B, 1))[None], pos[None])[0]
    # T: the packed tree of all branches under the Eq. 5 mask
    T = oracle.tree_attention_packed(ck, cv, bq, bk, bv, anchors, np.tile(parent, (B, 1)), pos)
    for b, a in enumerate(anchors):
        np.testing.assert_allclose(C1[b], R[a + 1: a + 1 + W], atol=1e-12)
        np.testing.assert_allclose(CB[b], R[a + 1: a + 1 + W], atol=1e-12)
        np.testing.assert_allclose(T[b], R[a + 1: a + 1 + W], atol=1e-12)
