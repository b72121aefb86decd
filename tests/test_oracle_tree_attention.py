"""Pins of the tree-attention oracle: rotary convention against complex
arithmetic and hand values, every row against an independent library
attention over its assembled history, the trunk-continuation equality (tree
rows equal a causal pass over the trunk, computed by a library routine),
isolation under poisoned values, and the toy tree of the pages' figures."""

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle
from conftest import golden_dict, golden_lines


# ---------------------------------------------------------------- rotary


def test_rope_pair_is_complex_rotation():
    rng = np.random.default_rng(0)
    D, base = 16, 10000.0
    x = rng.normal(size=(5, D))
    pos = np.array([0, 1, 7, 300, 32770])
    y = oracle.rope(x, pos, base)
    h = D // 2
    zc = x[:, :h] + 1j * x[:, h:]
    freqs = base ** (-np.arange(0, D, 2) / D)
    rot = zc * np.exp(1j * pos[:, None] * freqs[None, :])
    np.testing.assert_allclose(y[:, :h], rot.real, atol=1e-12)
    np.testing.assert_allclose(y[:, h:], rot.imag, atol=1e-12)


def test_rope_hand_values():
    # D=4, base 1e4: pair 0 turns 1 rad per position, pair 1 turns 0.01 rad.
    e0 = np.array([1.0, 0.0, 0.0, 0.0])
    e1 = np.array([0.0, 1.0, 0.0, 0.0])
    np.testing.assert_allclose(oracle.rope(e0, 100), [np.cos(100), 0, np.sin(100), 0], atol=1e-12)
    np.testing.assert_allclose(oracle.rope(e1, 100), [0, np.cos(1.0), 0, np.sin(1.0)], atol=1e-12)
    np.testing.assert_allclose(oracle.rope(e0, 0), e0, atol=0)


def test_rope_relative_and_isometric():
    rng = np.random.default_rng(1)
    q, k = rng.normal(size=64), rng.normal(size=64)
    d1 = oracle.rope(q, 1000) @ oracle.rope(k, 990)
    d2 = oracle.rope(q, 30) @ oracle.rope(k, 20)
    assert d1 == pytest.approx(d2, abs=1e-9)
    assert np.linalg.norm(oracle.rope(q, 12345)) == pytest.approx(np.linalg.norm(q), rel=1e-13)


# ---------------------------------------------------------------- helpers


def _problem(rng, L, B, parent, Hq, Hkv, D, P=None):
    P = P if P is not None else L // 4
    Wn = len(parent)
    anchors = rng.choice(np.arange(P, L - 1), size=B, replace=False)
    depth = oracle.tree_depths(parent)
    pos = anchors[:, None] + 1 + depth[None, :]
    return dict(
        trunk_k=rng.normal(size=(L, Hkv, D)), trunk_v=rng.normal(size=(L, Hkv, D)),
        q=rng.normal(size=(B, Wn, Hq, D)), k=rng.normal(size=(B, Wn, Hkv, D)),
        v=rng.normal(size=(B, Wn, Hkv, D)), anchors=anchors,
        parent=np.tile(np.asarray(parent), (B, 1)), pos=pos)


def _run(p, **kw):
    return oracle.tree_attention(p["trunk_k"][None], p["trunk_v"][None], p["q"][None],
                                 p["k"][None], p["v"][None], p["anchors"][None],
                                 p["parent"][None], p["pos"][None], **kw)[0]


def _sdpa_single(qv, keys, vals, scale):
    """torch's scaled_dot_product_attention (fp64, CPU) for one query."""
    qt = torch.from_numpy(qv)[None, None, None, :]
    kt = torch.from_numpy(keys)[None, None]
    vt = torch.from_numpy(vals)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)[0, 0, 0].numpy()


FORK = [-1, 0, 1, 2, 3, 4, 5, 3, 7, 8]


# ---------------------------------------------------------------- pins


@settings(max_examples=12, deadline=None)
@given(st.integers(0, 10_000), st.sampled_from([[-1], [-1, 0, 1, 2], FORK, [-1, 0, 0, 1, 1, 2]]),
       st.sampled_from([(2, 1, 8), (4, 2, 16), (6, 2, 8)]))
def test_each_row_is_plain_attention_over_its_history(seed, parent, heads):
    """(i) A row equals ordinary attention of its rotated query over the trunk
    prefix 0..a_b followed by its own ancestor path (rotated at their
    positions): the history it is conditioned on ([R] §3.1)."""
    rng = np.random.default_rng(seed)
    Hq, Hkv, D = heads
    p = _problem(rng, L=40, B=3, parent=parent, Hq=Hq, Hkv=Hkv, D=D)
    out = _run(p)
    G = Hq // Hkv
    scale = 1 / np.sqrt(D)
    for b in range(3):
        a = p["anchors"][b]
        for j in range(len(parent)):
            path = oracle.walk_ancestors(parent, j)[::-1]           # anchor child .. j
            for h in range(Hq):
                g = h // G
                keys = np.concatenate([p["trunk_k"][: a + 1, g],
                                       oracle.rope(p["k"][b, path, g], p["pos"][b, path])])
                vals = np.concatenate([p["trunk_v"][: a + 1, g], p["v"][b, path, g]])
                qv = oracle.rope(p["q"][b, j, h], p["pos"][b, j])
                np.testing.assert_allclose(out[b, j, h], _sdpa_single(qv, keys, vals, scale), atol=1e-12)


def test_single_node_branch_is_plain_causal_row():
    """(ii) W=1: the node reads trunk 0..a and itself."""
    rng = np.random.default_rng(3)
    p = _problem(rng, L=30, B=2, parent=[-1], Hq=2, Hkv=2, D=8)
    out = _run(p)
    for b in range(2):
        a = p["anchors"][b]
        for h in range(2):
            keys = np.concatenate([p["trunk_k"][: a + 1, h], oracle.rope(p["k"][b, :, h], a + 1)])
            vals = np.concatenate([p["trunk_v"][: a + 1, h], p["v"][b, :, h]])
            qv = oracle.rope(p["q"][b, 0, h], a + 1)
            np.testing.assert_allclose(out[b, 0, h], _sdpa_single(qv, keys, vals, 1 / np.sqrt(8)), atol=1e-12)


def test_branch_following_reference_equals_trunk_causal_rows():
    """(iii) A branch whose tokens are the reference's own continuation gives
    exactly the trunk's causal rows at positions a+1..a+W: tree execution
    equals full recomputation ([R] §3.2, Table 4)."""
    rng = np.random.default_rng(4)
    L, Hq, Hkv, D, W = 48, 4, 2, 16, 5
    raw_q = rng.normal(size=(L, Hq, D))
    raw_k = rng.normal(size=(L, Hkv, D))
    raw_v = rng.normal(size=(L, Hkv, D))
    posL = np.arange(L)
    rq = oracle.rope(raw_q, posL[:, None])
    rk = oracle.rope(raw_k, posL[:, None])
    G = Hq // Hkv
    # library causal attention over the whole trunk (GQA by repeating kv heads)
    qt = torch.from_numpy(rq).permute(1, 0, 2)[None]
    kt = torch.from_numpy(np.repeat(rk, G, axis=1)).permute(1, 0, 2)[None]
    vt = torch.from_numpy(np.repeat(raw_v, G, axis=1)).permute(1, 0, 2)[None]
    causal = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)[0].permute(1, 0, 2).numpy()
    anchors = np.array([10, 25, 40])
    B = len(anchors)
    parent = np.tile(np.array([-1, 0, 1, 2, 3]), (B, 1))
    pos = anchors[:, None] + 1 + np.arange(W)[None]
    q = np.stack([raw_q[a + 1: a + 1 + W] for a in anchors])
    k = np.stack([raw_k[a + 1: a + 1 + W] for a in anchors])
    v = np.stack([raw_v[a + 1: a + 1 + W] for a in anchors])
    out = oracle.tree_attention(rk[None], raw_v[None], q[None], k[None], v[None], anchors[None],
                                parent[None], pos[None])[0]
    for b, a in enumerate(anchors):
        np.testing.assert_allclose(out[b], causal[a + 1: a + 1 + W], atol=1e-12)


def test_packing_order_invariance():
    """(iv) Permuting branches permutes outputs (positions are logical)."""
    rng = np.random.default_rng(5)
    p = _problem(rng, L=50, B=5, parent=FORK, Hq=4, Hkv=2, D=8)
    out = _run(p)
    perm = rng.permutation(5)
    pp = {k: (v[perm] if k not in ("trunk_k", "trunk_v") else v) for k, v in p.items()}
    np.testing.assert_allclose(_run(pp), out[perm], atol=1e-13)


def test_packed_mask_matches_per_branch_and_isolates():
    """(v) The packed Eq. 5 form equals the per-branch form, and poisoning
    values a row must not read (later trunk positions, sibling branches)
    changes nothing."""
    rng = np.random.default_rng(6)
    p = _problem(rng, L=40, B=4, parent=[-1, 0, 0, 2], Hq=2, Hkv=1, D=8)
    args = [p[k] for k in ("trunk_k", "trunk_v", "q", "k", "v", "anchors", "parent", "pos")]
    packed = oracle.tree_attention_packed(*args)
    np.testing.assert_allclose(packed, _run(p), atol=1e-12)
    for b in range(4):
        a = p["anchors"][b]
        tv = p["trunk_v"].copy()
        tv[a + 1:] *= 1e4
        vv = p["v"].copy()
        for o in range(4):
            if o != b:
                vv[o] *= 1e4
        args2 = [p["trunk_k"], tv, p["q"], p["k"], vv, p["anchors"], p["parent"], p["pos"]]
        np.testing.assert_allclose(oracle.tree_attention_packed(*args2)[b], packed[b], atol=1e-10)
    # a node also must not read its siblings inside its own branch
    # (nodes 1 and 2 are both children of node 0)
    m = oracle.branch_mask(40, 20, [-1, 0, 0, 2])
    assert not m[1, 40 + 2] and not m[2, 40 + 1] and not m[3, 40 + 1]


def test_tree_rows_equal_either_chain():
    """(vi) In the forked tree, each root-to-leaf path gives the rows the same
    path gives as a chain on its own."""
    rng = np.random.default_rng(7)
    p = _problem(rng, L=60, B=2, parent=FORK, Hq=4, Hkv=2, D=16)
    out = _run(p)
    for path in ([0, 1, 2, 3, 4, 5, 6], [0, 1, 2, 3, 7, 8, 9]):
        pc = dict(p)
        for key in ("q", "k", "v", "pos"):
            pc[key] = p[key][:, path]
        pc["parent"] = np.tile(np.array([-1, 0, 1, 2, 3, 4, 5]), (2, 1))
        np.testing.assert_allclose(_run(pc), out[:, path], atol=1e-12)


def test_gqa_head_mapping():
    """(vii) Duplicating each kv head G times and running as MHA gives the
    same output as GQA with head h reading kv head floor(h/G)."""
    rng = np.random.default_rng(8)
    p = _problem(rng, L=30, B=2, parent=[-1, 0, 1], Hq=6, Hkv=2, D=8)
    out = _run(p)
    pm = dict(p)
    for key in ("trunk_k", "trunk_v", "k", "v"):
        pm[key] = np.repeat(p[key], 3, axis=-2)
    np.testing.assert_allclose(_run(pm), out, atol=1e-13)


def test_fig3_toy_tree():
    """(viii) The pages' toy tree: mask and score rows by hand."""
    g = golden_dict("fig3_toy_tree.txt")
    L = int(g["L"][0][0])
    anchors = np.array([int(x[1]) for x in sorted(g["anchor"], key=lambda r: int(r[0]))])
    nodes = sorted(g["node"], key=lambda r: (int(r[0]), int(r[1])))
    B = len(anchors)
    Wn = len(nodes) // B
    parent = np.array([[int(n[3]) for n in nodes if int(n[0]) == b] for b in range(B)])
    pos = np.array([[int(n[4]) for n in nodes if int(n[0]) == b] for b in range(B)])
    for b in range(B):
        oracle.check_positions(anchors[b], parent[b], pos[b])
    m = oracle.packed_tree_mask(L, anchors, parent)
    want = np.zeros_like(m)
    for row in g["mask"]:
        r, last = int(row[0]), int(row[1])
        want[r, : last + 1] = True
        for c in row[2:]:
            want[r, L + int(c)] = True
    assert np.array_equal(m, want)
    for b, j, kind, src in g["score"]:
        got = oracle.score_row_source(anchors[int(b)], parent[int(b)], int(j))
        assert got == (kind, int(src))
    assert sum(len(oracle.new_score_rows(parent[b])) for b in range(B)) == int(g["new_rows"][0][0])
    assert Wn == 2


def test_eq20_shared_row_count():
    g = golden_dict("eq20_rows.txt")
    L, W, K = int(g["L"][0][0]), int(g["W"][0][0]), int(g["K"][0][0])
    chain = [-1] + list(range(W - 1))
    shared = oracle.shared_row_count(L, [chain] * K)
    assert shared == int(g["shared_rows"][0][0])
    assert round(int(g["cacheless_rows"][0][0]) / shared, 2) == float(g["ratio"][0][0])


def test_malformed_inputs_rejected():
    with pytest.raises(ValueError):
        oracle.walk_ancestors([-1, 1], 1)          # self-parent
    with pytest.raises(ValueError):
        oracle.walk_ancestors([-1, 2, 0], 1)       # parent after child
    with pytest.raises(ValueError):
        oracle.check_positions(10, [-1, 0], [11, 13])


def test_bf16_torch_inputs_widen_exactly():
    rng = np.random.default_rng(9)
    p = _problem(rng, L=20, B=1, parent=[-1, 0], Hq=2, Hkv=1, D=8)
    tb = {k: torch.from_numpy(np.asarray(v)) for k, v in p.items()}
    for key in ("trunk_k", "trunk_v", "q", "k", "v"):
        tb[key] = tb[key].to(torch.bfloat16)
    out_t = oracle.tree_attention(*(tb[k][None] for k in ("trunk_k", "trunk_v", "q", "k", "v",
                                                          "anchors", "parent", "pos")))[0]
    pw = {k: (tb[k].double().numpy() if tb[k].is_floating_point() else p[k]) for k in p}
    np.testing.assert_allclose(out_t, _run(pw), atol=0)
