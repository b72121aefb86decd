"""Pins of the QSA block-selection oracle (CPU only).

Each pin checks the oracle against something other than its own code: hand
values of a two-dimensional example, invariances of the compression, a
Python-sort statement of top-k, and the method's exactness -- a branch row
selects what the same row selects in the plain sequence trunk[0..a] followed
by its ancestor path, every group compressed from scratch ([R] §3.2(b)) --
plus isolation from reference tokens after the anchor."""

import math

import numpy as np
import pytest

from oracle import qsa


def _tree(rng, Wn):
    """Random parent map: node 0 hangs on the anchor, each later node on an
    earlier one (forks happen)."""
    return [-1] + [int(rng.integers(0, j)) for j in range(1, Wn)]


def _depths(parent):
    d = []
    for j, p in enumerate(parent):
        d.append(0 if p < 0 else d[p] + 1)
    return np.array(d)


def _case(seed, L=48, Wn=7, Di=8, fork=True):
    rng = np.random.default_rng(seed)
    trunk_raw = rng.standard_normal((L, Di))
    x = rng.standard_normal((Wn, Di))
    y = rng.standard_normal((Wn, Di))
    gamma = 1.0 + 0.3 * rng.standard_normal(Di)
    parent = _tree(rng, Wn) if fork else [-1] + list(range(Wn - 1))
    return rng, trunk_raw, x, y, gamma, parent


def test_hand_values_two_dims():
    # Di = 2: one rotation pair with frequency base^0 = 1, so position p
    # rotates by p radians.  gamma = 1, eps = 0.
    g = np.ones(2)
    raw = np.array([[1, 0], [1, 0], [3, 0], [3, 0], [0, 2], [0, 2], [0, 2], [0, 2]], float)
    keys = qsa.sequence_group_keys(raw, g, eps=0.0)
    # group 0: mean (2, 0), mean square 2 -> (sqrt 2, 0), rotated by 0
    assert np.allclose(keys[0], [math.sqrt(2), 0.0], atol=1e-15)
    # group 1: mean (0, 2) -> (0, sqrt 2), rotated by 4 rad: (-sqrt2 sin 4, sqrt2 cos 4)
    assert np.allclose(keys[1], [1.0702696562268, -0.9243850953575], atol=1e-12)
    # a query (1, 0) at position 7 scores group g by cos of (7 - angle of key g)
    sel, sc, s = qsa.plain_row_select(raw, [1.0, 0.0], g, k=1, eps=0.0)
    assert np.allclose(s, [math.sqrt(2) * math.cos(7.0), math.sqrt(2) * math.cos(7.0 - 4.0 - math.pi / 2)])
    assert sel.tolist() == [int(np.argmax(s))]


def test_compression_invariances():
    rng = np.random.default_rng(1)
    Di = 16
    g = rng.standard_normal(Di)
    u = rng.standard_normal((4, Di))
    # RMSNorm ignores a positive scale (eps = 0); rotation keeps the length
    a = qsa.compress_group(u, g, 12, eps=0.0)
    b = qsa.compress_group(3.5 * u, g, 12, eps=0.0)
    assert np.allclose(a, b, rtol=1e-13)
    r = qsa.compress_group(u, g, 0, eps=0.0)
    assert np.isclose(np.linalg.norm(a), np.linalg.norm(r), rtol=1e-13)
    # four equal tokens pool to that token; gamma = 1: unit root-mean-square
    one = np.repeat(u[:1], 4, axis=0)
    k0 = qsa.compress_group(one, np.ones(Di), 0, eps=0.0)
    assert np.isclose(np.sqrt(np.mean(k0 ** 2)), 1.0, rtol=1e-13)
    assert np.allclose(k0 * np.sqrt(np.mean(u[0] ** 2)), u[0], rtol=1e-12)
    # the order of the four tokens does not matter
    assert np.allclose(qsa.compress_group(u[::-1], g, 8), qsa.compress_group(u, g, 8), rtol=1e-13)


def _topk_by_sort(s, k):
    order = sorted(range(len(s)), key=lambda i: (-s[i], i))
    return sorted(order[:k])


@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_sorting_rule(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 40))
    s = np.round(rng.standard_normal(n), 1)  # rounding makes ties
    for k in (1, 3, n - 1, n, n + 5):
        if k < 1:
            continue
        got = qsa.select_topk(s, k).tolist()
        assert got == _topk_by_sort(s, k)


@pytest.mark.parametrize("seed", range(12))
def test_branch_rows_equal_plain_sequence(seed):
    rng, trunk_raw, x, y, gamma, parent = _case(seed, fork=seed % 3 != 0)
    L, Di = trunk_raw.shape
    Wn = x.shape[0]
    anchor = 20 + seed % 4  # every residue mod 4 (a + 1 = 0 mod 4: no boundary group)
    pos = anchor + 1 + _depths(parent)
    gk = qsa.sequence_group_keys(trunk_raw, gamma)
    k = [1, 2, 3, 5, 8][seed % 5]
    res = qsa.qsa_branch_select(gk, trunk_raw, x, y, anchor, parent, pos, gamma, k)
    from oracle.tree_attention import walk_ancestors
    for j in range(Wn):
        path = walk_ancestors(parent, j)[::-1]
        seq = np.concatenate([trunk_raw[:anchor + 1], x[path]], axis=0)
        sel, sc, s = qsa.plain_row_select(seq, y[j], gamma, k)
        n = sel.shape[0]
        assert res["ncand"][j] == s.shape[0] == (pos[j] + 1) // 4
        assert res["sel"][j, :n].tolist() == sel.tolist()
        assert np.allclose(res["scores"][j], s, rtol=1e-12, atol=1e-12)
        assert np.allclose(res["score"][j, :n], sc, rtol=1e-12, atol=1e-12)
        assert (res["sel"][j, n:] == -1).all()


@pytest.mark.parametrize("seed", range(6))
def test_reference_tokens_after_the_anchor_do_not_leak(seed):
    rng, trunk_raw, x, y, gamma, parent = _case(100 + seed)
    anchor = 17 + seed % 4
    pos = anchor + 1 + _depths(parent)
    base = qsa.qsa_branch_select(qsa.sequence_group_keys(trunk_raw, gamma), trunk_raw, x, y,
                                 anchor, parent, pos, gamma, 3)
    poisoned = trunk_raw.copy()
    poisoned[anchor + 1:] = 1e4 * rng.standard_normal(poisoned[anchor + 1:].shape)
    # the trunk pass's cache of the poisoned trunk: its boundary group changes
    gk_p = qsa.sequence_group_keys(poisoned, gamma)
    res = qsa.qsa_branch_select(gk_p, poisoned, x, y, anchor, parent, pos, gamma, 3)
    assert np.array_equal(res["sel"], base["sel"])
    for a, b in zip(res["scores"], base["scores"]):
        assert np.array_equal(a, b)


def test_cached_groups_are_reused_as_given():
    rng, trunk_raw, x, y, gamma, parent = _case(7)
    anchor = 22
    pos = anchor + 1 + _depths(parent)
    gk = qsa.sequence_group_keys(trunk_raw, gamma)
    base = qsa.qsa_branch_select(gk, trunk_raw, x, y, anchor, parent, pos, gamma, 4)
    gt = (anchor + 1) // 4
    # cache entries of groups not complete at the anchor are never read
    gk2 = gk.copy()
    gk2[gt:] = np.nan
    res = qsa.qsa_branch_select(gk2, trunk_raw, x, y, anchor, parent, pos, gamma, 4)
    for a, b in zip(res["scores"], base["scores"]):
        assert np.array_equal(a, b)
    # an entry before the anchor is used as given: shifting it shifts that
    # group's score by exactly <rope(y, p), delta>
    from oracle.rope import rope
    delta = rng.standard_normal(gk.shape[1])
    gk3 = gk.copy()
    gk3[2] += delta
    res = qsa.qsa_branch_select(gk3, trunk_raw, x, y, anchor, parent, pos, gamma, 4)
    for j in range(len(parent)):
        d = res["scores"][j] - base["scores"][j]
        assert np.isclose(d[2], rope(y[j], pos[j]) @ delta, rtol=1e-12)
        assert np.allclose(np.delete(d, 2), 0.0)


def test_siblings_share_keys_before_the_fork_only():
    rng = np.random.default_rng(3)
    Di = 8
    trunk_raw = rng.standard_normal((40, Di))
    gamma = np.ones(Di)
    # chain of offsets 0..3, then two sub-branches of offsets 4..6 (ten nodes)
    parent = [-1, 0, 1, 2, 3, 4, 5, 3, 7, 8]
    x = rng.standard_normal((10, Di))
    # anchor 14: node 0 (position 15) closes the boundary group 3 (trunk 12..14
    # and itself); group 4 (positions 16..19) closes at node 4 and at node 7
    anchor = 14
    keys, gidx = qsa.branch_group_keys(trunk_raw, x, anchor, parent, gamma)
    assert gidx.tolist() == [3, -1, -1, -1, 4, -1, -1, 4, -1, -1]
    want = qsa.compress_group(np.stack([trunk_raw[12], trunk_raw[13], trunk_raw[14], x[0]]), gamma, 12)
    assert np.allclose(keys[0], want, rtol=1e-13)
    # node 4 and node 7 close group 4 from their own fourth token
    assert not np.allclose(keys[4], keys[7])
    x2 = x.copy()
    x2[7] = x[4]
    keys2, _ = qsa.branch_group_keys(trunk_raw, x2, anchor, parent, gamma)
    assert np.array_equal(keys2[7], keys2[4])
    # the boundary group (positions 12..15) is closed by node 0 from trunk 12..14
    keys3, g3 = qsa.branch_group_keys(trunk_raw, x, 11, parent, gamma)
    assert g3[3] == 3 and g3[0] == -1  # anchor 11 completes group 2 itself
    keys4, g4 = qsa.branch_group_keys(trunk_raw, x, 12, parent, gamma)
    assert g4[2] == 3
    want = qsa.compress_group(np.stack([trunk_raw[12], x[0], x[1], x[2]]), gamma, 12)
    assert np.allclose(keys4[2], want, rtol=1e-13)


@pytest.mark.parametrize("seed", range(4))
def test_candidates_and_tail_partition_the_history(seed):
    rng, trunk_raw, x, y, gamma, parent = _case(200 + seed)
    anchor = 9 + seed
    from oracle.tree_attention import walk_ancestors
    for j in range(len(parent)):
        path = walk_ancestors(parent, j)
        p = anchor + len(path)
        hist = [("trunk", s) for s in range(anchor + 1)] + [("node", i) for i in path[::-1]]
        ng = (p + 1) // 4
        tail = qsa.causal_tail(anchor, parent, j)
        assert hist[:4 * ng] + tail == hist
        assert len(tail) == (p + 1) % 4


def test_fewer_candidates_than_k_keep_all():
    rng, trunk_raw, x, y, gamma, parent = _case(5, Wn=3, fork=False)
    anchor = 2  # positions 3, 4, 5: at most one complete group
    pos = anchor + 1 + _depths(parent)
    res = qsa.qsa_branch_select(qsa.sequence_group_keys(trunk_raw, gamma), trunk_raw, x, y,
                                anchor, parent, pos, gamma, 8)
    assert res["ncand"].tolist() == [1, 1, 1]
    assert (res["sel"][:, 0] == 0).all() and (res["sel"][:, 1:] == -1).all()
    assert np.isneginf(res["score"][:, 1:]).all()


def test_malformed_positions_raise():
    rng, trunk_raw, x, y, gamma, parent = _case(6, fork=False)
    pos = 30 + _depths(parent)
    with pytest.raises(ValueError):
        qsa.qsa_branch_select(qsa.sequence_group_keys(trunk_raw, gamma), trunk_raw, x, y, 30,
                              parent, pos, gamma, 2)


def test_round_bf16_ties_to_even():
    # bf16 keeps 8 significant bits: 1 + 2^-7 is the neighbour above 1
    assert qsa.round_bf16(1.0 + 2.0 ** -8) == 1.0                       # tie, to even
    assert qsa.round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6       # tie, to even
    assert qsa.round_bf16(1.0 + 2.0 ** -8 + 2.0 ** -20) == 1.0 + 2.0 ** -7
    assert qsa.round_bf16(-3.0 - 2.0 ** -7) == -3.0                     # tie at 2^1 scale
    # against the library's conversion on random values
    import torch
    v = np.random.default_rng(0).standard_normal(4096) * 10.0 ** np.random.default_rng(1).integers(-6, 6, 4096)
    want = torch.tensor(v, dtype=torch.float32).to(torch.bfloat16).double().numpy()
    assert np.array_equal(qsa.round_bf16(v), want)


def test_bf16_operands_change_only_the_operands():
    rng, trunk_raw, x, y, gamma, parent = _case(9)
    anchor = 21
    pos = anchor + 1 + _depths(parent)
    gk = qsa.round_bf16(qsa.sequence_group_keys(trunk_raw, gamma))
    a = qsa.qsa_branch_select(gk, trunk_raw, x, y, anchor, parent, pos, gamma, 3, operands="bf16")
    from oracle.rope import rope
    for j in range(len(parent)):
        # trunk groups: the cached key times the rounded rotated query, exactly
        yq = qsa.round_bf16(rope(y[j], pos[j]))
        gt = (anchor + 1) // 4
        assert np.allclose(a["scores"][j][:gt], gk[:gt] @ yq, rtol=1e-15, atol=0)
    ok = a["bgroup"] >= 0
    assert np.array_equal(a["bkey"][ok], qsa.round_bf16(a["bkey"][ok]))
