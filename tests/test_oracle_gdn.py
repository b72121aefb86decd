"""Pins of the GDN branch-replay oracle (oracle.gdn).

The update is checked against an independent statement of the same linear
map (a Kronecker-product matrix acting on the flattened state) and against
textbook properties of the delta rule (a full-strength write to a unit key
is read back exactly; orthonormal keys store independent values; no write is
pure decay; the first token from the zero state in closed form).  The replay
machinery is checked against plain sequential recurrences over the whole
history (the pages' full-recomputation consistency, [R] §3.2 "numerical
consistency"), against the Figure 5 example ([R] §3.2(c)), and the update
counts against the 24.9x of [R] §3.4."""

import os

import numpy as np
import pytest

from oracle import gdn

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fig5_gdn_replay.txt")


def _unit(rng, *shape):
    x = rng.normal(size=shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def test_update_is_the_linear_map_on_the_flattened_state():
    # S' = S A + B with A = alpha (I - beta k k^T), B = beta v k^T, written as
    # (A^T kron I) vec(S) + vec(B) on the column-major flattening
    rng = np.random.default_rng(1)
    Dv, Dk = 3, 5
    for _ in range(5):
        S = rng.normal(size=(Dv, Dk))
        k = _unit(rng, Dk)
        v = rng.normal(size=Dv)
        alpha, beta = rng.uniform(0.5, 1.0), rng.uniform(0.0, 1.0)
        A = alpha * (np.eye(Dk) - beta * np.outer(k, k))
        M = np.kron(A.T, np.eye(Dv))
        vecS = S.reshape(-1, order="F")
        vecB = (beta * np.outer(v, k)).reshape(-1, order="F")
        want = (M @ vecS + vecB).reshape((Dv, Dk), order="F")
        np.testing.assert_allclose(gdn.gated_delta_update(S, k, v, alpha, beta), want, rtol=0, atol=1e-13)


def test_full_strength_write_reads_back_the_value():
    rng = np.random.default_rng(2)
    for _ in range(5):
        S = rng.normal(size=(6, 8))
        k = _unit(rng, 8)
        v = rng.normal(size=6)
        S1 = gdn.gated_delta_update(S, k, v, rng.uniform(0.1, 1.0), 1.0)
        np.testing.assert_allclose(S1 @ k, v, rtol=0, atol=1e-12)


def test_orthonormal_keys_store_independent_values():
    rng = np.random.default_rng(3)
    D, n = 8, 5
    Q, _ = np.linalg.qr(rng.normal(size=(D, D)))
    keys = Q[:, :n].T
    vals = rng.normal(size=(n, D))
    S = np.zeros((D, D))
    for i in range(n):
        S = gdn.gated_delta_update(S, keys[i], vals[i], 1.0, 1.0)
    for i in range(n):
        np.testing.assert_allclose(gdn.gdn_read(S, keys[i]), vals[i], rtol=0, atol=1e-12)


def test_no_write_is_pure_decay():
    rng = np.random.default_rng(4)
    S0 = rng.normal(size=(4, 4))
    alphas = rng.uniform(0.5, 1.0, size=7)
    states = gdn.run_tokens(S0, _unit(rng, 7, 4), rng.normal(size=(7, 4)), alphas, np.zeros(7))
    np.testing.assert_allclose(states[-1], np.prod(alphas) * S0, rtol=1e-13, atol=0)


def test_first_token_from_zero_state():
    rng = np.random.default_rng(5)
    k, q, v = _unit(rng, 6), rng.normal(size=6), rng.normal(size=6)
    beta = 0.3
    S = gdn.gated_delta_update(np.zeros((6, 6)), k, v, 0.7, beta)
    np.testing.assert_allclose(gdn.gdn_read(S, q), beta * (k @ q) * v, rtol=0, atol=1e-14)


def _trunk(rng, L, H, D):
    return (_unit(rng, L, H, D), rng.normal(size=(L, H, D)), rng.uniform(0.8, 1.0, size=(L, H)),
            rng.uniform(0.05, 0.95, size=(L, H)))


def test_checkpoints_are_states_after_every_C_tokens():
    rng = np.random.default_rng(6)
    L, H, D, C = 50, 2, 4, 8
    k, v, a, b = _trunk(rng, L, H, D)
    ck = gdn.trunk_checkpoints(k, v, a, b, C)
    assert ck.shape == (L // C, H, D, D)
    for h in range(H):
        states = gdn.run_tokens(np.zeros((D, D)), k[:, h], v[:, h], a[:, h], b[:, h])
        for m in range(L // C):
            np.testing.assert_allclose(ck[m, h], states[(m + 1) * C - 1], rtol=0, atol=1e-13)


@pytest.mark.parametrize("anchor", [0, 5, 6, 7, 8, 9, 15, 16, 33, 49])
def test_replayed_anchor_state_equals_the_full_history(anchor):
    rng = np.random.default_rng(7)
    L, H, D, C = 50, 2, 4, 8
    k, v, a, b = _trunk(rng, L, H, D)
    ck = gdn.trunk_checkpoints(k, v, a, b, C)
    for h in range(H):
        full = gdn.run_tokens(np.zeros((D, D)), k[:anchor + 1, h], v[:anchor + 1, h], a[:anchor + 1, h],
                              b[:anchor + 1, h])[-1]
        np.testing.assert_allclose(gdn.anchor_state(ck, k, v, a, b, anchor, h, C), full, rtol=0, atol=1e-12)


def test_figure5_replay_spans():
    lines = [l.split() for l in open(GOLDEN) if l.strip() and not l.startswith("#")]
    C = int(next(l[1] for l in lines if l[0] == "C"))
    after = int(next(l[1] for l in lines if l[0] == "checkpoint_after"))
    assert after == C - 1  # the checkpoint holds the state after the 64th token
    for l in lines:
        if l[0] != "anchor":
            continue
        a, want = int(l[1]), [int(x) for x in l[3:]]
        c, t0 = gdn.replay_span(a, C)
        assert c == 0 and list(range(t0, a + 1)) == want


def _path(parent, j):
    p = []
    while j >= 0:
        p.append(j)
        j = int(parent[j])
    return p[::-1]


FORK = (-1, 0, 1, 2, 3, 4, 5, 3, 7, 8)


def _branch_inputs(rng, Wn, H, D):
    return (rng.normal(size=(Wn, H, D)), _unit(rng, Wn, H, D), rng.normal(size=(Wn, H, D)),
            rng.uniform(0.8, 1.0, size=(Wn, H)), rng.uniform(0.05, 0.95, size=(Wn, H)))


@pytest.mark.parametrize("anchor", [3, 7, 8, 30, 49])
def test_branch_equals_full_recomputation_of_its_history(anchor):
    """Node j's output equals reading the state of one sequential pass over
    trunk tokens 0..a followed by the nodes on j's root path."""
    rng = np.random.default_rng(8)
    L, H, D, C = 50, 2, 4, 8
    tk, tv, ta, tb = _trunk(rng, L, H, D)
    ck = gdn.trunk_checkpoints(tk, tv, ta, tb, C)
    q, k, v, a, b = _branch_inputs(rng, len(FORK), H, D)
    out = gdn.gdn_branch(ck, tk, tv, ta, tb, anchor, FORK, q, k, v, a, b, C)
    for j in range(len(FORK)):
        path = _path(FORK, j)
        for h in range(H):
            ks = np.concatenate([tk[:anchor + 1, h], k[path, h]])
            vs = np.concatenate([tv[:anchor + 1, h], v[path, h]])
            As = np.concatenate([ta[:anchor + 1, h], a[path, h]])
            Bs = np.concatenate([tb[:anchor + 1, h], b[path, h]])
            S = gdn.run_tokens(np.zeros((D, D)), ks, vs, As, Bs)[-1]
            np.testing.assert_allclose(out[j, h], S @ q[j, h], rtol=0, atol=1e-12)


def test_sibling_subtrees_do_not_see_each_other():
    rng = np.random.default_rng(9)
    L, H, D, C = 40, 1, 4, 8
    tk, tv, ta, tb = _trunk(rng, L, H, D)
    ck = gdn.trunk_checkpoints(tk, tv, ta, tb, C)
    q, k, v, a, b = _branch_inputs(rng, len(FORK), H, D)
    base = gdn.gdn_branch(ck, tk, tv, ta, tb, 20, FORK, q, k, v, a, b, C)
    v2 = v.copy()
    v2[4:7] += 5.0  # the first sub-branch (nodes 4..6)
    pert = gdn.gdn_branch(ck, tk, tv, ta, tb, 20, FORK, q, k, v2, a, b, C)
    np.testing.assert_array_equal(pert[[0, 1, 2, 3, 7, 8, 9]], base[[0, 1, 2, 3, 7, 8, 9]])
    assert np.abs(pert[4:7] - base[4:7]).max() > 1e-3


def test_malformed_branches_raise():
    rng = np.random.default_rng(10)
    L, H, D, C = 20, 1, 4, 8
    tk, tv, ta, tb = _trunk(rng, L, H, D)
    ck = gdn.trunk_checkpoints(tk, tv, ta, tb, C)
    q, k, v, a, b = _branch_inputs(rng, 3, H, D)
    with pytest.raises(ValueError):
        gdn.gdn_branch(ck, tk, tv, ta, tb, L, (-1, 0, 1), q, k, v, a, b, C)
    with pytest.raises(ValueError):
        gdn.gdn_branch(ck, tk, tv, ta, tb, 5, (-1, 2, 1), q, k, v, a, b, C)
    with pytest.raises(ValueError):
        gdn.gdn_branch(ck, tk, tv, ta, tb, 5, (-1, 0, -2), q, k, v, a, b, C)


def test_update_counts_match_the_page_ratio():
    # [R] §3.4: L = 2048, W = 7, K = 512 anchors spread over the response:
    # 24.9x fewer GDN updates, replay included
    L, W, K = 2048, 7, 512
    anchors = np.round(np.linspace(W, L - 1, K)).astype(int)
    cacheless, shared = gdn.update_counts(L, anchors, W, 64)
    assert round(cacheless / shared, 1) == 24.9
    # the replay after the nearest checkpoint averages (C - 1) / 2 tokens
    rep = [a + 1 - gdn.replay_span(a)[1] for a in range(64 * 10)]
    assert np.mean(rep) == 31.5 and max(rep) == 63 and min(rep) == 0


# ---- the short convolution along the parent map ([R] §3.2(c): the
# convolution history follows only the branch's ancestors)

def _silu(z):
    from scipy.special import expit
    return z * expit(z)


@pytest.mark.parametrize("K,a", [(4, 37), (3, 5), (4, 1), (2, 0)])
def test_chain_conv_is_the_causal_convolution_of_its_history(K, a):
    """For a chain, the branch is a continuation of the trunk: each node's
    output is the plain causal convolution (numpy's) of the sequence trunk
    0..a followed by the nodes, zero-padded before the trunk's start."""
    rng = np.random.default_rng(20 + K + a)
    L, Wn, C = 40, 6, 5
    trunk_x, x = rng.normal(size=(L, C)), rng.normal(size=(Wn, C))
    w = rng.normal(size=(C, K))
    parent = np.arange(Wn) - 1
    got = gdn.branch_conv(trunk_x, x, w, a, parent)
    seq = np.concatenate([trunk_x[: a + 1], x])
    for c in range(C):
        full = np.convolve(seq[:, c], w[c])  # full[t] = sum_i w[c, i] seq[t - i]
        np.testing.assert_allclose(got[:, c], _silu(full[a + 1: a + 1 + Wn]), rtol=0, atol=1e-13)


def test_fork_history_follows_the_parent_map():
    # the forked tree of the long-context configuration: node 7 hangs off
    # node 3, so its window skips nodes 4-6; a root reaches into the trunk
    par = [-1, 0, 1, 2, 3, 4, 5, 3, 7, 8]
    assert gdn.conv_history(100, par, 7, 4) == [("n", 7), ("n", 3), ("n", 2), ("n", 1)]
    assert gdn.conv_history(100, par, 8, 4) == [("n", 8), ("n", 7), ("n", 3), ("n", 2)]
    assert gdn.conv_history(100, par, 1, 4) == [("n", 1), ("n", 0), ("t", 100), ("t", 99)]
    assert gdn.conv_history(1, par, 0, 4) == [("n", 0), ("t", 1), ("t", 0), None]


def test_conv_ignores_nodes_outside_the_window():
    """Poisoning a node changes exactly the outputs whose window holds it."""
    rng = np.random.default_rng(31)
    par = [-1, 0, 1, 2, 3, 4, 5, 3, 7, 8]
    L, C, K, a = 50, 4, 4, 30
    trunk_x, x, w = rng.normal(size=(L, C)), rng.normal(size=(len(par), C)), rng.normal(size=(C, K))
    base = gdn.branch_conv(trunk_x, x, w, a, par)
    for poison in range(len(par)):
        xp = x.copy()
        xp[poison] = np.nan
        got = gdn.branch_conv(trunk_x, xp, w, a, par)
        for j in range(len(par)):
            sees = ("n", poison) in gdn.conv_history(a, par, j, K)
            assert np.isnan(got[j]).all() == sees
            if not sees:
                np.testing.assert_array_equal(got[j], base[j])


def test_width_one_is_silu_of_the_scaled_input():
    rng = np.random.default_rng(32)
    x, w = rng.normal(size=(3, 6)), rng.normal(size=(6, 1))
    got = gdn.branch_conv(rng.normal(size=(10, 6)), x, w, 4, [-1, 0, 0])
    np.testing.assert_allclose(got, _silu(x * w[:, 0]), rtol=0, atol=1e-14)


def test_l2norm_gives_unit_heads_in_the_same_direction():
    rng = np.random.default_rng(33)
    H, D = 3, 8
    trunk_x, x, w = rng.normal(size=(20, H * D)), rng.normal(size=(4, H * D)), rng.normal(size=(H * D, 4))
    par = [-1, 0, 1, 1]
    plain = gdn.branch_conv(trunk_x, x, w, 10, par).reshape(4, H, D)
    unit = gdn.branch_conv(trunk_x, x, w, 10, par, D=D, l2norm=True).reshape(4, H, D)
    nrm = np.linalg.norm(plain, axis=2, keepdims=True)
    np.testing.assert_allclose(unit, plain / np.sqrt(nrm ** 2 + 1e-6), rtol=1e-13, atol=0)
    np.testing.assert_allclose(np.linalg.norm(unit, axis=2), 1.0, atol=1e-5)


def test_conv_of_malformed_branch_raises():
    x, w = np.zeros((3, 2)), np.ones((2, 4))
    with pytest.raises(ValueError):
        gdn.branch_conv(np.zeros((5, 2)), x, w, 5, [-1, 0, 1])
    with pytest.raises(ValueError):
        gdn.branch_conv(np.zeros((5, 2)), x, w, 2, [-1, 2, 1])
