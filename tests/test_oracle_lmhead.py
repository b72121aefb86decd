"""Pins of the fused LM-head + E2E-TV oracle (CPU only).

The oracle composes a linear head with oracle.e2etv; the pins check the
composition against facts that do not come from its code: an identity head
reduces it to E2E-TV on the hidden states, softmax is blind to a per-row
logit shift (a head changed by a direction every row sees equally), the
target gather follows the score-row rule ([R] §3.2(a), Fig. 3: siblings share
their parent's row), and the returned logit gradient times the draft head is
the finite-difference gradient with respect to the hidden states."""

import numpy as np
import pytest

import oracle
from oracle import lmhead as lm


def _case(seed, R=3, Wn=4, H=12, V=30, M=None):
    rng = np.random.default_rng(seed)
    M = M or R * Wn
    return (rng, rng.standard_normal((R, Wn, H)), rng.standard_normal((V, H)) / np.sqrt(H) * 3,
            rng.standard_normal((M, H)), rng.standard_normal((V, H)) / np.sqrt(H) * 3,
            rng.integers(0, M, (R, Wn)), np.tile([-1] + list(range(Wn - 1)), (R, 1)))


def test_identity_head_is_e2etv_on_the_hidden_states():
    rng = np.random.default_rng(0)
    R, Wn, V = 2, 3, 9
    hd = rng.standard_normal((R, Wn, V))
    ht = rng.standard_normal((R * Wn, V))
    par = np.array([[-1, 0, 1], [-1, 0, 0]])
    I = np.eye(V)
    a = lm.lmhead_e2etv(hd, I, ht, I, np.arange(R * Wn).reshape(R, Wn), par)
    b = oracle.e2etv(hd, ht.reshape(R, Wn, V), par)
    assert a["loss"] == pytest.approx(b["loss"], abs=1e-15)
    assert np.allclose(a["grad"], b["grad"], atol=1e-15)
    assert np.allclose(a["alpha"], b["alpha"], atol=1e-15)


def test_a_shift_every_row_sees_equally_changes_nothing():
    rng, hd, Wd, ht, Wt, tr, par = _case(1)
    base = lm.lmhead_e2etv(hd, Wd, ht, Wt, tr, par)
    # adding the same vector u to every head row adds h.u to all of a row's
    # logits: the softmaxes, and so loss and logit gradient, do not move
    u = rng.standard_normal(Wd.shape[1])
    sh = lm.lmhead_e2etv(hd, Wd + u, ht, Wt + 2 * u, tr, par)
    assert sh["loss"] == pytest.approx(base["loss"], rel=1e-12)
    assert np.allclose(sh["grad"], base["grad"], atol=1e-12)


def test_siblings_read_their_parents_row():
    # a forked branch: node 0 on the anchor, nodes 1 and 2 both children of 0
    rng = np.random.default_rng(2)
    H, V = 6, 11
    hd = rng.standard_normal((1, 3, H))
    trunk = rng.standard_normal((5, H))       # trunk score rows; anchor 3
    nodes = rng.standard_normal((3, H))       # branch score rows
    ht = np.concatenate([trunk, nodes])
    par = np.array([[-1, 0, 0]])
    rows = []
    for j in range(3):
        kind, i = oracle.score_row_source(3, par[0], j)
        rows.append(i if kind == "trunk" else 5 + i)
    assert rows == [3, 5, 5]
    Wd, Wt = rng.standard_normal((V, H)), rng.standard_normal((V, H))
    res = lm.lmhead_e2etv(hd, Wd, ht, Wt, np.array([rows]), par)
    # the same target rows written out by hand
    t = np.stack([trunk[3], nodes[0], nodes[0]]) @ Wt.T
    ref = oracle.e2etv(hd @ Wd.T, t[None], par)
    assert np.allclose(res["alpha"], ref["alpha"], atol=1e-14)
    assert res["alpha"][0, 1] != res["alpha"][0, 2] or np.allclose(hd[0, 1], hd[0, 2])


def test_logit_gradient_times_head_is_the_hidden_gradient():
    rng, hd, Wd, ht, Wt, tr, par = _case(3, R=2, Wn=3, H=5, V=13)
    res = lm.lmhead_e2etv(hd, Wd, ht, Wt, tr, par)
    dh = res["grad"] @ Wd   # [R][Wn][H]
    eps = 1e-6
    for (r, j, k) in [(0, 0, 0), (0, 2, 3), (1, 1, 4), (1, 0, 2)]:
        hp, hm = hd.copy(), hd.copy()
        hp[r, j, k] += eps
        hm[r, j, k] -= eps
        fd = (lm.lmhead_e2etv(hp, Wd, ht, Wt, tr, par, with_grad=False)["loss"]
              - lm.lmhead_e2etv(hm, Wd, ht, Wt, tr, par, with_grad=False)["loss"]) / (2 * eps)
        assert fd == pytest.approx(dh[r, j, k], rel=1e-5, abs=1e-9)


def test_logits_are_the_linear_map():
    rng = np.random.default_rng(4)
    h = rng.standard_normal((3, 4))
    W = rng.standard_normal((5, 4))
    got = lm.lmhead_logits(h, W)
    for i in range(3):
        for v in range(5):
            assert got[i, v] == pytest.approx(sum(h[i, k] * W[v, k] for k in range(4)), abs=1e-13)
