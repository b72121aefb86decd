"""Pins of the E2E-TV oracle against facts fixed outside its own code:
worked examples printed on the pages, the rejection-sampling identity by
Monte Carlo, closed forms, brute-force derivative sums and finite
differences."""

import math

import numpy as np
import pytest
from hypothesis import assume, given, settings, strategies as st

import oracle
from conftest import golden_dict


def _logits(probs):
    p = np.asarray(probs, np.float64)
    with np.errstate(divide="ignore"):
        return np.log(p)


def _one_row(q, p):
    z = _logits(q)[None, None, :]
    t = _logits(p)[None, None, :]
    return oracle.e2etv(z, t, np.array([[-1]]))


def test_eq13_worked_example():
    g = golden_dict("eq13_overlap.txt")
    q = [float(x) for x in g["q"][0]]
    p = [float(x) for x in g["p"][0]]
    res = _one_row(q, p)
    assert res["alpha"][0, 0] == pytest.approx(float(g["overlap"][0][0]), abs=1e-12)
    tv = 0.5 * sum(abs(a - b) for a, b in zip(q, p))
    assert tv == pytest.approx(float(g["tv"][0][0]), abs=1e-12)
    # Renormalising p over q's support (what the method avoids) would read 1.
    supp = [i for i, x in enumerate(q) if x > 0]
    pr = np.zeros(len(p))
    pr[supp] = np.asarray(p)[supp] / sum(p[i] for i in supp)
    res2 = _one_row(q, pr)
    assert res2["alpha"][0, 0] == pytest.approx(float(g["overlap_renormalised"][0][0]), abs=1e-12)
    # loss of a one-node branch is 1 - alpha
    assert res["loss"] == pytest.approx(1.0 - 0.8, abs=1e-12)


def test_appC2_first_overlap():
    g = golden_dict("appC2_alpha.txt")
    q = [float(x) for x in g["q1"][0]]
    p = [float(x) for x in g["p1"][0]]
    assert _one_row(q, p)["alpha"][0, 0] == pytest.approx(float(g["alpha1"][0][0]), abs=1e-12)


def test_overlap_is_one_minus_tv_and_symmetric():
    rng = np.random.default_rng(1)
    z = rng.normal(0, 2, (3, 5, 37))
    t = rng.normal(0, 2, (3, 5, 37))
    par = np.tile(np.array([-1, 0, 1, 2, 3]), (3, 1))
    a = oracle.e2etv(z, t, par)["alpha"]
    b = oracle.e2etv(t, z, par)["alpha"]
    q = np.exp(z - z.max(-1, keepdims=True)); q /= q.sum(-1, keepdims=True)
    p = np.exp(t - t.max(-1, keepdims=True)); p /= p.sum(-1, keepdims=True)
    tv = 0.5 * np.abs(q - p).sum(-1)
    np.testing.assert_allclose(a, 1 - tv, atol=1e-12)
    np.testing.assert_allclose(a, b, atol=1e-12)
    assert np.all(a >= 0) and np.all(a <= 1)


def test_monte_carlo_acceptance_equals_overlap():
    # [R] §1.1: one-sample rejection sampling accepts a drafted token with
    # probability equal to the overlap.  Draw x ~ q, accept w.p. min(1, p_x/q_x).
    rng = np.random.default_rng(7)
    q = np.array([0.35, 0.25, 0.2, 0.15, 0.05])
    p = np.array([0.1, 0.4, 0.1, 0.3, 0.1])
    n = 1_000_000
    x = rng.choice(len(q), size=n, p=q)
    acc = rng.random(n) < np.minimum(1.0, p[x] / q[x])
    rate = acc.mean()
    alpha = _one_row(q, p)["alpha"][0, 0]
    sigma = math.sqrt(alpha * (1 - alpha) / n)
    assert abs(rate - alpha) < 4 * sigma


def test_identical_and_disjoint():
    rng = np.random.default_rng(2)
    z = rng.normal(0, 1, (2, 4, 50))
    par = np.tile(np.array([-1, 0, 1, 2]), (2, 1))
    r = oracle.e2etv(z, z.copy(), par)
    np.testing.assert_allclose(r["alpha"], 1.0, atol=1e-12)
    assert r["loss"] == pytest.approx(0.0, abs=1e-12)
    assert np.all(r["grad"] == 0.0)
    # disjoint supports
    z = np.full((1, 3, 6), -np.inf)
    t = np.full((1, 3, 6), -np.inf)
    z[..., :3] = 0.0
    t[..., 3:] = 0.0
    r = oracle.e2etv(z, t, np.array([[-1, 0, 1]]))
    np.testing.assert_allclose(r["alpha"], 0.0, atol=1e-15)
    assert r["loss"] == pytest.approx(1.0, abs=1e-15)


def _row_with_overlap(a):
    """Two-token logits with overlap a: q = (1, 0), p = (a, 1-a)."""
    return _logits([1.0, 0.0]), _logits([a, 1.0 - a])


def test_earlier_error_costs_more():
    # [R] §3.3: the same per-token error costs more when it comes earlier.
    # W = 2, alpha = (.5, 1) vs (1, .5): prefix means .5 vs .75.
    def loss(alphas):
        z = np.stack([_row_with_overlap(a)[0] for a in alphas])[None]
        t = np.stack([_row_with_overlap(a)[1] for a in alphas])[None]
        return oracle.e2etv(z, t, np.array([[-1, 0]]))["loss"]
    early, late = loss([0.5, 1.0]), loss([1.0, 0.5])
    assert early == pytest.approx(0.5, abs=1e-12)
    assert late == pytest.approx(0.25, abs=1e-12)
    assert early > late


@pytest.mark.parametrize("a", [0.0, 0.3, 0.7, 1.0])
@pytest.mark.parametrize("W", [1, 2, 7])
def test_constant_alpha_chain_closed_form(a, W):
    zr, tr = _row_with_overlap(a)
    z = np.tile(zr, (1, W, 1))
    t = np.tile(tr, (1, W, 1))
    par = np.array([[-1] + list(range(W - 1))])
    got = oracle.e2etv(z, t, par)["loss"]
    # mean of a, a^2, ..., a^W (geometric series)
    want = 0.0 if a == 1.0 else 1.0 - a * (1 - a ** W) / (W * (1 - a))
    assert got == pytest.approx(want, abs=1e-12)


def test_eq18_split_invariance():
    # [R] §3.2 (Eq. 18): per-rank numerators normalised by the global count.
    rng = np.random.default_rng(3)
    R, Wn, V = 12, 5, 40
    z = rng.normal(0, 1.5, (R, Wn, V))
    t = z + rng.normal(0, 1, (R, Wn, V))
    par = np.tile(np.array([-1, 0, 1, 1, 3]), (R, 1))
    full = oracle.e2etv(z, t, par)
    cut = [0, 3, 4, 9, 12]
    numer = 0.0
    for a, b in zip(cut[:-1], cut[1:]):
        part = oracle.e2etv(z[a:b], t[a:b], par[a:b], norm_count=R * Wn)
        numer += part["numer"]
        np.testing.assert_allclose(part["grad"], full["grad"][a:b], atol=1e-15)
    assert 1 - numer / (R * Wn) == pytest.approx(full["loss"], abs=1e-12)


def _random_tree(rng, Wn):
    return np.array([-1] + [int(rng.integers(-1, j)) for j in range(1, Wn)])


@settings(max_examples=40, deadline=None)
@given(st.integers(0, 10_000), st.integers(1, 9))
def test_prefix_products_nonincreasing(seed, Wn):
    rng = np.random.default_rng(seed)
    par = np.stack([_random_tree(rng, Wn) for _ in range(3)])
    z = rng.normal(0, 2, (3, Wn, 11))
    t = rng.normal(0, 2, (3, Wn, 11))
    r = oracle.e2etv(z, t, par)
    P = r["prefix"]
    for b in range(3):
        for j in range(Wn):
            p = par[b, j]
            parent_val = 1.0 if p < 0 else P[b, p]
            assert P[b, j] <= parent_val + 1e-15
            # brute force: product of alphas on the path
            path = oracle.walk_ancestors(par[b], j)
            assert P[b, j] == pytest.approx(np.prod(r["alpha"][b, path]), rel=1e-12)


def test_division_free_equals_descendant_sum():
    # dL/dalpha_n = -(1/count) * sum over m in subtree(n) of P_m / alpha_n
    rng = np.random.default_rng(4)
    R, Wn = 4, 8
    par = np.stack([_random_tree(rng, Wn) for _ in range(R)])
    z = rng.normal(0, 1, (R, Wn, 9))
    t = rng.normal(0, 1, (R, Wn, 9))
    r = oracle.e2etv(z, t, par)
    count = R * Wn
    for b in range(R):
        for n in range(Wn):
            sub = [m for m in range(Wn) if n in oracle.walk_ancestors(par[b], m)]
            naive = -sum(r["prefix"][b, m] for m in sub) / r["alpha"][b, n] / count
            assert r["dL_dalpha"][b, n] == pytest.approx(naive, rel=1e-10)


@settings(max_examples=25, deadline=None)
@given(st.integers(0, 10_000))
def test_gradient_finite_difference(seed):
    rng = np.random.default_rng(seed)
    R, Wn, V = 2, int(rng.integers(1, 6)), 7
    par = np.stack([_random_tree(rng, Wn) for _ in range(R)])
    z = rng.normal(0, 1.5, (R, Wn, V))
    t = rng.normal(0, 1.5, (R, Wn, V))
    r = oracle.e2etv(z, t, par, grad_scale=1.0)
    assume(np.min(np.abs(r["margin"])) > 1e-4)  # stay off the kinks of min()
    eps = 1e-6
    for _ in range(10):
        b, j, u = rng.integers(R), rng.integers(Wn), rng.integers(V)
        zp, zm = z.copy(), z.copy()
        zp[b, j, u] += eps
        zm[b, j, u] -= eps
        fd = (oracle.e2etv(zp, t, par, with_grad=False)["loss"]
              - oracle.e2etv(zm, t, par, with_grad=False)["loss"]) / (2 * eps)
        assert r["grad"][b, j, u] == pytest.approx(fd, abs=1e-8)


def test_grad_scale_and_row_sums():
    rng = np.random.default_rng(5)
    z = rng.normal(0, 2, (3, 4, 30))
    t = rng.normal(0, 2, (3, 4, 30))
    par = np.tile(np.array([-1, 0, 1, 2]), (3, 1))
    r1 = oracle.e2etv(z, t, par)
    r2 = oracle.e2etv(z, t, par, grad_scale=2.5)
    np.testing.assert_allclose(r2["grad"], 2.5 * r1["grad"], rtol=1e-14)
    # softmax Jacobian: each gradient row sums to zero
    np.testing.assert_allclose(r1["grad"].sum(-1), 0.0, atol=1e-15)


def test_single_node_closed_form():
    # W = 1, count 1: L = 1 - alpha, dL/dz_u = -q_u ([q_u<p_u] - G)
    q = np.array([0.5, 0.3, 0.2])
    p = np.array([0.2, 0.3001, 0.4999])
    r = _one_row(q, p)
    ind = (q < p).astype(float)
    G = float((q * ind).sum())
    np.testing.assert_allclose(r["grad"][0, 0], -q * (ind - G), atol=1e-15)
