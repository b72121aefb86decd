"""The comparison rules themselves (tests/parity.py), on the CPU: the
per-element tie bound follows from fp32 rounding, and the gradient check
accepts a flipped indicator only inside that bound."""

import numpy as np
import pytest

from parity import check_grad_rows, tie_tau


def test_tie_tau_is_a_few_fp32_ulps():
    # |lq| = 17 log2 units (a typical probability at V = 151,936): ulp 2^-19
    lq = np.array([-17.0 / 1.4426950408889634])
    tau = tie_tau(lq, lq)[0]
    assert tau == pytest.approx(0.6931471805599453 * (4 * 2.0 ** -19 + 2e-6))
    assert 5e-6 < tau < 1e-5
    # larger magnitudes, larger bound; never below the log-sum-exp term
    assert tie_tau(np.array([-60.0]), np.array([-60.0]))[0] > tau
    assert tie_tau(np.array([0.0]), np.array([0.0]))[0] >= 0.6931471805599453 * 2e-6


def _row(margin_at_flip):
    """A 3-token row; the oracle decides token 0's indicator in fp64 with
    log p - log q = margin_at_flip, and the "GPU" flipped it."""
    q = np.array([0.2, 0.3, 0.5])
    lq = np.log(q)
    lp = lq + np.array([margin_at_flip, -0.5, 0.3])
    ind = (lq < lp).astype(float)
    G = float((q * ind).sum())
    c = -0.7
    ref = c * q * (ind - G)
    flip = ind.copy()
    flip[0] = 1.0 - flip[0]
    Gf = float((q * flip).sum())
    gpu = c * q * (flip - Gf)
    return gpu[None], ref[None], (lp - lq)[None], q[None], np.array([c])


def test_a_flip_inside_the_bound_is_accepted():
    gpu, ref, margin, q, c = _row(1e-6)   # bound here: ln2 * (4 ulp(2.3) + 2e-6) = 2.05e-6
    check_grad_rows(gpu, ref, margin, q, c)


def test_a_flip_outside_the_bound_is_caught():
    gpu, ref, margin, q, c = _row(1e-3)
    with pytest.raises(AssertionError):
        check_grad_rows(gpu, ref, margin, q, c)
