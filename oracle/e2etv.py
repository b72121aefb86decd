"""E2E-TV surrogate over a proposal tree, forward and gradient (oracle, fp64).

What the pages fix:
  * [R] §1.1 and §3.3 (Eq. 8): under one-sample rejection sampling the
    probability that a drafted token is accepted is the overlap of the draft
    distribution q and the target distribution p, sum_v min(q_v, p_v) =
    1 - TV(q, p).
  * [R] §3.3 (Eq. 9, Bebop's E2E-TV), [S] §2.3: per-position overlaps are
    multiplied along the branch into prefix products, so an early mismatch
    discounts every later term.  [S]: the loss minimised is 1 minus the mean
    prefix product over the B*W proposed tokens.  ([R] states the same
    objective as an average over branches of the sum of prefix products, a
    quantity to maximise; the two are affine in each other.)
  * [R] §3.3: tokens and the target distribution are held fixed; only the
    drafter's probabilities are differentiated (no score-function term).
  * [R] §3.3, Eq. 13: target mass outside the drafter's support stays in the
    loss; q is the softmax over the full vocabulary and p is not
    renormalised.
  * [R] §3.2 (Eq. 18): numerators and counts are kept separate so that a
    global count can normalise per-rank numerators.

Readings where the pages are silent:
  * on a tree, the prefix product of node j runs along its parent chain:
    P_j = alpha_j * P_parent(j), P of the anchor = 1; the mean is over all
    nodes;
  * count = R*Wn unless the caller supplies a global count;
  * derivative of min at a tie q_v = p_v: the strict indicator [q_v < p_v]
    (0 at the tie).

Gradient, written without division so it holds at alpha = 0:
  dL/dalpha_j = -(1/count) * P_parent(j) * S_j,
      S_j = 1 + sum over children c of j of alpha_c * S_c;
  dalpha_j/dz_u = q_u * ([q_u < p_u] - G_j),  G_j = sum_{v: q_v < p_v} q_v
(softmax Jacobian dq_v/dz_u = q_v (delta_uv - q_u)).
"""

from __future__ import annotations

import math

import numpy as np


def logsumexp(x):
    """log sum_v exp(x_v) over the last axis in fp64 (keeps the axis)."""
    x = np.asarray(x, np.float64)
    m = np.max(x, axis=-1, keepdims=True)
    return m + np.log(np.sum(np.exp(x - m), axis=-1, keepdims=True))


def log_softmax(x):
    """log softmax over the last axis in fp64; -inf entries stay -inf."""
    x = np.asarray(x, np.float64)
    return x - logsumexp(x)


def overlap(lq, lp):
    """alpha = sum_v min(q_v, p_v) from log-probabilities (last axis)."""
    return np.sum(np.minimum(np.exp(lq), np.exp(lp)), axis=-1)


def prefix_products(alpha, parent):
    """P_j = alpha_j * P_parent(j) along each branch; alpha/parent [R][Wn]."""
    alpha = np.asarray(alpha, np.float64)
    parent = np.asarray(parent)
    P = np.zeros_like(alpha)
    R, Wn = alpha.shape
    for r in range(R):
        for j in range(Wn):
            p = int(parent[r, j])
            P[r, j] = alpha[r, j] * (1.0 if p < 0 else P[r, p])
    return P


def suffix_sums(alpha, parent):
    """S_j = 1 + sum over children c of alpha_c * S_c, children after parents."""
    alpha = np.asarray(alpha, np.float64)
    parent = np.asarray(parent)
    R, Wn = alpha.shape
    S = np.ones_like(alpha)
    for r in range(R):
        for j in range(Wn - 1, -1, -1):
            p = int(parent[r, j])
            if p >= 0:
                S[r, p] += alpha[r, j] * S[r, j]
    return S


def _rows(x):
    if hasattr(x, "detach"):
        x = x.detach().cpu()
        if x.is_floating_point():
            x = x.double()
        x = x.numpy()
    return np.asarray(x, np.float64)


def e2etv(draft, target, parent, norm_count=None, grad_scale=1.0, with_grad=True,
          row_chunk=64):
    """Forward and gradient for logits [R][Wn][V] and parent [R][Wn].

    Returns a dict with alpha, prefix, G, lse_draft, lse_target ([R][Wn]),
    numer, count, loss (floats) and, if with_grad, grad ([R][Wn][V]) and
    margin = log p - log q ([R][Wn][V]) for tie analysis."""
    parent = np.asarray(parent.detach().cpu() if hasattr(parent, "detach") else parent)
    R, Wn = parent.shape
    V = draft.shape[-1]
    N = R * Wn
    dz = draft.reshape(N, V)
    dt = target.reshape(N, V)
    alpha = np.zeros(N)
    G = np.zeros(N)
    lse_q = np.zeros(N)
    lse_p = np.zeros(N)
    for r0 in range(0, N, row_chunk):
        r1 = min(N, r0 + row_chunk)
        z = _rows(dz[r0:r1])
        t = _rows(dt[r0:r1])
        sz = logsumexp(z)
        st = logsumexp(t)
        lq = z - sz
        lp = t - st
        lse_q[r0:r1] = sz[:, 0]
        lse_p[r0:r1] = st[:, 0]
        alpha[r0:r1] = overlap(lq, lp)
        q = np.exp(lq)
        G[r0:r1] = np.sum(np.where(lq < lp, q, 0.0), axis=-1)
    alpha = alpha.reshape(R, Wn)
    G = G.reshape(R, Wn)
    P = prefix_products(alpha, parent)
    numer = math.fsum(P.ravel().tolist())
    count = float(norm_count) if (norm_count is not None and norm_count > 0) else float(N)
    out = {
        "alpha": alpha, "prefix": P, "G": G,
        "lse_draft": lse_q.reshape(R, Wn), "lse_target": lse_p.reshape(R, Wn),
        "numer": numer, "count": count, "loss": 1.0 - numer / count,
    }
    if not with_grad:
        return out
    S = suffix_sums(alpha, parent)
    Ppar = np.where(parent < 0, 1.0, np.take_along_axis(P, np.maximum(parent, 0), axis=1))
    c = -grad_scale * Ppar * S / count
    out["S"] = S
    out["dL_dalpha"] = c
    grad = np.zeros((N, V))
    margin = np.zeros((N, V))
    cf = c.reshape(N)
    Gf = G.reshape(N)
    for r0 in range(0, N, row_chunk):
        r1 = min(N, r0 + row_chunk)
        lq = log_softmax(_rows(dz[r0:r1]))
        lp = log_softmax(_rows(dt[r0:r1]))
        q = np.exp(lq)
        ind = (lq < lp).astype(np.float64)
        grad[r0:r1] = cf[r0:r1, None] * q * (ind - Gf[r0:r1, None])
        with np.errstate(invalid="ignore"):
            margin[r0:r1] = lp - lq  # nan where both are -inf (no mass either side)
    out["grad"] = grad.reshape(R, Wn, V)
    out["margin"] = margin.reshape(R, Wn, V)
    return out


def e2etv_branch(draft_b, target_b, parent_b, count, grad_scale=1.0):
    """One branch's alpha, prefix, dL/dalpha and gradient rows, given the
    global count.  Everything a branch needs lives inside it (prefix products
    and suffix sums never cross branches), so sampled branches of a large
    batch can be checked one at a time."""
    parent_b = np.asarray(parent_b).reshape(1, -1)
    Wn = parent_b.shape[1]
    V = draft_b.shape[-1]
    res = e2etv(draft_b.reshape(1, Wn, V), target_b.reshape(1, Wn, V), parent_b,
                norm_count=count, grad_scale=grad_scale)
    return res
