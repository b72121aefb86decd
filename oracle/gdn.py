"""Linear-attention (GDN) branch scoring by indexed state replay (oracle, fp64)
— TEST INFRASTRUCTURE.

What the pages fix ([R] §3.2(c), Fig. 5; [S] §1):
  * a linear-attention target keeps one recurrent state per head, so a mask
    cannot rewind it to an anchor: the shared trunk pass stores the state as
    immutable FP32 checkpoints every C = 64 trunk tokens (Fig. 5: the state
    after the 64th token);
  * the state at an anchor is restored by copying the nearest checkpoint and
    replaying only the trunk suffix after it up to the anchor; the branch
    tokens then update and read that private copy, so the shared checkpoints
    never change;
  * [R] §3.4 (Eq. 20 and the text after it): the GDN updates of shared
    execution, replay included, are counted against cacheless scoring
    (24.9x at L = 2048, W = 7, K = 512).

  * [R] §3.2(c): the convolution history, like the recurrent state, follows
    only the branch's ancestors.

Readings where the pages are silent:
  * the recurrence is the gated delta rule as published for Gated DeltaNet:
    per head, with a state S of shape [Dv][Dk],
        S_t = alpha_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
        o_t = S_t q_t,
    alpha_t in (0, 1] a decay gate, beta_t in [0, 1] a write strength, keys
    unit length; the projections, the short convolution and the output gate
    of a GDN layer are upstream or downstream of this step and not part of it;
  * a checkpoint holds the state after trunk tokens 0..(m+1)C-1; the state at
    anchor a (after trunk tokens 0..a) starts from the last checkpoint at or
    before a (none: the zero state) and replays the (a + 1) mod C tokens after
    it;
  * a branch node's state is its parent's state (the anchor state for a root)
    updated with the node's own (k, v, alpha, beta); its output reads that
    state with the node's query.  Nodes come in an order where each parent
    precedes its children.
  * the convolution is Gated DeltaNet's short convolution: per channel a
    causal depthwise convolution of width K over the layer's projected
    inputs, then SiLU (z sigmoid(z)); q and k are then scaled to unit length
    per head (x / sqrt(sum x^2 + 1e-6), the epsilon guarding a zero vector).
    For a branch node the K inputs are the node's own, then its ancestors',
    then trunk tokens a, a - 1, ..., with zeros before the trunk's start.
"""

from __future__ import annotations

import numpy as np


def gated_delta_update(S, k, v, alpha, beta):
    """One gated delta-rule step on state S [Dv][Dk] with key k [Dk], value
    v [Dv], gate alpha and write strength beta (fp64)."""
    S = np.asarray(S, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    Sk = S @ k
    return float(alpha) * (S - float(beta) * np.outer(Sk, k)) + float(beta) * np.outer(v, k)


def gdn_read(S, q):
    """A token's output: the state applied to its query."""
    return np.asarray(S, np.float64) @ np.asarray(q, np.float64)


def run_tokens(S0, k, v, alpha, beta):
    """Apply a sequence of updates (k [n][Dk], v [n][Dv], alpha, beta [n]) to
    S0 and return every intermediate state [n][Dv][Dk]."""
    S = np.asarray(S0, np.float64).copy()
    out = np.empty((len(alpha),) + S.shape)
    for t in range(len(alpha)):
        S = gated_delta_update(S, k[t], v[t], alpha[t], beta[t])
        out[t] = S
    return out


def trunk_checkpoints(k, v, alpha, beta, C=64):
    """The shared trunk pass's checkpoints: k, v [L][H][D], alpha, beta [L][H]
    -> [L // C][H][D][D], entry m the state after trunk tokens 0..(m+1)C-1,
    starting from the zero state."""
    k = np.asarray(k, np.float64)
    L, H, D = k.shape
    Dv = np.asarray(v).shape[2]
    ck = np.zeros((L // C, H, Dv, D))
    for h in range(H):
        S = np.zeros((Dv, D))
        for t in range(L):
            S = gated_delta_update(S, k[t, h], v[t, h], alpha[t, h], beta[t, h])
            if (t + 1) % C == 0:
                ck[(t + 1) // C - 1, h] = S
    return ck


def replay_span(a, C=64):
    """(checkpoint index or -1 for the zero state, first replayed trunk token)
    for anchor a: the last checkpoint at or before a, then tokens up to a."""
    m = (int(a) + 1) // C
    return m - 1, m * C


def anchor_state(ckpt, k, v, alpha, beta, a, h, C=64):
    """State of head h after trunk tokens 0..a, restored from the checkpoints
    ckpt [NC][H][Dv][Dk] and the trunk tokens k, v [L][H][D], alpha, beta
    [L][H] by replaying the suffix after the nearest checkpoint."""
    c, t0 = replay_span(a, C)
    S = np.asarray(ckpt[c, h], np.float64).copy() if c >= 0 else np.zeros(np.asarray(ckpt).shape[2:])
    for t in range(t0, int(a) + 1):
        S = gated_delta_update(S, k[t][h], v[t][h], alpha[t][h], beta[t][h])
    return S


def check_branch(parent, a, L):
    """Raise ValueError unless 0 <= a < L and every parent precedes its node."""
    if not (0 <= int(a) < L):
        raise ValueError(f"anchor {a} outside [0, {L})")
    for j, p in enumerate(parent):
        if not (-1 <= int(p) < j):
            raise ValueError(f"node {j}: parent {p} does not precede it")


def gdn_branch(ckpt, trunk_k, trunk_v, trunk_alpha, trunk_beta, a, parent,
               q, k, v, alpha, beta, C=64):
    """Outputs [Wn][H][Dv] of one branch anchored at a.

    ckpt [NC][H][Dv][Dk]; trunk_* [L][H]...; parent [Wn]; q, k, v [Wn][H][D];
    alpha, beta [Wn][H]."""
    L = np.asarray(trunk_alpha).shape[0]
    check_branch(parent, a, L)
    Wn, H, _ = np.asarray(q).shape
    Dv = np.asarray(v).shape[2]
    out = np.empty((Wn, H, Dv))
    for h in range(H):
        Sa = anchor_state(ckpt, trunk_k, trunk_v, trunk_alpha, trunk_beta, a, h, C)
        states = []
        for j in range(Wn):
            Sp = Sa if parent[j] < 0 else states[int(parent[j])]
            Sj = gated_delta_update(Sp, k[j][h], v[j][h], alpha[j][h], beta[j][h])
            states.append(Sj)
            out[j, h] = gdn_read(Sj, q[j][h])
    return out


def gdn_replay(ckpt, trunk_k, trunk_v, trunk_gate, trunk_beta, anchors, parent,
               q, k, v, gate, beta, C=64, branches=None):
    """Every branch's node outputs [T][B][Wn][H][Dv] (NaN for branches not in
    ``branches``, a list of (t, b), when given)."""
    ckpt = np.asarray(ckpt, np.float64)
    trunk_k = np.asarray(trunk_k, np.float64)
    trunk_v = np.asarray(trunk_v, np.float64)
    trunk_gate = np.asarray(trunk_gate, np.float64)
    trunk_beta = np.asarray(trunk_beta, np.float64)
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    gate = np.asarray(gate, np.float64)
    beta = np.asarray(beta, np.float64)
    anchors = np.asarray(anchors)
    parent = np.asarray(parent)
    T, B, Wn, H, _ = q.shape
    out = np.full((T, B, Wn, H, v.shape[-1]), np.nan)
    todo = branches if branches is not None else [(t, b) for t in range(T) for b in range(B)]
    for t, b in todo:
        out[t, b] = gdn_branch(ckpt[t], trunk_k[t], trunk_v[t], trunk_gate[t], trunk_beta[t],
                               anchors[t, b], parent[t, b], q[t, b], k[t, b], v[t, b],
                               gate[t, b], beta[t, b], C)
    return out


def update_counts(L, anchors, W, C=64):
    """GDN state updates of cacheless scoring and of shared execution for
    W-token branches at the given anchors ([R] §3.4): cacheless scoring runs
    every branch's whole history, the a + 1 trunk tokens and its W - 1 scored
    tokens, from scratch; shared execution runs the trunk once, then per
    branch the replay after the nearest checkpoint and W - 1 branch updates."""
    anchors = np.asarray(anchors, np.int64)
    cacheless = int(np.sum(anchors + 1 + (W - 1)))
    replay = np.array([int(a) + 1 - replay_span(a, C)[1] for a in anchors])
    shared = int(L + np.sum(replay) + len(anchors) * (W - 1))
    return cacheless, shared


def conv_history(a, parent, j, K):
    """The K inputs node j's convolution reads, newest first: ('n', i) for
    branch node i, ('t', s) for trunk token s, None before the trunk."""
    out = []
    x = int(j)
    s = int(a)
    for _ in range(K):
        if x >= 0:
            out.append(("n", x))
            x = int(parent[x])
        elif s >= 0:
            out.append(("t", s))
            s -= 1
        else:
            out.append(None)
    return out


def branch_conv(trunk_x, x, w, a, parent, D=None, l2norm=False):
    """One branch's convolved inputs [Wn][C]: trunk_x [L][C] and x [Wn][C] are
    the layer's projected inputs before the convolution, w [C][K] its weights
    (w[:, i] multiplies the i-th newest input).  With l2norm, every head of D
    channels is scaled to unit length."""
    trunk_x = np.asarray(trunk_x, np.float64)
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    check_branch(parent, a, trunk_x.shape[0])
    Wn, C = x.shape
    K = w.shape[1]
    out = np.empty((Wn, C))
    for j in range(Wn):
        z = np.zeros(C)
        for i, src in enumerate(conv_history(a, parent, j, K)):
            if src is None:
                continue
            z += w[:, i] * (x[src[1]] if src[0] == "n" else trunk_x[src[1]])
        y = z / (1.0 + np.exp(-z))
        if l2norm:
            y = y.reshape(-1, D)
            y = y / np.sqrt((y * y).sum(axis=1, keepdims=True) + 1e-6)
            y = y.reshape(C)
        out[j] = y
    return out


def gdn_branch_conv(trunk_x, x, w, anchors, parent, D=None, l2norm=False, branches=None):
    """Every branch's convolved inputs: trunk_x [T][L][C], x [T][B][Wn][C] ->
    [T][B][Wn][C] (NaN for branches not in ``branches`` when given)."""
    x = np.asarray(x, np.float64)
    T, B = x.shape[:2]
    out = np.full(x.shape, np.nan)
    todo = branches if branches is not None else [(t, b) for t in range(T) for b in range(B)]
    for t, b in todo:
        out[t, b] = branch_conv(trunk_x[t], x[t, b], w, anchors[t, b], parent[t, b], D, l2norm)
    return out
