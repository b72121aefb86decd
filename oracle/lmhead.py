"""LM head fused with the E2E-TV surrogate (oracle, fp64) — TEST
INFRASTRUCTURE.

What the pages fix:
  * [R] §3.3 (Eqs. 8, 9, 13): the loss compares, at every proposed token, the
    drafter's distribution q with the target's distribution p over the full
    vocabulary; both are softmaxes of the two models' output logits.
  * [R] §3.2(a) reading rule (Fig. 3) and [S] §2.2: the target logits that
    score branch token j come from the row of its parent (the anchor's trunk
    row for a token attached to the anchor), so sibling tokens read the same
    target row; oracle.rows states the rule.

Readings where the pages are silent:
  * an LM head is a plain linear map of the last hidden state, logits =
    h W^T, no bias, for the drafter and for the target (the two heads may be
    the same matrix);
  * the target side is constant (no gradient); the gradient returned is with
    respect to the draft logits, the quantity a linear head turns into the
    hidden-state gradient dL/dh = (dL/dz) W_draft.

The fused kernel never stores the logits; this oracle is the plain
definition: form both logit matrices, then oracle.e2etv.
"""

from __future__ import annotations

import numpy as np

from .e2etv import e2etv


def lmhead_logits(h, W):
    """Logits h W^T in fp64 for hidden states h [..., H] and a head W [V][H]."""
    return np.asarray(h, np.float64) @ np.asarray(W, np.float64).T


def lmhead_e2etv(h_draft, W_draft, h_target, W_target, target_row, parent, norm_count=None,
                 grad_scale=1.0, with_grad=True):
    """E2E-TV of the two heads' distributions.

    h_draft [R][Wn][H]: the drafter's hidden state at every branch node;
    h_target [M][H]: the target's hidden states of the score rows;
    target_row [R][Wn]: the score row whose target logits node n is scored
    against; parent [R][Wn]; W_draft, W_target [V][H].  Returns what
    oracle.e2etv returns for logits z = h_draft W_draft^T and
    t = h_target[target_row] W_target^T (grad is dL/dz)."""
    parent = np.asarray(parent)
    R, Wn = parent.shape
    hd = np.asarray(h_draft, np.float64).reshape(R * Wn, -1)
    ht = np.asarray(h_target, np.float64)[np.asarray(target_row).reshape(-1)]
    z = lmhead_logits(hd, W_draft)
    t = lmhead_logits(ht, W_target)
    V = z.shape[-1]
    return e2etv(z.reshape(R, Wn, V), t.reshape(R, Wn, V), parent, norm_count=norm_count,
                 grad_scale=grad_scale, with_grad=with_grad)
