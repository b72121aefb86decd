"""Which packed row scores which branch token (oracle bookkeeping).

[R] §3.2(a) (Fig. 3) and [S] §2.2: the anchor's trunk row scores a branch's
first token and each branch row scores the token after it.  A row reads
itself, but logits come from the predecessor row, so the scored token never
leaks into its own prediction.  The last sample of a branch is scored but
predicts nothing, so it needs no query row: a W-token chain adds W-1 new
score rows, and B chains add B(W-1) after the shared trunk pass.  [R] §3.4
(Eq. 20): trunk rows plus new rows, L + K(W-1) in total.
"""

from __future__ import annotations


def score_row_source(anchor: int, parent, j: int):
    """Row whose output scores branch token j: ("trunk", anchor) for a token
    attached to the anchor, else ("node", parent[j])."""
    p = int(parent[j])
    return ("trunk", int(anchor)) if p < 0 else ("node", p)


def new_score_rows(parent):
    """Branch nodes whose rows are read by some score (nodes that are some
    token's parent).  Leaves are not in the set."""
    return sorted({int(p) for p in parent if int(p) >= 0})


def shared_row_count(L: int, branch_parents) -> int:
    """Rows of the shared pass: the L trunk rows plus every branch's new rows."""
    return L + sum(len(new_score_rows(p)) for p in branch_parents)
