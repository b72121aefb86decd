"""Tree-masked GQA attention of branch rows against a shared trunk cache
(oracle, fp64, explicit masks).

What the pages fix:
  * [R] §3.1 step 2 and [S] §2.1: position i of branch b is conditioned on
    the reference prefix up to the anchor a_b and the branch's own earlier
    samples, nothing else.  The first node's parent is the anchor; later
    nodes' parents are earlier samples; the semantic position of a node is the
    anchor position plus its offset.
  * [R] §3.2(a), Eq. 5, and [S] §2.2: the trunk K/V is computed once and
    cached; every branch query is attached to that cache in one packed batch;
    a tree mask lets each query read only itself and its ancestors.  Sibling
    branches and reference tokens after the anchor are masked.  Rotary
    embeddings use logical positions (oracle.rope).

Readings where the pages are silent:
  * the trunk cache holds keys already rotated at their trunk positions; the
    branch q/k arrive unrotated and are rotated at their semantic positions;
  * a row sees trunk positions 0..a_b inclusive (the anchor token is the first
    node's parent) and itself;
  * scores are scaled by 1/sqrt(D); query head h reads kv head floor(h/G),
    G = Hq/Hkv;
  * every node gets an output row, including the terminal one whose output no
    score reads ([R] §3.2(a) reading rule; oracle.rows).

The method is exact: tree scoring must give what scoring each branch on its
own would give ([R] §3.2 "numerical consistency", Table 4), so this oracle is
plain masked softmax attention with the mask built by walking parent chains.
"""

from __future__ import annotations

import numpy as np

from .rope import rope


def walk_ancestors(parent, j: int):
    """Nodes on the path from node j up to the anchor, self first.

    Raises ValueError for a malformed parent map (parent not earlier, or out
    of range)."""
    parent = [int(p) for p in parent]
    out = []
    k = j
    while k != -1:
        if not (0 <= k < len(parent)):
            raise ValueError(f"parent chain leaves the branch at {k}")
        p = parent[k]
        if not (-1 <= p < k):
            raise ValueError(f"node {k} has parent {p}; parents must precede children")
        out.append(k)
        k = p
    return out


def tree_depths(parent):
    """Offset of every node from its anchor (0 for the anchor's child)."""
    return np.array([len(walk_ancestors(parent, j)) - 1 for j in range(len(parent))],
                    dtype=np.int64)


def check_positions(anchor: int, parent, pos) -> None:
    """Semantic position of node j must be anchor + 1 + depth(j) ([S] §2.1)."""
    d = tree_depths(parent)
    want = int(anchor) + 1 + d
    got = np.asarray(pos, dtype=np.int64)
    if not np.array_equal(want, got):
        raise ValueError(f"semantic positions {got.tolist()} != anchor+1+depth {want.tolist()}")


def branch_mask(L: int, anchor: int, parent) -> np.ndarray:
    """Boolean mask [Wn, L + Wn] over keys (trunk 0..L-1, then the branch's
    own nodes): row j may read trunk s iff s <= anchor, node k iff k is j or
    an ancestor of j."""
    Wn = len(parent)
    m = np.zeros((Wn, L + Wn), dtype=bool)
    for j in range(Wn):
        m[j, : int(anchor) + 1] = True
        for k in walk_ancestors(parent, j):
            m[j, L + k] = True
    return m


def packed_tree_mask(L: int, anchors, parent) -> np.ndarray:
    """The whole packed batch's mask for one trunk (Eq. 5): rows are the B*Wn
    branch nodes in packing order, keys are trunk 0..L-1 followed by all B*Wn
    branch nodes.  A row never reads another branch's nodes."""
    anchors = np.asarray(anchors)
    parent = np.asarray(parent)
    B, Wn = parent.shape
    m = np.zeros((B * Wn, L + B * Wn), dtype=bool)
    for b in range(B):
        mb = branch_mask(L, int(anchors[b]), parent[b])
        rows = slice(b * Wn, (b + 1) * Wn)
        m[rows, :L] = mb[:, :L]
        m[rows, L + b * Wn: L + (b + 1) * Wn] = mb[:, L:]
    return m


def _masked_softmax_attend(qrot, keys, vals, mask_row, scale):
    """softmax(scale * keys @ q) over allowed keys, times vals (fp64)."""
    s = (keys @ qrot) * scale
    s = np.where(mask_row, s, -np.inf)
    m = np.max(s)
    w = np.where(mask_row, np.exp(s - m), 0.0)
    return (w @ vals) / np.sum(w)


def tree_attention_branch(trunk_k, trunk_v, q, k, v, anchor, parent, pos,
                          rope_base=10000.0, scale=None):
    """Outputs [Wn][Hq][D] of one branch.

    trunk_k, trunk_v: [L][Hkv][D] (keys already rotated);
    q: [Wn][Hq][D]; k, v: [Wn][Hkv][D] (q, k unrotated)."""
    trunk_k = np.asarray(trunk_k, np.float64)
    trunk_v = np.asarray(trunk_v, np.float64)
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    L, Hkv, D = trunk_k.shape
    Wn, Hq, _ = q.shape
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    if scale is None or scale == 0:
        scale = 1.0 / np.sqrt(D)
    if not (0 <= int(anchor) < L):
        raise ValueError("anchor outside the trunk")
    pos = np.asarray(pos, np.int64)
    check_positions(anchor, parent, pos)
    mask = branch_mask(L, int(anchor), parent)
    qrot = rope(q, pos[:, None], rope_base)          # [Wn][Hq][D]
    krot = rope(k, pos[:, None], rope_base)          # [Wn][Hkv][D]
    out = np.zeros((Wn, Hq, D))
    for g in range(Hkv):
        keys = np.concatenate([trunk_k[:, g, :], krot[:, g, :]], axis=0)
        vals = np.concatenate([trunk_v[:, g, :], v[:, g, :]], axis=0)
        for h in range(g * G, (g + 1) * G):
            for j in range(Wn):
                out[j, h] = _masked_softmax_attend(qrot[j, h], keys, vals, mask[j], scale)
    return out


def tree_attention(trunk_k, trunk_v, q, k, v, anchors, parent, pos,
                   rope_base=10000.0, scale=None, branches=None):
    """Outputs [T][B][Wn][Hq][D], one branch at a time.

    ``branches``: optional list of (t, b) to compute; other entries stay 0.
    Inputs may be numpy arrays or CPU torch tensors (bf16 is widened exactly)."""
    a = [_np(x) for x in (trunk_k, trunk_v, q, k, v)]
    anchors, parent, pos = (_np(x).astype(np.int64) for x in (anchors, parent, pos))
    T, B, Wn, Hq, D = a[2].shape
    out = np.zeros((T, B, Wn, Hq, D))
    todo = branches if branches is not None else [(t, b) for t in range(T) for b in range(B)]
    for (t, b) in todo:
        out[t, b] = tree_attention_branch(a[0][t], a[1][t], a[2][t, b], a[3][t, b], a[4][t, b],
                                          anchors[t, b], parent[t, b], pos[t, b], rope_base, scale)
    return out


def tree_attention_packed(trunk_k, trunk_v, q, k, v, anchors, parent, pos,
                          rope_base=10000.0, scale=None):
    """Same outputs for one trunk, computed the way the pages draw it: every
    branch row of the packed batch against ALL keys (trunk plus every branch's
    nodes) under the packed Eq. 5 mask.  For small inputs; shows that the
    per-branch form loses nothing.

    trunk_k/v: [L][Hkv][D]; q: [B][Wn][Hq][D]; k, v: [B][Wn][Hkv][D]."""
    trunk_k, trunk_v, q, k, v = (_np(x) for x in (trunk_k, trunk_v, q, k, v))
    anchors, parent, pos = (_np(x).astype(np.int64) for x in (anchors, parent, pos))
    L, Hkv, D = trunk_k.shape
    B, Wn, Hq, _ = q.shape
    G = Hq // Hkv
    if scale is None or scale == 0:
        scale = 1.0 / np.sqrt(D)
    for b in range(B):
        check_positions(anchors[b], parent[b], pos[b])
    mask = packed_tree_mask(L, anchors, parent)
    qrot = rope(q, pos[:, :, None], rope_base).reshape(B * Wn, Hq, D)
    krot = rope(k, pos[:, :, None], rope_base).reshape(B * Wn, Hkv, D)
    vv = v.reshape(B * Wn, Hkv, D)
    out = np.zeros((B * Wn, Hq, D))
    for h in range(Hq):
        g = h // G
        keys = np.concatenate([trunk_k[:, g], krot[:, g]], axis=0)
        vals = np.concatenate([trunk_v[:, g], vv[:, g]], axis=0)
        for r in range(B * Wn):
            out[r, h] = _masked_softmax_attend(qrot[r, h], keys, vals, mask[r], scale)
    return out.reshape(B, Wn, Hq, D)


def _np(x):
    if hasattr(x, "detach"):
        x = x.detach().cpu()
        if x.is_floating_point():
            x = x.double()
        return x.numpy()
    return np.asarray(x)
