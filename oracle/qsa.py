"""Sparse-attention (QSA) block selection with branch-consistent indexer
groups (oracle, fp64) — TEST INFRASTRUCTURE.

What the pages fix ([R] §3.2(b) and the Fig. 4 walk-through; [S] §1):
  * the sparse layer picks blocks of 4 consecutive tokens ("groups") by a
    compressed indexer key and reads the top-k of them;
  * a group's compressed key is the mean of its tokens' raw indexer keys,
    RMS-normalised, then rotated at the group's first position;
  * on a branch, groups completed before the anchor reuse the trunk's cached
    group keys unchanged; the incomplete group at the anchor (the boundary
    group) and every later group are compressed again from the branch's own
    history, so reference tokens after the anchor never enter a key; a branch
    keeps four raw indexer-key slots to fill the rest of its boundary group;
  * selection is separate from reading: attention reads the selected groups'
    K/V plus the incomplete causal tail, which bypasses the top-k.

Readings where the pages are silent (each a parameter or a stated choice):
  * one indexer head: every token has one raw indexer key x and one indexer
    query y of size Di; the selection is shared by the layer's heads;
  * RMSNorm(u) = u / sqrt(mean(u^2) + eps) * gamma with eps = 1e-6 and a
    learned gain gamma of size Di;
  * the rotation is the rotate-half convention of oracle.rope (base 10000);
    the query is rotated at its own position, so a score depends on the
    distance between the query and the group's first token;
  * the score of group g for a query at position p is the plain dot product
    <rope(y, p), key_g> (no scale: it would not change the order);
  * the candidates of a query at position p are the groups complete at p,
    g = 0 .. floor((p + 1) / 4) - 1 (4g + 3 <= p); the tokens of the group
    holding p that is not yet complete are the causal tail;
  * top-k keeps the k largest scores, ties going to the lower group index;
    with fewer than k candidates every candidate is kept; the kept groups
    are reported in increasing group order;
  * the trunk pass caches the key of every complete trunk group,
    floor(L / 4) of them.
The method is exact by construction: a branch row must select what the same
row selects in the plain sequence trunk[0..a] followed by its ancestor path,
with every group compressed from scratch.  ``plain_row_select`` is that
definition; ``qsa_branch_select`` is the cache-reusing form the pages
describe, and the tests hold the two equal.
"""

from __future__ import annotations

import numpy as np

from .rope import rope
from .tree_attention import check_positions, walk_ancestors

GROUP = 4  # tokens per indexer group ([R] §3.2(b))


def rms_norm(u, gamma, eps: float = 1e-6):
    """u / sqrt(mean(u^2) + eps) * gamma over the last axis (fp64)."""
    u = np.asarray(u, np.float64)
    ms = np.mean(u * u, axis=-1, keepdims=True)
    return u / np.sqrt(ms + eps) * np.asarray(gamma, np.float64)


def compress_group(raw, gamma, first_pos: int, base: float = 10000.0, eps: float = 1e-6):
    """Compressed key of one group from its 4 raw keys [4][Di]: mean pooling,
    RMSNorm, rotation at the group's first position."""
    raw = np.asarray(raw, np.float64)
    assert raw.shape[0] == GROUP
    return rope(rms_norm(raw.mean(axis=0), gamma, eps), first_pos, base)


def sequence_group_keys(raw, gamma, base: float = 10000.0, eps: float = 1e-6):
    """Keys of every complete group of a plain sequence of raw keys [n][Di]:
    [floor(n / 4)][Di].  The trunk pass's cache is this over a trunk."""
    raw = np.asarray(raw, np.float64)
    ng = raw.shape[0] // GROUP
    out = np.empty((ng, raw.shape[1]), np.float64)
    for g in range(ng):
        out[g] = compress_group(raw[GROUP * g:GROUP * g + GROUP], gamma, GROUP * g, base, eps)
    return out


def round_bf16(x):
    """Nearest bf16 value (ties to even), reached through fp32: the operand
    precision of a bf16 matrix-core kernel.  Finite inputs only."""
    f = np.asarray(x, np.float64).astype(np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


def select_topk(scores, k: int):
    """Indices of the k largest scores, ties to the lower index, returned in
    increasing index order (all indices when there are at most k)."""
    s = np.asarray(scores, np.float64)
    n = s.shape[0]
    if n <= k:
        return np.arange(n, dtype=np.int64)
    # sort by (-score, index): a stable sort on -score keeps lower indices first
    order = np.argsort(-s, kind="stable")
    return np.sort(order[:k])


def plain_row_select(seq_raw, y, gamma, k: int, base: float = 10000.0, eps: float = 1e-6):
    """Selection of the last token of a plain sequence (the definition).

    seq_raw [p+1][Di] holds the raw keys of positions 0..p, y the query of
    position p.  Returns (selected groups, their scores, every candidate's
    score)."""
    seq_raw = np.asarray(seq_raw, np.float64)
    p = seq_raw.shape[0] - 1
    keys = sequence_group_keys(seq_raw, gamma, base, eps)  # groups complete at p
    s = keys @ rope(np.asarray(y, np.float64), p, base) if keys.shape[0] else np.zeros(0)
    sel = select_topk(s, k)
    return sel, s[sel], s


def branch_group_keys(trunk_raw, x, anchor: int, parent, gamma, base: float = 10000.0,
                      eps: float = 1e-6):
    """Keys a branch compresses itself: node j completes group
    g = (pos_j - 3) / 4 when pos_j = anchor + 1 + depth_j is 3 mod 4; its key
    comes from the 4 tokens ending at j along j's own path -- j, its parent,
    ..., the anchor's child, then trunk tokens anchor, anchor - 1, ... (the
    boundary group's trunk part, held in the branch's raw reservation slots).

    Returns (keys [Wn][Di] with NaN rows for nodes completing no group,
    group index [Wn] with -1 for those nodes)."""
    trunk_raw = np.asarray(trunk_raw, np.float64)
    x = np.asarray(x, np.float64)
    Wn, Di = x.shape
    keys = np.full((Wn, Di), np.nan)
    gidx = np.full(Wn, -1, np.int64)
    for j in range(Wn):
        path = walk_ancestors(parent, j)  # j first, then its ancestors
        p = int(anchor) + len(path)       # semantic position of j
        if p % GROUP != GROUP - 1:
            continue
        toks = []
        for i in range(GROUP):            # positions p, p-1, p-2, p-3
            q = p - i
            if q > anchor:
                toks.append(x[path[i]])
            else:
                toks.append(trunk_raw[q])
        keys[j] = compress_group(np.stack(toks[::-1]), gamma, p - (GROUP - 1), base, eps)
        gidx[j] = (p - (GROUP - 1)) // GROUP
    return keys, gidx


def qsa_branch_select(trunk_gk, trunk_raw, x, y, anchor: int, parent, pos, gamma, k: int,
                      base: float = 10000.0, eps: float = 1e-6, operands: str = "f64"):
    """Block selection of every node of one branch, the cache-reusing way.

    trunk_gk [floor(L/4)][Di]: the trunk's cached group keys (used as given
    for groups complete at the anchor, g < floor((anchor + 1) / 4));
    trunk_raw [L][Di]: trunk raw keys (only the boundary group's trunk part
    is read); x, y [Wn][Di]: the nodes' raw keys and queries.

    operands="bf16" takes the selection in a bf16 kernel's precision: the
    rotated query and the keys the branch compresses are rounded to bf16
    before the (exact, fp64) dot products, so that a decision between two
    nearly equal scores is taken on the values such a kernel multiplies.

    Returns dict(sel [Wn][k] int64 (-1 padded), score [Wn][k] (-inf padded),
    ncand [Wn], scores list of every candidate's score per node, bkey,
    bgroup)."""
    check_positions(anchor, parent, pos)
    trunk_gk = np.asarray(trunk_gk, np.float64)
    y = np.asarray(y, np.float64)
    Wn = y.shape[0]
    rnd = round_bf16 if operands == "bf16" else (lambda v: v)
    bkey, bgroup = branch_group_keys(trunk_raw, x, anchor, parent, gamma, base, eps)
    bkey = np.where(np.isnan(bkey), np.nan, rnd(np.nan_to_num(bkey)))
    g_trunk = (int(anchor) + 1) // GROUP
    sel = np.full((Wn, k), -1, np.int64)
    sc = np.full((Wn, k), -np.inf)
    ncand = np.zeros(Wn, np.int64)
    all_scores = []
    for j in range(Wn):
        p = int(pos[j])
        G = (p + 1) // GROUP
        keys = np.empty((G, trunk_gk.shape[1]))
        keys[:min(G, g_trunk)] = trunk_gk[:min(G, g_trunk)]
        for i in walk_ancestors(parent, j):
            if bgroup[i] >= 0:
                keys[bgroup[i]] = bkey[i]
        s = keys @ rnd(rope(y[j], p, base)) if G else np.zeros(0)
        ss = select_topk(s, k)
        sel[j, :ss.shape[0]] = ss
        sc[j, :ss.shape[0]] = s[ss]
        ncand[j] = G
        all_scores.append(s)
    return {"sel": sel, "score": sc, "ncand": ncand, "scores": all_scores,
            "bkey": bkey, "bgroup": bgroup}


def qsa_select(trunk_gk, trunk_raw, x, y, anchors, parent, pos, gamma, k: int,
               base: float = 10000.0, eps: float = 1e-6, branches=None):
    """qsa_branch_select over [T][B] branches (or the listed (t, b) pairs).

    Shapes: trunk_gk [T][floor(L/4)][Di], trunk_raw [T][L][Di], x and y
    [T][B][Wn][Di], anchors [T][B], parent and pos [T][B][Wn]."""
    anchors = np.asarray(anchors)
    T, B = anchors.shape
    todo = branches if branches is not None else [(t, b) for t in range(T) for b in range(B)]
    return {(t, b): qsa_branch_select(trunk_gk[t], trunk_raw[t], x[t][b], y[t][b],
                                      int(anchors[t, b]), parent[t][b], pos[t][b], gamma, k,
                                      base, eps)
            for (t, b) in todo}


def causal_tail(anchor: int, parent, j: int):
    """Tokens of node j's incomplete group (read by attention without
    selection): trunk positions and branch nodes, oldest first, as
    ("trunk", s) / ("node", i).  Empty when j completes its group."""
    path = walk_ancestors(parent, j)
    p = int(anchor) + len(path)
    first = GROUP * ((p + 1) // GROUP)
    out = []
    for q in range(first, p + 1):
        out.append(("trunk", q) if q <= anchor else ("node", path[p - q]))
    return out
