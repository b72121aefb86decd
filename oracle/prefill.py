"""Trunk prefill (oracle, fp64) — TEST INFRASTRUCTURE.

What the pages fix:
  * [R] §3.1 step 1: the target's context features up to every anchor come
    from one pass over the reference trajectory (the trunk);
  * [R] §3.2(a) and [S] §2.2: that pass is done once, its keys and values are
    cached, and every branch attaches to the cache;
  * [R] §3.2 "numerical consistency" (Table 4): recomputing a full prefix,
    scoring branches one at a time or in a batch from the cache, and the
    merged tree must give the same signal for the same history.

Readings where the pages are silent (the same as for branch rows):
  * the trunk pass is causal self-attention: token s attends to tokens 0..s;
  * rotary embedding at the trunk positions 0..L-1 (oracle.rope's
    rotate-half pairing); the cache holds the rotated keys and the values as
    given;
  * scores scaled by 1/sqrt(D); query head h reads kv head floor(h/G).
"""

from __future__ import annotations

import numpy as np

from .rope import rope


def trunk_prefill_cache(k, v, rope_base=10000.0):
    """The KV cache a trunk pass leaves: keys rotated at 0..L-1, values as given.

    k, v: [L][Hkv][D]."""
    k = np.asarray(k, np.float64)
    L = k.shape[0]
    return rope(k, np.arange(L)[:, None], rope_base), np.asarray(v, np.float64).copy()


def trunk_prefill(q, k, v, rope_base=10000.0, scale=None, rows=None):
    """Causal GQA attention of the trunk over itself.

    q: [L][Hq][D], k, v: [L][Hkv][D], all unrotated.  Returns (out, cache_k,
    cache_v): out [L][Hq][D] (only ``rows`` filled when given, else every
    row), cache_k / cache_v [L][Hkv][D]."""
    q = np.asarray(q, np.float64)
    L, Hq, D = q.shape
    ck, cv = trunk_prefill_cache(k, v, rope_base)
    Hkv = ck.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    if scale is None or scale == 0:
        scale = 1.0 / np.sqrt(D)
    qrot = rope(q, np.arange(L)[:, None], rope_base)
    todo = np.arange(L) if rows is None else np.asarray(rows, np.int64)
    out = np.zeros((L, Hq, D))
    for h in range(Hq):
        g = h // G
        # scores of the wanted rows against every key, keys after the row masked
        s = (qrot[todo, h] @ ck[:, g].T) * scale                  # [rows][L]
        s = np.where(np.arange(L)[None, :] <= todo[:, None], s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        w = np.exp(s)
        out[todo, h] = (w @ cv[:, g]) / w.sum(axis=1, keepdims=True)
    return out, ck, cv
