"""Rotary position embedding at a token's logical position (oracle, fp64).

[R] §3.2(a): rotary embeddings are applied at each token's logical position,
not at its index in the packed batch.  [S] §2.1: a branch node's semantic
position is the anchor position plus the node's offset.

Reading (the pages do not print the rotary formula): the common
"rotate-half" pairing, where coordinate i is rotated together with
coordinate i + D/2 by the angle pos * theta_i, theta_i = base^(-2i/D),
base 10000.  Written out for one pair (x_i, x_{i+D/2}):
    x_i'       = x_i cos(pos theta_i) - x_{i+D/2} sin(pos theta_i)
    x_{i+D/2}' = x_{i+D/2} cos(pos theta_i) + x_i sin(pos theta_i)
"""

from __future__ import annotations

import numpy as np


def rope_angles(pos, D: int, base: float = 10000.0):
    """cos and sin of pos * theta_i, shape pos.shape + (D/2,), fp64."""
    pos = np.asarray(pos, dtype=np.float64)
    i = np.arange(D // 2, dtype=np.float64)
    theta = np.power(np.float64(base), -2.0 * i / D)
    ang = pos[..., None] * theta
    return np.cos(ang), np.sin(ang)


def rope(x, pos, base: float = 10000.0):
    """Rotate the last axis of x (size D, even) at positions ``pos``.

    ``pos`` broadcasts against x.shape[:-1]."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    assert D % 2 == 0
    h = D // 2
    c, s = rope_angles(pos, D, base)
    c = np.broadcast_to(c, x.shape[:-1] + (h,))
    s = np.broadcast_to(s, x.shape[:-1] + (h,))
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)
