"""Seeded synthetic inputs for tree attention and the E2E-TV loss.

The generator only draws numbers and lays them out; it performs none of the
scoring method's arithmetic.  Tensors are drawn with ``torch`` on the device
they are requested on (CPU for oracle-only tests, ``cuda`` for GPU runs, where
multi-GB logits would be slow to draw on the host).  The same (config, seed,
device) always yields the same bytes; a GPU parity test that needs oracle
values copies the generated inputs to the host, so both sides see identical
bytes.

Distributions (the workload descriptions give sizes and value laws, no data):
  * trunk K/V, branch q/k/v: i.i.d. N(0, 1), rounded to the workload dtype.
    The trunk key cache is taken to hold keys already rotated at their trunk
    positions; an i.i.d. isotropic Gaussian is invariant under the pairwise
    rotations, so drawing it directly is distributionally identical to
    rotating raw N(0, 1) keys.
  * anchors: per trunk, B distinct positions drawn uniformly without
    replacement from the response part [P, L-1), left unsorted.
  * parent map / semantic positions: the config's literal tree shape;
    pos = anchor + 1 + depth.
  * logits: see ``LossConfig.recipe``.
bf16 values are round-to-nearest-even conversions of fp32 draws.
"""

from __future__ import annotations

from typing import Dict

import numpy as np
import torch

from .configs import AttnConfig, GdnConfig, LmHeadConfig, LossConfig, QsaConfig

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}

# tensor ids for seed derivation
_T_TRUNK_K, _T_TRUNK_V, _T_Q, _T_K, _T_V, _T_ANCH = 1, 2, 3, 4, 5, 6
_T_DRAFT, _T_TARGET, _T_PERM, _T_PEAK = 11, 12, 13, 14
_T_PF_Q, _T_PF_K, _T_PF_V = 21, 22, 23
_T_G_CKPT, _T_G_TK, _T_G_TV, _T_G_TA, _T_G_TB = 31, 32, 33, 34, 35
_T_G_Q, _T_G_K, _T_G_V, _T_G_A, _T_G_B = 36, 37, 38, 39, 40
_T_G_CX, _T_G_CTX, _T_G_CW = 41, 42, 43
_T_Q_TRAW, _T_Q_TGK, _T_Q_X, _T_Q_Y, _T_Q_GAMMA = 51, 52, 53, 54, 55
_T_L_HD, _T_L_HT, _T_L_WD, _T_L_WT = 61, 62, 63, 64


def derive_seed(seed: int, cid: int, tensor: int) -> int:
    """63-bit seed for one tensor of one workload."""
    st = np.random.SeedSequence([seed, cid, tensor]).generate_state(2, dtype=np.uint32)
    return int((int(st[0]) << 31) ^ int(st[1])) & ((1 << 63) - 1)


def _gen(device, seed: int, cid: int, tensor: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(derive_seed(seed, cid, tensor))
    return g


def _normal(shape, dtype, device, g, chunk_rows: int = 0) -> torch.Tensor:
    """N(0,1) draws in fp32, rounded to dtype; drawn in row chunks along dim 0
    so huge tensors never need an fp32 copy of themselves."""
    out = torch.empty(shape, dtype=dtype, device=device)
    if chunk_rows <= 0 or shape[0] <= chunk_rows:
        out.copy_(torch.randn(shape, generator=g, device=device, dtype=torch.float32))
        return out
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        sub = (r1 - r0,) + tuple(shape[1:])
        out[r0:r1].copy_(torch.randn(sub, generator=g, device=device, dtype=torch.float32))
    return out


def anchors_for(cfg: AttnConfig, seed: int, cid: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(derive_seed(seed, cid, _T_ANCH)))
    a = np.empty((cfg.T, cfg.B), dtype=np.int32)
    for t in range(cfg.T):
        a[t] = rng.choice(np.arange(cfg.P, cfg.L - 1), size=cfg.B, replace=False)
    return a


def gen_attn(cfg: AttnConfig, seed: int = 0, device="cpu", cid: int = 0) -> Dict[str, torch.Tensor]:
    """Tree-attention inputs.

    Layouts (row-major): trunk_k/trunk_v [T][L][Hkv][D]; q [T][B][Wn][Hq][D];
    k/v [T][B][Wn][Hkv][D]; anchors [T][B]; parent/pos [T][B][Wn] (int32).
    """
    dt = _DT[cfg.dtype]
    T, L, B, Wn, Hq, Hkv, D = cfg.T, cfg.L, cfg.B, cfg.Wn, cfg.Hq, cfg.Hkv, cfg.D
    out = {
        "trunk_k": _normal((T * L, Hkv, D), dt, device, _gen(device, seed, cid, _T_TRUNK_K), 8192).view(T, L, Hkv, D),
        "trunk_v": _normal((T * L, Hkv, D), dt, device, _gen(device, seed, cid, _T_TRUNK_V), 8192).view(T, L, Hkv, D),
        "q": _normal((T, B, Wn, Hq, D), dt, device, _gen(device, seed, cid, _T_Q)),
        "k": _normal((T, B, Wn, Hkv, D), dt, device, _gen(device, seed, cid, _T_K)),
        "v": _normal((T, B, Wn, Hkv, D), dt, device, _gen(device, seed, cid, _T_V)),
    }
    anch = anchors_for(cfg, seed, cid)
    parent = np.broadcast_to(np.asarray(cfg.parent, np.int32), (T, B, Wn)).copy()
    pos = (anch[:, :, None] + 1 + np.asarray(cfg.depth, np.int32)[None, None, :]).astype(np.int32)
    out["anchors"] = torch.from_numpy(anch).to(device)
    out["parent"] = torch.from_numpy(parent).to(device)
    out["pos"] = torch.from_numpy(pos).to(device)
    return out


def gen_prefill(cfg: AttnConfig, seed: int = 0, device="cpu", cid: int = 0) -> Dict[str, torch.Tensor]:
    """Trunk-prefill inputs of a workload's trunks: q [T][L][Hq][D] and k, v
    [T][L][Hkv][D], i.i.d. N(0, 1) rounded to the workload dtype, keys NOT
    rotated (the prefill rotates them)."""
    dt = _DT[cfg.dtype]
    T, L, Hq, Hkv, D = cfg.T, cfg.L, cfg.Hq, cfg.Hkv, cfg.D
    return {
        "q": _normal((T * L, Hq, D), dt, device, _gen(device, seed, cid, _T_PF_Q), 8192).view(T, L, Hq, D),
        "k": _normal((T * L, Hkv, D), dt, device, _gen(device, seed, cid, _T_PF_K), 8192).view(T, L, Hkv, D),
        "v": _normal((T * L, Hkv, D), dt, device, _gen(device, seed, cid, _T_PF_V), 8192).view(T, L, Hkv, D),
    }


def stress_classes(cfg: LossConfig, seed: int, cid: int) -> np.ndarray:
    """Row classes for the "stress" recipe: 0 identical, 1 disjoint, 2 noise."""
    N = cfg.N
    rng = np.random.Generator(np.random.PCG64(derive_seed(seed, cid, _T_PERM)))
    perm = rng.permutation(N)
    cls = np.full(N, 2, dtype=np.int8)
    cls[perm[: N // 2]] = 0
    cls[perm[N // 2: N // 2 + N // 4]] = 1
    return cls


def gen_loss(cfg: LossConfig, seed: int = 0, device="cpu", cid: int = 0,
             chunk_rows: int = 256) -> Dict[str, torch.Tensor]:
    """E2E-TV inputs: draft/target logits [R][Wn][V] and parent [R][Wn].

    Row n = r*Wn + j holds the drafter's (draft) and the target's (target)
    next-token logits for node j of branch r."""
    dt = _DT[cfg.dtype]
    N, V = cfg.N, cfg.V
    gz = _gen(device, seed, cid, _T_DRAFT)
    gt = _gen(device, seed, cid, _T_TARGET)
    draft = torch.empty((N, V), dtype=dt, device=device)
    target = torch.empty((N, V), dtype=dt, device=device)
    cls = stress_classes(cfg, seed, cid) if cfg.recipe == "stress" else None
    peaks = None
    if cls is not None:
        rng = np.random.Generator(np.random.PCG64(derive_seed(seed, cid, _T_PEAK)))
        a = rng.integers(0, V, size=N)
        b = (a + 1 + rng.integers(0, V - 1, size=N)) % V  # b != a
        peaks = (a, b)
    for r0 in range(0, N, chunk_rows):
        r1 = min(N, r0 + chunk_rows)
        n = r1 - r0
        e1 = torch.randn((n, V), generator=gz, device=device, dtype=torch.float32)
        e2 = torch.randn((n, V), generator=gt, device=device, dtype=torch.float32)
        if cfg.recipe == "indep":
            z, t = cfg.sd * e1, cfg.sd * e2
        elif cfg.recipe == "noise":
            z, t = e1, e1 + e2
        elif cfg.recipe == "rho":
            z = cfg.sd * e1
            t = cfg.rho * z + cfg.sd * float(np.sqrt(1.0 - cfg.rho ** 2)) * e2
        elif cfg.recipe == "stress":
            z, t = e1, e1 + e2
            c = torch.from_numpy(cls[r0:r1]).to(device)
            dis = torch.nonzero(c == 1).flatten()
            if dis.numel():
                t[dis] = e2[dis]
                ia = torch.from_numpy(peaks[0][r0:r1]).to(device)[dis]
                ib = torch.from_numpy(peaks[1][r0:r1]).to(device)[dis]
                z[dis, ia] += cfg.peak
                t[dis, ib] += cfg.peak
        else:
            raise ValueError(cfg.recipe)
        draft[r0:r1] = z.to(dt)
        target[r0:r1] = t.to(dt)
        if cls is not None:
            same = torch.nonzero(torch.from_numpy(cls[r0:r1]).to(device) == 0).flatten()
            if same.numel():
                target[r0 + same] = draft[r0 + same]
    parent = np.broadcast_to(np.asarray(cfg.parent, np.int32), (cfg.R, cfg.Wn)).copy()
    return {
        "draft": draft.view(cfg.R, cfg.Wn, V),
        "target": target.view(cfg.R, cfg.Wn, V),
        "parent": torch.from_numpy(parent).to(device),
    }


def _unit_rows(shape, dtype, device, g, chunk_rows: int = 0) -> torch.Tensor:
    """Vectors along the last dim uniform on the unit sphere: Gaussian draws
    scaled to unit length in fp32, then rounded to dtype."""
    out = torch.empty(shape, dtype=dtype, device=device)
    step = shape[0] if chunk_rows <= 0 else chunk_rows
    for r0 in range(0, shape[0], step):
        r1 = min(shape[0], r0 + step)
        x = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=g, device=device, dtype=torch.float32)
        out[r0:r1].copy_(x / torch.linalg.vector_norm(x, dim=-1, keepdim=True))
    return out


def _uniform(shape, lo: float, hi: float, device, g) -> torch.Tensor:
    return lo + (hi - lo) * torch.rand(shape, generator=g, device=device, dtype=torch.float32)


def gen_gdn(cfg: GdnConfig, seed: int = 0, device="cpu", cid: int = 0) -> Dict[str, torch.Tensor]:
    """GDN branch-replay inputs.

    Layouts (row-major): ckpt [T][L/C][H][D][D] fp32 (state after trunk
    tokens (m+1)C - 1, rows = value dims, columns = key dims); trunk_k,
    trunk_v [T][L][H][D]; trunk_gate, trunk_beta [T][L][H] fp32; q, k, v
    [T][B][Wn][H][D]; gate, beta [T][B][Wn][H] fp32; anchors [T][B];
    parent [T][B][Wn] (int32).  Anchors as for tree attention."""
    dt = _DT[cfg.dtype]
    T, L, B, Wn, H, D, NC = cfg.T, cfg.L, cfg.B, cfg.Wn, cfg.H, cfg.D, cfg.NC
    g = lambda tid: _gen(device, seed, cid, tid)
    ck = torch.empty((T * NC * H, D, D), dtype=torch.float32, device=device)
    gc = g(_T_G_CKPT)
    for r0 in range(0, ck.shape[0], 256):
        r1 = min(ck.shape[0], r0 + 256)
        ck[r0:r1] = cfg.state_sd * torch.randn((r1 - r0, D, D), generator=gc, device=device, dtype=torch.float32)
    out = {
        "ckpt": ck.view(T, NC, H, D, D),
        "trunk_k": _unit_rows((T * L, H, D), dt, device, g(_T_G_TK), 8192).view(T, L, H, D),
        "trunk_v": _normal((T * L, H, D), dt, device, g(_T_G_TV), 8192).view(T, L, H, D),
        "trunk_gate": _uniform((T, L, H), cfg.gate_lo, 1.0, device, g(_T_G_TA)),
        "trunk_beta": _uniform((T, L, H), 0.05, 0.95, device, g(_T_G_TB)),
        "q": _normal((T, B, Wn, H, D), dt, device, g(_T_G_Q)),
        "k": _unit_rows((T, B, Wn, H, D), dt, device, g(_T_G_K)),
        "v": _normal((T, B, Wn, H, D), dt, device, g(_T_G_V)),
        "gate": _uniform((T, B, Wn, H), cfg.gate_lo, 1.0, device, g(_T_G_A)),
        "beta": _uniform((T, B, Wn, H), 0.05, 0.95, device, g(_T_G_B)),
    }
    anch = anchors_for(cfg, seed, cid)
    parent = np.broadcast_to(np.asarray(cfg.parent, np.int32), (T, B, Wn)).copy()
    out["anchors"] = torch.from_numpy(anch).to(device)
    out["parent"] = torch.from_numpy(parent).to(device)
    return out


def gen_gdn_conv(cfg: GdnConfig, seed: int = 0, device="cpu", cid: int = 0, K: int = 4) -> Dict[str, torch.Tensor]:
    """Inputs of the branch short convolution of one projection (q, k or v).

    trunk_x [T][L][H*D] and x [T][B][Wn][H*D]: N(0,1) projections before the
    convolution, in cfg.dtype; w [H*D][K] fp32 N(0, 1/K) weights; anchors and
    parent as gen_gdn draws them (the same seed gives the same tree)."""
    dt = _DT[cfg.dtype]
    T, L, B, Wn, C = cfg.T, cfg.L, cfg.B, cfg.Wn, cfg.H * cfg.D
    g = lambda tid: _gen(device, seed, cid, tid)
    w = torch.randn((C, K), generator=g(_T_G_CW), device=device, dtype=torch.float32) / float(np.sqrt(K))
    out = {
        "trunk_x": _normal((T * L, C), dt, device, g(_T_G_CTX), 8192).view(T, L, C),
        "x": _normal((T * B * Wn, C), dt, device, g(_T_G_CX), 8192).view(T, B, Wn, C),
        "w": w,
    }
    anch = anchors_for(cfg, seed, cid)
    parent = np.broadcast_to(np.asarray(cfg.parent, np.int32), (T, B, Wn)).copy()
    out["anchors"] = torch.from_numpy(anch).to(device)
    out["parent"] = torch.from_numpy(parent).to(device)
    return out


def gen_qsa(cfg: QsaConfig, seed: int = 0, device="cpu", cid: int = 0) -> Dict[str, torch.Tensor]:
    """QSA block-selection inputs.

    Layouts (row-major): trunk_raw [T][L][Di] and trunk_gk [T][L/4][Di]
    (bf16); x, y [T][B][Wn][Di] (bf16, the nodes' raw indexer keys and
    indexer queries); gamma [Di] fp32; anchors [T][B]; parent, pos
    [T][B][Wn] int32 (pos = anchor + 1 + depth).  trunk_gk is drawn, not
    computed from trunk_raw (see QsaConfig); a test that needs the two
    consistent replaces it."""
    dt = _DT[cfg.dtype]
    T, L, B, Wn, Di = cfg.T, cfg.L, cfg.B, cfg.Wn, cfg.Di
    g = lambda tid: _gen(device, seed, cid, tid)
    out = {
        "trunk_raw": _normal((T * L, Di), dt, device, g(_T_Q_TRAW), 65536).view(T, L, Di),
        "trunk_gk": _normal((T * (L // 4), Di), dt, device, g(_T_Q_TGK), 65536).view(T, L // 4, Di),
        "x": _normal((T * B * Wn, Di), dt, device, g(_T_Q_X), 65536).view(T, B, Wn, Di),
        "y": _normal((T * B * Wn, Di), dt, device, g(_T_Q_Y), 65536).view(T, B, Wn, Di),
        "gamma": 1.0 + 0.1 * torch.randn((Di,), generator=g(_T_Q_GAMMA), device=device, dtype=torch.float32),
    }
    anch = anchors_for(cfg, seed, cid)
    parent = np.broadcast_to(np.asarray(cfg.parent, np.int32), (T, B, Wn)).copy()
    depth = np.zeros(Wn, np.int64)
    for j, p in enumerate(cfg.parent):
        depth[j] = 0 if p < 0 else depth[p] + 1
    pos = (anch[:, :, None].astype(np.int64) + 1 + depth[None, None, :]).astype(np.int32)
    out["anchors"] = torch.from_numpy(anch).to(device)
    out["parent"] = torch.from_numpy(parent).to(device)
    out["pos"] = torch.from_numpy(np.ascontiguousarray(pos)).to(device)
    return out


def gen_lmhead(cfg: LmHeadConfig, seed: int = 0, device="cpu", cid: int = 0) -> Dict[str, torch.Tensor]:
    """Inputs of the LM head fused with E2E-TV.

    Layouts (row-major): h_draft [R][Wn][H]; h_target [L + R*Wn][H] (the
    trunk's score rows, then every branch node's); w_draft, w_target [V][H]
    (bf16); target_row [R][Wn] int32 (the parent's branch row L + r*Wn +
    parent, or the anchor's trunk row); parent [R][Wn]; anchors [R]."""
    dt = _DT[cfg.dtype]
    R, Wn, H, V, L = cfg.R, cfg.Wn, cfg.H, cfg.V, cfg.L
    g = lambda tid: _gen(device, seed, cid, tid)
    scale = cfg.sd / float(np.sqrt(H))

    def head(tid):
        w = torch.empty((V, H), dtype=dt, device=device)
        gw = g(tid)
        for r0 in range(0, V, 16384):
            r1 = min(V, r0 + 16384)
            w[r0:r1].copy_(scale * torch.randn((r1 - r0, H), generator=gw, device=device, dtype=torch.float32))
        return w

    out = {
        "h_draft": _normal((R * Wn, H), dt, device, g(_T_L_HD), 8192).view(R, Wn, H),
        "h_target": _normal((L + R * Wn, H), dt, device, g(_T_L_HT), 8192),
        "w_draft": head(_T_L_WD),
        "w_target": head(_T_L_WT),
    }
    anch = anchors_for(cfg, seed, cid)[0]
    par = np.asarray(cfg.parent, np.int64)
    rows = np.empty((R, Wn), np.int32)
    for r in range(R):
        for j in range(Wn):
            rows[r, j] = anch[r] if par[j] < 0 else L + r * Wn + par[j]
    out["target_row"] = torch.from_numpy(rows).to(device)
    out["parent"] = torch.from_numpy(np.broadcast_to(par.astype(np.int32), (R, Wn)).copy()).to(device)
    out["anchors"] = torch.from_numpy(anch.astype(np.int32)).to(device)
    return out
