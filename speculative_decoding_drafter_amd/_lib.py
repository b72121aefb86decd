"""ctypes binding of libspecopd (include/specopd.h).

Argument marshalling only: every step of the computation runs in the HIP
library.  torch is used for device memory and the current stream.  If the
library has not been built this module raises at import; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_double, c_float, c_int, c_int32, c_size_t, c_uint32, c_void_p

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libspecopd.so")

SPECOPD_OK = 0
SPECOPD_ERR_INVALID_ARGUMENT = -1
SPECOPD_ERR_UNSUPPORTED = -2
SPECOPD_ERR_WORKSPACE = -3
SPECOPD_ERR_HIP = -4
SPECOPD_ERR_DEVICE_VALIDATION = -5

SPECOPD_F32 = 0
SPECOPD_BF16 = 1

SPECOPD_TREE_BATCH_INVARIANT = 1
SPECOPD_E2ETV_DEFER_ALL = 1
SPECOPD_GDN_CONV_L2NORM = 1

E2ETV_NOALLOC_SCRATCH_BYTES = 4 << 20  # SPECOPD_E2ETV_NOALLOC_SCRATCH_BYTES

# every symbol include/specopd.h declares
EXPORTS = (
    "specopd_tree_attn_workspace_size", "specopd_tree_attn_fwd", "specopd_tree_attn_device_status",
    "specopd_score_rows",
    "specopd_e2etv_workspace_size", "specopd_e2etv_fwd_bwd", "specopd_e2etv_device_status",
    "specopd_e2etv_fwd_bwd_noalloc",
    "specopd_prefill_workspace_size", "specopd_prefill_fwd",
    "specopd_gdn_workspace_size", "specopd_gdn_replay_fwd", "specopd_gdn_device_status",
    "specopd_gdn_conv_fwd",
    "specopd_qsa_trunk_groups_fwd", "specopd_qsa_workspace_size", "specopd_qsa_select_fwd",
    "specopd_qsa_device_status",
    "specopd_lmhead_e2etv_workspace_size", "specopd_lmhead_e2etv_fwd_bwd",
    "specopd_lmhead_e2etv_device_status",
    "specopd_kernel_timing", "specopd_kernel_time",
    "specopd_status_string", "specopd_version",
)


class TreeAttnDesc(ctypes.Structure):
    _fields_ = [("T", c_int32), ("L", c_int32), ("B", c_int32), ("Wn", c_int32),
                ("Hq", c_int32), ("Hkv", c_int32), ("D", c_int32), ("dtype", c_int),
                ("rope_base", c_float), ("scale", c_float), ("flags", c_uint32)]


class E2etvDesc(ctypes.Structure):
    _fields_ = [("R", c_int32), ("Wn", c_int32), ("V", c_int32), ("logits_dtype", c_int),
                ("grad_dtype", c_int), ("norm_count", c_double), ("grad_scale", c_float),
                ("flags", c_uint32), ("wait_polls", c_int32), ("target_rows", c_int32)]


class PrefillDesc(ctypes.Structure):
    _fields_ = [("T", c_int32), ("L", c_int32), ("Hq", c_int32), ("Hkv", c_int32), ("D", c_int32),
                ("dtype", c_int), ("rope_base", c_float), ("scale", c_float), ("flags", c_uint32)]


class GdnDesc(ctypes.Structure):
    _fields_ = [("T", c_int32), ("L", c_int32), ("B", c_int32), ("Wn", c_int32), ("H", c_int32),
                ("D", c_int32), ("C", c_int32), ("dtype", c_int), ("flags", c_uint32)]


class GdnConvDesc(ctypes.Structure):
    _fields_ = [("T", c_int32), ("L", c_int32), ("B", c_int32), ("Wn", c_int32), ("H", c_int32),
                ("D", c_int32), ("K", c_int32), ("dtype", c_int), ("flags", c_uint32)]


class QsaDesc(ctypes.Structure):
    _fields_ = [("T", c_int32), ("L", c_int32), ("B", c_int32), ("Wn", c_int32), ("Di", c_int32),
                ("topk", c_int32), ("rope_base", c_float), ("eps", c_float), ("flags", c_uint32)]


class LmHeadDesc(ctypes.Structure):
    _fields_ = [("R", c_int32), ("Wn", c_int32), ("V", c_int32), ("H", c_int32), ("M", c_int32),
                ("norm_count", c_double), ("grad_scale", c_float), ("flags", c_uint32)]


class SpecopdError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                          "(python speculative_decoding_drafter_amd/build.py)")
    lib = ctypes.CDLL(LIB_PATH)
    P = c_void_p
    lib.specopd_tree_attn_workspace_size.argtypes = [POINTER(TreeAttnDesc), POINTER(c_size_t)]
    lib.specopd_tree_attn_fwd.argtypes = [POINTER(TreeAttnDesc)] + [P] * 9 + [P, c_size_t, P]
    lib.specopd_tree_attn_device_status.argtypes = [POINTER(TreeAttnDesc), P, c_size_t,
                                                    POINTER(c_int32), P]
    lib.specopd_e2etv_workspace_size.argtypes = [POINTER(E2etvDesc), POINTER(c_size_t)]
    lib.specopd_e2etv_fwd_bwd.argtypes = [POINTER(E2etvDesc)] + [P] * 8 + [P, c_size_t, P]
    lib.specopd_e2etv_fwd_bwd_noalloc.argtypes = [POINTER(E2etvDesc)] + [P] * 8 + [P]
    lib.specopd_score_rows.argtypes = [POINTER(TreeAttnDesc), P, P, P, P]
    lib.specopd_e2etv_device_status.argtypes = [POINTER(E2etvDesc), P, c_size_t,
                                                POINTER(c_int32), POINTER(c_int32), P]
    lib.specopd_prefill_workspace_size.argtypes = [POINTER(PrefillDesc), POINTER(c_size_t)]
    lib.specopd_prefill_fwd.argtypes = [POINTER(PrefillDesc)] + [P] * 6 + [P, c_size_t, P]
    lib.specopd_gdn_workspace_size.argtypes = [POINTER(GdnDesc), POINTER(c_size_t)]
    lib.specopd_gdn_replay_fwd.argtypes = [POINTER(GdnDesc)] + [P] * 13 + [P, c_size_t, P]
    lib.specopd_gdn_device_status.argtypes = [POINTER(GdnDesc), P, c_size_t, POINTER(c_int32), P]
    lib.specopd_gdn_conv_fwd.argtypes = [POINTER(GdnConvDesc)] + [P] * 7
    lib.specopd_qsa_trunk_groups_fwd.argtypes = [POINTER(QsaDesc), P, P, P, P]
    lib.specopd_qsa_workspace_size.argtypes = [POINTER(QsaDesc), POINTER(c_size_t)]
    lib.specopd_qsa_select_fwd.argtypes = [POINTER(QsaDesc)] + [P] * 11 + [P, c_size_t, P]
    lib.specopd_qsa_device_status.argtypes = [POINTER(QsaDesc), P, c_size_t, POINTER(c_int32), P]
    lib.specopd_lmhead_e2etv_workspace_size.argtypes = [POINTER(LmHeadDesc), POINTER(c_size_t)]
    lib.specopd_lmhead_e2etv_fwd_bwd.argtypes = [POINTER(LmHeadDesc)] + [P] * 10 + [P, c_size_t, P]
    lib.specopd_lmhead_e2etv_device_status.argtypes = [POINTER(LmHeadDesc), P, c_size_t, POINTER(c_int32), P]
    lib.specopd_kernel_timing.argtypes = [c_int]
    lib.specopd_kernel_time.argtypes = [c_int, POINTER(c_double), POINTER(c_int)]
    lib.specopd_status_string.argtypes = [c_int]
    lib.specopd_status_string.restype = ctypes.c_char_p
    lib.specopd_version.argtypes = []
    for name in EXPORTS:
        if name not in ("specopd_status_string",):
            getattr(lib, name).restype = c_int if name != "specopd_version" else c_int
    return lib


LIB = _load()


def status_string(status: int) -> str:
    return LIB.specopd_status_string(int(status)).decode()


def specopd_version() -> int:
    return LIB.specopd_version()


def specopd_kernel_timing(enable: bool) -> None:
    """Start (or stop and discard) event recording around each call's main kernel."""
    st = LIB.specopd_kernel_timing(1 if enable else 0)
    if st != SPECOPD_OK:
        raise SpecopdError(st, "specopd_kernel_timing")


def specopd_kernel_time(which: int):
    """(total ms, launches) recorded for the attention (0), E2E-TV (1), prefill (2),
    GDN replay (3), GDN convolution (4), QSA scoring (5), QSA top-k (6) kernel, or the
    LM head + E2E-TV call's passes (7)."""
    ms, n = c_double(0.0), c_int(0)
    st = LIB.specopd_kernel_time(int(which), ctypes.byref(ms), ctypes.byref(n))
    if st != SPECOPD_OK:
        raise SpecopdError(st, "specopd_kernel_time")
    return ms.value, n.value


def _ptr(t):
    if t is None:
        return None
    return c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return c_void_p(int(stream))
    if torch.cuda.is_available():
        return c_void_p(torch.cuda.current_stream().cuda_stream)
    return c_void_p(None)


_DT = {torch.float32: SPECOPD_F32, torch.bfloat16: SPECOPD_BF16}


def tree_attn_desc(T, L, B, Wn, Hq, Hkv, D, dtype, rope_base=10000.0, scale=0.0, flags=0):
    return TreeAttnDesc(T, L, B, Wn, Hq, Hkv, D, _DT.get(dtype, dtype) if not isinstance(dtype, int) else dtype,
                        rope_base, scale, flags)


def e2etv_desc(R, Wn, V, logits_dtype, grad_dtype=torch.float32, norm_count=0.0, grad_scale=1.0,
               flags=0, wait_polls=0, target_rows=0):
    ld = _DT.get(logits_dtype, logits_dtype) if not isinstance(logits_dtype, int) else logits_dtype
    gd = _DT.get(grad_dtype, grad_dtype) if not isinstance(grad_dtype, int) else grad_dtype
    return E2etvDesc(R, Wn, V, ld, gd, norm_count, grad_scale, flags, wait_polls, target_rows)


def prefill_desc(T, L, Hq, Hkv, D, dtype, rope_base=10000.0, scale=0.0, flags=0):
    return PrefillDesc(T, L, Hq, Hkv, D, _DT.get(dtype, dtype) if not isinstance(dtype, int) else dtype,
                       rope_base, scale, flags)


def specopd_prefill_workspace_size(desc: PrefillDesc) -> int:
    n = c_size_t(0)
    st = LIB.specopd_prefill_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    if st != SPECOPD_OK:
        raise SpecopdError(st, "specopd_prefill_workspace_size")
    return n.value


def specopd_prefill_fwd(desc, q, k, v, cache_k, cache_v, out, workspace, stream=None, raw_status=False):
    st = LIB.specopd_prefill_fwd(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(cache_k), _ptr(cache_v), _ptr(out),
        _ptr(workspace),
        c_size_t(workspace.numel() * workspace.element_size() if workspace is not None else 0),
        _stream(stream))
    if raw_status:
        return st
    if st != SPECOPD_OK:
        raise SpecopdError(st, "specopd_prefill_fwd")
    return out


def specopd_tree_attn_workspace_size(desc: TreeAttnDesc) -> int:
    n = c_size_t(0)
    st = LIB.specopd_tree_attn_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    if st != SPECOPD_OK:
        raise SpecopdError(st, "specopd_tree_attn_workspace_size")
    return n.value


def specopd_e2etv_workspace_size(desc: E2etvDesc) -> int:
    n = c_size_t(0)
    st = LIB.specopd_e2etv_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    if st != SPECOPD_OK:
        raise SpecopdError(st, "specopd_e2etv_workspace_size")
    return n.value


def specopd_tree_attn_fwd(desc, trunk_k, trunk_v, q, k, v, anchors, parent, pos, out, workspace,
                          stream=None, raw_status=False):
    st = LIB.specopd_tree_attn_fwd(
        ctypes.byref(desc), _ptr(trunk_k), _ptr(trunk_v), _ptr(q), _ptr(k), _ptr(v), _ptr(anchors),
        _ptr(parent), _ptr(pos), _ptr(out), _ptr(workspace),
        c_size_t(workspace.numel() * workspace.element_size() if workspace is not None else 0),
        _stream(stream))
    if raw_status:
        return st
    if st != SPECOPD_OK:
        raise SpecopdError(st, "specopd_tree_attn_fwd")
    return out


def specopd_score_rows(desc, anchors, parent, rows, stream=None, raw_status=False):
    st = LIB.specopd_score_rows(ctypes.byref(desc), _ptr(anchors), _ptr(parent), _ptr(rows),
                                _stream(stream))
    if raw_status:
        return st
    if st != SPECOPD_OK:
        raise SpecopdError(st, "specopd_score_rows")
    return rows


def specopd_tree_attn_device_status(desc, workspace, stream=None) -> int:
    bad = c_int32(0)
    st = LIB.specopd_tree_attn_device_status(ctypes.byref(desc), _ptr(workspace),
                                             c_size_t(workspace.numel() * workspace.element_size()),
                                             ctypes.byref(bad), _stream(stream))
    if st not in (SPECOPD_OK, SPECOPD_ERR_DEVICE_VALIDATION):
        raise SpecopdError(st, "specopd_tree_attn_device_status")
    return bad.value


def specopd_e2etv_fwd_bwd(desc, draft, target, parent, alpha_out, prefix_out, loss_out, grad,
                          workspace, stream=None, raw_status=False, target_row=None):
    st = LIB.specopd_e2etv_fwd_bwd(
        ctypes.byref(desc), _ptr(draft), _ptr(target), _ptr(target_row), _ptr(parent), _ptr(alpha_out),
        _ptr(prefix_out), _ptr(loss_out), _ptr(grad), _ptr(workspace),
        c_size_t(workspace.numel() * workspace.element_size() if workspace is not None else 0),
        _stream(stream))
    if raw_status:
        return st
    if st != SPECOPD_OK:
        raise SpecopdError(st, "specopd_e2etv_fwd_bwd")


def specopd_e2etv_fwd_bwd_noalloc(desc, draft, target, parent, alpha_out, prefix_out, loss_out, grad,
                                  stream=None, raw_status=False, target_row=None):
    st = LIB.specopd_e2etv_fwd_bwd_noalloc(
        ctypes.byref(desc), _ptr(draft), _ptr(target), _ptr(target_row), _ptr(parent), _ptr(alpha_out),
        _ptr(prefix_out), _ptr(loss_out), _ptr(grad), _stream(stream))
    if raw_status:
        return st
    if st != SPECOPD_OK:
        raise SpecopdError(st, "specopd_e2etv_fwd_bwd_noalloc")


def specopd_e2etv_device_status(desc, workspace, stream=None, with_deferred=False):
    """Malformed branches of the last call on this workspace (and, with
    with_deferred, the rows that the follow-up kernel finished)."""
    bad, deferred = c_int32(0), c_int32(0)
    st = LIB.specopd_e2etv_device_status(ctypes.byref(desc), _ptr(workspace),
                                         c_size_t(workspace.numel() * workspace.element_size()),
                                         ctypes.byref(bad), ctypes.byref(deferred), _stream(stream))
    if st not in (SPECOPD_OK, SPECOPD_ERR_DEVICE_VALIDATION):
        raise SpecopdError(st, "specopd_e2etv_device_status")
    return (bad.value, deferred.value) if with_deferred else bad.value


# ------------------------------------------------------------------ helpers


def gdn_desc(T, L, B, Wn, H, D, C, dtype, flags=0):
    return GdnDesc(T, L, B, Wn, H, D, C, _DT.get(dtype, dtype) if not isinstance(dtype, int) else dtype, flags)


def specopd_gdn_workspace_size(desc: GdnDesc) -> int:
    n = c_size_t(0)
    st = LIB.specopd_gdn_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    if st != SPECOPD_OK:
        raise SpecopdError(st, "specopd_gdn_workspace_size")
    return n.value


def specopd_gdn_replay_fwd(desc, ckpt, trunk_k, trunk_v, trunk_gate, trunk_beta, anchors, parent, q, k, v,
                           gate, beta, out, workspace, stream=None, raw_status=False):
    st = LIB.specopd_gdn_replay_fwd(
        ctypes.byref(desc), _ptr(ckpt), _ptr(trunk_k), _ptr(trunk_v), _ptr(trunk_gate), _ptr(trunk_beta),
        _ptr(anchors), _ptr(parent), _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta), _ptr(out),
        _ptr(workspace),
        c_size_t(workspace.numel() * workspace.element_size() if workspace is not None else 0),
        _stream(stream))
    if raw_status:
        return st
    if st != SPECOPD_OK:
        raise SpecopdError(st, "specopd_gdn_replay_fwd")
    return out


def specopd_gdn_device_status(desc, workspace, stream=None) -> int:
    bad = c_int32(0)
    st = LIB.specopd_gdn_device_status(ctypes.byref(desc), _ptr(workspace),
                                       c_size_t(workspace.numel() * workspace.element_size()),
                                       ctypes.byref(bad), _stream(stream))
    if st not in (SPECOPD_OK, SPECOPD_ERR_DEVICE_VALIDATION):
        raise SpecopdError(st, "specopd_gdn_device_status")
    return bad.value


def gdn_replay(inp: dict, C=64, ws=None, out=None):
    """GDN branch replay on generated inputs (dict of device tensors);
    returns (out [T][B][Wn][H][D] fp32, desc, ws)."""
    q = inp["q"]
    T, B, Wn, H, D = q.shape
    L = inp["trunk_k"].shape[1]
    desc = gdn_desc(T, L, B, Wn, H, D, C, q.dtype)
    if ws is None:
        ws = workspace(specopd_gdn_workspace_size(desc), q.device)
    if out is None:
        out = torch.empty((T, B, Wn, H, D), dtype=torch.float32, device=q.device)
    specopd_gdn_replay_fwd(desc, inp["ckpt"] if L // C > 0 else None, inp["trunk_k"], inp["trunk_v"],
                           inp["trunk_gate"], inp["trunk_beta"], inp["anchors"], inp["parent"], q, inp["k"],
                           inp["v"], inp["gate"], inp["beta"], out, ws)
    return out, desc, ws


def gdn_conv_desc(T, L, B, Wn, H, D, K, dtype, flags=0):
    return GdnConvDesc(T, L, B, Wn, H, D, K, _DT.get(dtype, dtype) if not isinstance(dtype, int) else dtype,
                       flags)


def specopd_gdn_conv_fwd(desc, trunk_x, x, w, anchors, parent, out, stream=None, raw_status=False):
    st = LIB.specopd_gdn_conv_fwd(ctypes.byref(desc), _ptr(trunk_x), _ptr(x), _ptr(w), _ptr(anchors),
                                  _ptr(parent), _ptr(out), _stream(stream))
    if raw_status:
        return st
    if st != SPECOPD_OK:
        raise SpecopdError(st, "specopd_gdn_conv_fwd")
    return out


def gdn_conv(trunk_x, x, w, anchors, parent, H, l2norm=False, out=None):
    """Short convolution of branch-node inputs x [T][B][Wn][H*D] along the
    parent map, trunk_x [T][L][H*D], w [H*D][K] fp32; returns (out, desc)."""
    T, B, Wn, C = x.shape
    desc = gdn_conv_desc(T, trunk_x.shape[1], B, Wn, H, C // H, w.shape[1], x.dtype,
                         SPECOPD_GDN_CONV_L2NORM if l2norm else 0)
    if out is None:
        out = torch.empty_like(x)
    specopd_gdn_conv_fwd(desc, trunk_x, x, w, anchors, parent, out)
    return out, desc


def qsa_desc(T, L, B, Wn, Di, topk, rope_base=10000.0, eps=0.0, flags=0):
    return QsaDesc(T, L, B, Wn, Di, topk, rope_base, eps, flags)


def specopd_qsa_trunk_groups_fwd(desc, trunk_raw, gamma, trunk_gk, stream=None, raw_status=False):
    st = LIB.specopd_qsa_trunk_groups_fwd(ctypes.byref(desc), _ptr(trunk_raw), _ptr(gamma), _ptr(trunk_gk),
                                          _stream(stream))
    if raw_status:
        return st
    if st != SPECOPD_OK:
        raise SpecopdError(st, "specopd_qsa_trunk_groups_fwd")
    return trunk_gk


def specopd_qsa_workspace_size(desc: QsaDesc) -> int:
    n = c_size_t(0)
    st = LIB.specopd_qsa_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    if st != SPECOPD_OK:
        raise SpecopdError(st, "specopd_qsa_workspace_size")
    return n.value


def specopd_qsa_select_fwd(desc, trunk_gk, trunk_raw, x, y, gamma, anchors, parent, pos, sel, score, bkey,
                           ws, stream=None, raw_status=False):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    st = LIB.specopd_qsa_select_fwd(ctypes.byref(desc), _ptr(trunk_gk), _ptr(trunk_raw), _ptr(x), _ptr(y),
                                    _ptr(gamma), _ptr(anchors), _ptr(parent), _ptr(pos), _ptr(sel),
                                    _ptr(score), _ptr(bkey), _ptr(ws), c_size_t(nbytes), _stream(stream))
    if raw_status:
        return st
    if st != SPECOPD_OK:
        raise SpecopdError(st, "specopd_qsa_select_fwd")
    return sel, score


def specopd_qsa_device_status(desc, workspace, stream=None) -> int:
    bad = c_int32(0)
    st = LIB.specopd_qsa_device_status(ctypes.byref(desc), _ptr(workspace),
                                       c_size_t(workspace.numel() * workspace.element_size()),
                                       ctypes.byref(bad), _stream(stream))
    if st not in (SPECOPD_OK, SPECOPD_ERR_DEVICE_VALIDATION):
        raise SpecopdError(st, "specopd_qsa_device_status")
    return bad.value


def qsa_trunk_groups(trunk_raw, gamma, rope_base=10000.0, eps=0.0, out=None):
    """Group-key cache [T][L/4][Di] of trunk raw indexer keys trunk_raw
    [T][L][Di] (bf16), gain gamma [Di] fp32."""
    T, L, Di = trunk_raw.shape
    desc = qsa_desc(T, L, 1, 1, Di, 1, rope_base, eps)
    if out is None:
        out = torch.empty((T, L // 4, Di), dtype=trunk_raw.dtype, device=trunk_raw.device)
    specopd_qsa_trunk_groups_fwd(desc, trunk_raw, gamma, out)
    return out


def qsa_select(inp: dict, topk: int, rope_base=10000.0, eps=0.0, ws=None, outs=None, want_bkey=True):
    """Block selection of every branch node on generated inputs (dict of
    device tensors: trunk_gk, trunk_raw, x, y, gamma, anchors, parent, pos);
    returns dict(sel, score, bkey, desc, ws)."""
    x = inp["x"]
    T, B, Wn, Di = x.shape
    L = inp["trunk_raw"].shape[1]
    desc = qsa_desc(T, L, B, Wn, Di, topk, rope_base, eps)
    if ws is None:
        ws = workspace(specopd_qsa_workspace_size(desc), x.device)
    if outs is None:
        outs = {"sel": torch.empty((T, B, Wn, topk), dtype=torch.int32, device=x.device),
                "score": torch.empty((T, B, Wn, topk), dtype=torch.float32, device=x.device),
                "bkey": torch.empty_like(x) if want_bkey else None}
    specopd_qsa_select_fwd(desc, inp["trunk_gk"], inp["trunk_raw"], x, inp["y"], inp["gamma"],
                           inp["anchors"], inp["parent"], inp["pos"], outs["sel"], outs["score"],
                           outs.get("bkey"), ws)
    return dict(outs, desc=desc, ws=ws)


def lmhead_desc(R, Wn, V, H, M, norm_count=0.0, grad_scale=1.0, flags=0):
    return LmHeadDesc(R, Wn, V, H, M, norm_count, grad_scale, flags)


def specopd_lmhead_e2etv_workspace_size(desc: LmHeadDesc) -> int:
    n = c_size_t(0)
    st = LIB.specopd_lmhead_e2etv_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    if st != SPECOPD_OK:
        raise SpecopdError(st, "specopd_lmhead_e2etv_workspace_size")
    return n.value


def specopd_lmhead_e2etv_fwd_bwd(desc, h_draft, w_draft, h_target, w_target, target_row, parent, alpha,
                                 prefix, loss, grad, ws, stream=None, raw_status=False):
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    st = LIB.specopd_lmhead_e2etv_fwd_bwd(ctypes.byref(desc), _ptr(h_draft), _ptr(w_draft), _ptr(h_target),
                                          _ptr(w_target), _ptr(target_row), _ptr(parent), _ptr(alpha),
                                          _ptr(prefix), _ptr(loss), _ptr(grad), _ptr(ws), c_size_t(nbytes),
                                          _stream(stream))
    if raw_status:
        return st
    if st != SPECOPD_OK:
        raise SpecopdError(st, "specopd_lmhead_e2etv_fwd_bwd")
    return loss


def specopd_lmhead_e2etv_device_status(desc, workspace, stream=None) -> int:
    bad = c_int32(0)
    st = LIB.specopd_lmhead_e2etv_device_status(ctypes.byref(desc), _ptr(workspace),
                                                c_size_t(workspace.numel() * workspace.element_size()),
                                                ctypes.byref(bad), _stream(stream))
    if st not in (SPECOPD_OK, SPECOPD_ERR_DEVICE_VALIDATION):
        raise SpecopdError(st, "specopd_lmhead_e2etv_device_status")
    return bad.value


def lmhead_e2etv(inp: dict, grad=True, norm_count=0.0, grad_scale=1.0, ws=None, outs=None):
    """LM head + E2E-TV on generated inputs (dict of device tensors h_draft,
    w_draft, h_target, w_target, target_row, parent); returns dict(alpha,
    prefix, loss (double[3]), grad or None, desc, ws)."""
    hd = inp["h_draft"]
    R, Wn, H = hd.shape
    V = inp["w_draft"].shape[0]
    desc = lmhead_desc(R, Wn, V, H, inp["h_target"].shape[0], norm_count, grad_scale)
    if ws is None:
        ws = workspace(specopd_lmhead_e2etv_workspace_size(desc), hd.device)
    if outs is None:
        outs = {"alpha": torch.empty((R, Wn), dtype=torch.float32, device=hd.device),
                "prefix": torch.empty((R, Wn), dtype=torch.float32, device=hd.device),
                "loss": torch.zeros(4, dtype=torch.float64, device=hd.device),
                "grad": torch.empty((R, Wn, V), dtype=torch.float32, device=hd.device) if grad else None}
    specopd_lmhead_e2etv_fwd_bwd(desc, hd, inp["w_draft"], inp["h_target"], inp["w_target"], inp["target_row"],
                                 inp["parent"], outs["alpha"], outs["prefix"], outs["loss"], outs.get("grad"), ws)
    return dict(outs, desc=desc, ws=ws)


def workspace(nbytes: int, device) -> torch.Tensor:
    """A 256-byte aligned uint8 device buffer of at least nbytes."""
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def score_rows(anchors, parent, L):
    """Score row of every branch node ([T][B][Wn] int32) for anchors [T][B]
    and parent [T][B][Wn] on a trunk of length L (specopd_score_rows)."""
    T, B, Wn = parent.shape
    desc = tree_attn_desc(T, L, B, Wn, 1, 1, 64, SPECOPD_BF16)
    rows = torch.empty((T, B, Wn), dtype=torch.int32, device=parent.device)
    specopd_score_rows(desc, anchors, parent, rows)
    return rows


def tree_attn(inp: dict, rope_base=10000.0, scale=0.0, ws=None, out=None, flags=0):
    """Tree attention on generated inputs (dict of device tensors)."""
    q = inp["q"]
    T, B, Wn, Hq, D = q.shape
    L, Hkv = inp["trunk_k"].shape[1], inp["trunk_k"].shape[2]
    desc = tree_attn_desc(T, L, B, Wn, Hq, Hkv, D, q.dtype, rope_base, scale, flags)
    if ws is None:
        ws = workspace(specopd_tree_attn_workspace_size(desc), q.device)
    if out is None:
        out = torch.empty_like(q)
    specopd_tree_attn_fwd(desc, inp["trunk_k"], inp["trunk_v"], q, inp["k"], inp["v"],
                          inp["anchors"], inp["parent"], inp["pos"], out, ws)
    return out, desc, ws


def prefill(q, k, v, rope_base=10000.0, scale=0.0, ws=None, outs=None):
    """Trunk prefill of q [T][L][Hq][D], k, v [T][L][Hkv][D] (device tensors);
    returns (out, cache_k, cache_v, desc, ws)."""
    T, L, Hq, D = q.shape
    Hkv = k.shape[2]
    desc = prefill_desc(T, L, Hq, Hkv, D, q.dtype, rope_base, scale)
    if ws is None:
        ws = workspace(specopd_prefill_workspace_size(desc), q.device)
    if outs is None:
        outs = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    out, ck, cv = outs
    specopd_prefill_fwd(desc, q, k, v, ck, cv, out, ws)
    return out, ck, cv, desc, ws


def e2etv(draft, target, parent, grad=True, grad_dtype=torch.float32, norm_count=0.0,
          grad_scale=1.0, ws=None, outs=None, wait_polls=0, target_row=None, flags=0):
    """E2E-TV forward + gradient; returns dict of device tensors.  With
    target_row ([R][Wn] int32), target is a matrix of score rows [rows][V]
    and node n's target distribution is row target_row[n] of it."""
    R, Wn, V = draft.shape
    dev = draft.device
    desc = e2etv_desc(R, Wn, V, draft.dtype, grad_dtype, norm_count, grad_scale,
                      flags=flags, wait_polls=wait_polls,
                      target_rows=target.numel() // V if target_row is not None else 0)
    if ws is None:
        ws = workspace(specopd_e2etv_workspace_size(desc), dev)
    if outs is None:
        outs = {
            "alpha": torch.empty((R, Wn), dtype=torch.float32, device=dev),
            "prefix": torch.empty((R, Wn), dtype=torch.float32, device=dev),
            "loss": torch.empty(3, dtype=torch.float64, device=dev),
            "grad": torch.empty((R, Wn, V), dtype=grad_dtype, device=dev) if grad else None,
        }
    specopd_e2etv_fwd_bwd(desc, draft, target, parent, outs["alpha"], outs["prefix"], outs["loss"],
                          outs["grad"], ws, target_row=target_row)
    outs["desc"] = desc
    outs["ws"] = ws
    return outs
