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

# every symbol include/specopd.h declares
EXPORTS = (
    "specopd_tree_attn_workspace_size", "specopd_tree_attn_fwd", "specopd_tree_attn_device_status",
    "specopd_e2etv_workspace_size", "specopd_e2etv_fwd_bwd", "specopd_e2etv_device_status",
    "specopd_prefill_workspace_size", "specopd_prefill_fwd",
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
                ("flags", c_uint32)]


class PrefillDesc(ctypes.Structure):
    _fields_ = [("T", c_int32), ("L", c_int32), ("Hq", c_int32), ("Hkv", c_int32), ("D", c_int32),
                ("dtype", c_int), ("rope_base", c_float), ("scale", c_float), ("flags", c_uint32)]


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
    lib.specopd_e2etv_fwd_bwd.argtypes = [POINTER(E2etvDesc)] + [P] * 7 + [P, c_size_t, P]
    lib.specopd_e2etv_device_status.argtypes = [POINTER(E2etvDesc), P, c_size_t,
                                                POINTER(c_int32), P]
    lib.specopd_prefill_workspace_size.argtypes = [POINTER(PrefillDesc), POINTER(c_size_t)]
    lib.specopd_prefill_fwd.argtypes = [POINTER(PrefillDesc)] + [P] * 6 + [P, c_size_t, P]
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
    """(total ms, launches) recorded for the attention (0), E2E-TV (1) or prefill (2) kernel."""
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
               flags=0):
    ld = _DT.get(logits_dtype, logits_dtype) if not isinstance(logits_dtype, int) else logits_dtype
    gd = _DT.get(grad_dtype, grad_dtype) if not isinstance(grad_dtype, int) else grad_dtype
    return E2etvDesc(R, Wn, V, ld, gd, norm_count, grad_scale, flags)


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


def specopd_tree_attn_device_status(desc, workspace, stream=None) -> int:
    bad = c_int32(0)
    st = LIB.specopd_tree_attn_device_status(ctypes.byref(desc), _ptr(workspace),
                                             c_size_t(workspace.numel() * workspace.element_size()),
                                             ctypes.byref(bad), _stream(stream))
    if st not in (SPECOPD_OK, SPECOPD_ERR_DEVICE_VALIDATION):
        raise SpecopdError(st, "specopd_tree_attn_device_status")
    return bad.value


def specopd_e2etv_fwd_bwd(desc, draft, target, parent, alpha_out, prefix_out, loss_out, grad,
                          workspace, stream=None, raw_status=False):
    st = LIB.specopd_e2etv_fwd_bwd(
        ctypes.byref(desc), _ptr(draft), _ptr(target), _ptr(parent), _ptr(alpha_out),
        _ptr(prefix_out), _ptr(loss_out), _ptr(grad), _ptr(workspace),
        c_size_t(workspace.numel() * workspace.element_size() if workspace is not None else 0),
        _stream(stream))
    if raw_status:
        return st
    if st != SPECOPD_OK:
        raise SpecopdError(st, "specopd_e2etv_fwd_bwd")


def specopd_e2etv_device_status(desc, workspace, stream=None) -> int:
    bad = c_int32(0)
    st = LIB.specopd_e2etv_device_status(ctypes.byref(desc), _ptr(workspace),
                                         c_size_t(workspace.numel() * workspace.element_size()),
                                         ctypes.byref(bad), _stream(stream))
    if st not in (SPECOPD_OK, SPECOPD_ERR_DEVICE_VALIDATION):
        raise SpecopdError(st, "specopd_e2etv_device_status")
    return bad.value


# ------------------------------------------------------------------ helpers


def workspace(nbytes: int, device) -> torch.Tensor:
    """A 256-byte aligned uint8 device buffer of at least nbytes."""
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def tree_attn(inp: dict, rope_base=10000.0, scale=0.0, ws=None, out=None):
    """Tree attention on generated inputs (dict of device tensors)."""
    q = inp["q"]
    T, B, Wn, Hq, D = q.shape
    L, Hkv = inp["trunk_k"].shape[1], inp["trunk_k"].shape[2]
    desc = tree_attn_desc(T, L, B, Wn, Hq, Hkv, D, q.dtype, rope_base, scale)
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
          grad_scale=1.0, ws=None, outs=None):
    """E2E-TV forward + gradient; returns dict of device tensors."""
    R, Wn, V = draft.shape
    dev = draft.device
    desc = e2etv_desc(R, Wn, V, draft.dtype, grad_dtype, norm_count, grad_scale)
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
                          outs["grad"], ws)
    outs["desc"] = desc
    outs["ws"] = ws
    return outs
