"""The C ABI on a machine without a GPU: the library loads, exports every
function include/specopd.h declares, and rejects every host-detectable error
before touching the GPU (so these calls are safe here).  No compute call is
made: every call below carries at least one invalid argument."""

import ctypes
import os
import re

import pytest

import speculative_decoding_drafter_amd as sd
from speculative_decoding_drafter_amd import _lib

HDR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "specopd.h")

FAKE = 0x7f0000000000  # 16-byte aligned stand-in pointer, never dereferenced


def _declared():
    src = open(HDR).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(specopd_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert len(names) >= 8
    for n in names:
        assert hasattr(sd.LIB, n), n
        assert n in _lib.EXPORTS
    assert set(_lib.EXPORTS) == set(names)


def test_flag_constants_match_the_header():
    src = open(HDR).read()
    for name in ("SPECOPD_TREE_BATCH_INVARIANT", "SPECOPD_E2ETV_DEFER_ALL", "SPECOPD_GDN_CONV_L2NORM"):
        m = re.search(r"#define\s+" + name + r"\s+(\d+)u", src)
        assert m and int(m.group(1)) == getattr(sd, name), name


def test_version_and_status_strings():
    assert sd.specopd_version() == 2
    assert sd.status_string(0) == "ok"
    for s in (-1, -2, -3, -4, -5):
        assert sd.status_string(s) not in ("ok", "unknown status")


def _tdesc(**kw):
    base = dict(T=1, L=128, B=4, Wn=4, Hq=8, Hkv=2, D=128, dtype=sd.SPECOPD_BF16)
    base.update(kw)
    return sd.tree_attn_desc(**base)


def _tcall(desc, ws_bytes=1 << 30, **over):
    args = dict(trunk_k=FAKE, trunk_v=FAKE + 16, q=FAKE + 32, k=FAKE + 48, v=FAKE + 64,
                anchors=FAKE + 80, parent=FAKE + 96, pos=FAKE + 112, out=FAKE + 128,
                ws=FAKE + 144)
    args.update(over)
    P = ctypes.c_void_p
    return sd.LIB.specopd_tree_attn_fwd(
        ctypes.byref(desc), P(args["trunk_k"]), P(args["trunk_v"]), P(args["q"]), P(args["k"]),
        P(args["v"]), P(args["anchors"]), P(args["parent"]), P(args["pos"]), P(args["out"]),
        P(args["ws"]), ctypes.c_size_t(ws_bytes), P(None))


@pytest.mark.parametrize("field,value,code", [
    ("D", 96, sd.SPECOPD_ERR_UNSUPPORTED),
    ("D", 0, sd.SPECOPD_ERR_INVALID_ARGUMENT),
    ("Hq", 7, sd.SPECOPD_ERR_INVALID_ARGUMENT),     # Hq % Hkv != 0
    ("Wn", 65, sd.SPECOPD_ERR_UNSUPPORTED),
    ("Wn", 0, sd.SPECOPD_ERR_INVALID_ARGUMENT),
    ("L", 0, sd.SPECOPD_ERR_INVALID_ARGUMENT),
    ("B", -3, sd.SPECOPD_ERR_INVALID_ARGUMENT),
    ("dtype", 7, sd.SPECOPD_ERR_INVALID_ARGUMENT),
    ("flags", 2, sd.SPECOPD_ERR_INVALID_ARGUMENT),     # only SPECOPD_TREE_BATCH_INVARIANT is defined
    ("rope_base", float("nan"), sd.SPECOPD_ERR_INVALID_ARGUMENT),
    ("L", 20_000_000, sd.SPECOPD_ERR_UNSUPPORTED),  # one trunk's bf16 K beyond 4 GiB
    ("B", 3_000_000, sd.SPECOPD_ERR_UNSUPPORTED),   # one trunk's bf16 branch-node keys beyond 4 GiB
])
def test_tree_desc_errors(field, value, code):
    d = _tdesc()
    setattr(d, field, value)
    assert _tcall(d) == code
    n = ctypes.c_size_t(0)
    assert sd.LIB.specopd_tree_attn_workspace_size(ctypes.byref(d), ctypes.byref(n)) == code


@pytest.mark.parametrize("over,code", [
    (dict(q=0), sd.SPECOPD_ERR_INVALID_ARGUMENT),
    (dict(out=0), sd.SPECOPD_ERR_INVALID_ARGUMENT),
    (dict(anchors=FAKE + 4), sd.SPECOPD_ERR_INVALID_ARGUMENT),   # misaligned
    (dict(out=FAKE), sd.SPECOPD_ERR_INVALID_ARGUMENT),           # out aliases trunk_k
    (dict(ws=0), sd.SPECOPD_ERR_WORKSPACE),
    (dict(ws=FAKE + 152), sd.SPECOPD_ERR_WORKSPACE),             # misaligned workspace
])
def test_tree_pointer_errors(over, code):
    assert _tcall(_tdesc(), **over) == code


def test_tree_workspace_too_small():
    d = _tdesc()
    need = sd.specopd_tree_attn_workspace_size(d)
    assert need > 0
    assert _tcall(d, ws_bytes=need - 1) == sd.SPECOPD_ERR_WORKSPACE


def test_null_desc():
    n = ctypes.c_size_t(0)
    assert sd.LIB.specopd_tree_attn_workspace_size(None, ctypes.byref(n)) == sd.SPECOPD_ERR_INVALID_ARGUMENT
    assert sd.LIB.specopd_e2etv_workspace_size(None, ctypes.byref(n)) == sd.SPECOPD_ERR_INVALID_ARGUMENT


def _edesc(**kw):
    base = dict(R=4, Wn=7, V=151936, logits_dtype=sd.SPECOPD_BF16, grad_dtype=sd.SPECOPD_F32)
    base.update(kw)
    return sd.e2etv_desc(**base)


def _ecall(desc, ws_bytes=1 << 30, **over):
    args = dict(draft=FAKE, target=FAKE + 16, parent=FAKE + 32, alpha=FAKE + 48, prefix=FAKE + 64,
                loss=FAKE + 80, grad=FAKE + 96, ws=FAKE + 112)
    args.update(over)
    P = ctypes.c_void_p
    return sd.LIB.specopd_e2etv_fwd_bwd(
        ctypes.byref(desc), P(args["draft"]), P(args["target"]), P(args.get("target_row")),
        P(args["parent"]),
        P(args["alpha"]), P(args["prefix"]), P(args["loss"]), P(args["grad"]), P(args["ws"]),
        ctypes.c_size_t(ws_bytes), P(None))


@pytest.mark.parametrize("field,value,code", [
    ("V", 0, sd.SPECOPD_ERR_INVALID_ARGUMENT),
    ("R", 0, sd.SPECOPD_ERR_INVALID_ARGUMENT),
    ("Wn", 65, sd.SPECOPD_ERR_UNSUPPORTED),
    ("logits_dtype", 3, sd.SPECOPD_ERR_INVALID_ARGUMENT),
    ("grad_dtype", -1, sd.SPECOPD_ERR_INVALID_ARGUMENT),
    ("flags", 2, sd.SPECOPD_ERR_INVALID_ARGUMENT),
    ("grad_scale", float("inf"), sd.SPECOPD_ERR_INVALID_ARGUMENT),
    ("V", 200_000_000, sd.SPECOPD_ERR_UNSUPPORTED),  # beyond 32-bit element indexing
])
def test_e2etv_desc_errors(field, value, code):
    d = _edesc()
    setattr(d, field, value)
    assert _ecall(d) == code


@pytest.mark.parametrize("over,code", [
    (dict(draft=0), sd.SPECOPD_ERR_INVALID_ARGUMENT),
    (dict(loss=0), sd.SPECOPD_ERR_INVALID_ARGUMENT),
    (dict(parent=FAKE + 36), sd.SPECOPD_ERR_INVALID_ARGUMENT),
    (dict(grad=FAKE), sd.SPECOPD_ERR_INVALID_ARGUMENT),          # grad aliases draft
    (dict(alpha=FAKE + 50), sd.SPECOPD_ERR_INVALID_ARGUMENT),
    (dict(ws=0), sd.SPECOPD_ERR_WORKSPACE),
])
def test_e2etv_pointer_errors(over, code):
    assert _ecall(_edesc(), **over) == code


def test_e2etv_workspace_size_and_too_small():
    d = _edesc()
    need = sd.specopd_e2etv_workspace_size(d)
    assert need >= 4 * 7 * (16 + 4)
    assert _ecall(d, ws_bytes=need - 1) == sd.SPECOPD_ERR_WORKSPACE


def test_status_readback_rejects_bad_workspace_before_gpu():
    d = _tdesc()
    bad = ctypes.c_int32(0)
    assert sd.LIB.specopd_tree_attn_device_status(ctypes.byref(d), ctypes.c_void_p(None), 0,
                                                  ctypes.byref(bad), None) == sd.SPECOPD_ERR_WORKSPACE
    e = _edesc()
    assert sd.LIB.specopd_e2etv_device_status(ctypes.byref(e), ctypes.c_void_p(FAKE), 1,
                                              ctypes.byref(bad), None, None) == sd.SPECOPD_ERR_WORKSPACE


def _pdesc(**kw):
    base = dict(T=2, L=300, Hq=8, Hkv=2, D=128, dtype=sd.SPECOPD_BF16)
    base.update(kw)
    return sd.prefill_desc(**base)


def _pcall(desc, ws_bytes=1 << 30, **over):
    args = dict(q=FAKE, k=FAKE + 16, v=FAKE + 32, cache_k=FAKE + 48, cache_v=FAKE + 64,
                out=FAKE + 80, ws=FAKE + 96)
    args.update(over)
    P = ctypes.c_void_p
    return sd.LIB.specopd_prefill_fwd(
        ctypes.byref(desc), P(args["q"]), P(args["k"]), P(args["v"]), P(args["cache_k"]),
        P(args["cache_v"]), P(args["out"]), P(args["ws"]), ctypes.c_size_t(ws_bytes), P(None))


@pytest.mark.parametrize("field,value,code", [
    ("D", 96, sd.SPECOPD_ERR_UNSUPPORTED),
    ("D", 0, sd.SPECOPD_ERR_INVALID_ARGUMENT),
    ("Hq", 7, sd.SPECOPD_ERR_INVALID_ARGUMENT),
    ("L", 0, sd.SPECOPD_ERR_INVALID_ARGUMENT),
    ("T", -1, sd.SPECOPD_ERR_INVALID_ARGUMENT),
    ("dtype", 5, sd.SPECOPD_ERR_INVALID_ARGUMENT),
    ("flags", 1, sd.SPECOPD_ERR_INVALID_ARGUMENT),
    ("scale", float("nan"), sd.SPECOPD_ERR_INVALID_ARGUMENT),
    ("L", 300_000_000, sd.SPECOPD_ERR_UNSUPPORTED),  # L * Hq beyond 32-bit row indexing
    ("L", 20_000_000, sd.SPECOPD_ERR_UNSUPPORTED),   # one trunk's bf16 K beyond 4 GiB
])
def test_prefill_desc_errors(field, value, code):
    d = _pdesc()
    setattr(d, field, value)
    assert _pcall(d) == code
    n = ctypes.c_size_t(0)
    assert sd.LIB.specopd_prefill_workspace_size(ctypes.byref(d), ctypes.byref(n)) == code


@pytest.mark.parametrize("over,code", [
    (dict(q=0), sd.SPECOPD_ERR_INVALID_ARGUMENT),
    (dict(cache_v=0), sd.SPECOPD_ERR_INVALID_ARGUMENT),
    (dict(out=FAKE + 88), sd.SPECOPD_ERR_INVALID_ARGUMENT),       # misaligned
    (dict(out=FAKE), sd.SPECOPD_ERR_INVALID_ARGUMENT),            # out aliases q
    (dict(cache_k=FAKE + 16), sd.SPECOPD_ERR_INVALID_ARGUMENT),   # cache aliases k
    (dict(cache_v=FAKE + 48), sd.SPECOPD_ERR_INVALID_ARGUMENT),   # the two caches alias
    (dict(ws=0), sd.SPECOPD_ERR_WORKSPACE),
])
def test_prefill_pointer_errors(over, code):
    assert _pcall(_pdesc(), **over) == code


def test_prefill_workspace_size_and_too_small():
    d = _pdesc()
    need = sd.specopd_prefill_workspace_size(d)
    # the rotated, scaled queries of tokens 1..L-1 of every trunk, in bf16
    assert need >= 2 * 299 * 8 * 128 * 2
    assert _pcall(d, ws_bytes=need - 1) == sd.SPECOPD_ERR_WORKSPACE
    # a trunk of one token needs no plan
    assert sd.specopd_prefill_workspace_size(_pdesc(L=1)) < need
    # fp32 takes the exact per-trunk tree path and its own workspace
    assert sd.specopd_prefill_workspace_size(_pdesc(dtype=sd.SPECOPD_F32)) > 0


def _declared_arities():
    """Parameter count of every function include/specopd.h declares."""
    src = re.sub(r"/\*.*?\*/", "", open(HDR).read(), flags=re.S)
    out = {}
    for m in re.finditer(r"\b(specopd_[a-z0-9_]+)\s*\(([^)]*)\)\s*;", src):
        params = m.group(2).strip()
        out[m.group(1)] = 0 if params in ("", "void") else len(params.split(","))
    return out


def test_binding_argument_counts_match_the_header():
    """The ctypes signatures the binding sets agree with the header's
    parameter lists (a wrong count would pass garbage through the ABI)."""
    ar = _declared_arities()
    assert set(ar) == set(_lib.EXPORTS)
    for name, n in ar.items():
        fn = getattr(sd.LIB, name)
        assert fn.argtypes is not None, name
        assert len(fn.argtypes) == n, (name, len(fn.argtypes), n)


def test_header_is_plain_c_and_the_library_links_from_c(tmp_path):
    """include/specopd.h compiles as C99 with warnings as errors, and a C
    program linked against libspecopd.so gets the documented statuses."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    src = os.path.join(root, "tests", "c", "abi_errors.c")
    libdir = os.path.dirname(_lib.LIB_PATH)
    exe = str(tmp_path / "abi_errors")
    r = subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                        "-I", os.path.join(root, "include"), src, "-o", exe,
                        "-L", libdir, "-lspecopd", "-Wl,-rpath," + libdir],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr


def test_noalloc_rejects_host_errors_before_the_gpu():
    """The allocation-free E2E-TV call refuses, before any HIP call, a call
    whose workspace would exceed its static scratch, and bad arguments."""
    P = ctypes.c_void_p
    big = _edesc(R=1_000_000, Wn=7, V=16)
    n = ctypes.c_size_t(0)
    assert sd.LIB.specopd_e2etv_workspace_size(ctypes.byref(big), ctypes.byref(n)) == 0
    assert n.value > sd.E2ETV_NOALLOC_SCRATCH_BYTES

    def call(desc, **over):
        a = dict(draft=FAKE, target=FAKE + 16, parent=FAKE + 32, alpha=FAKE + 48, prefix=FAKE + 64,
                 loss=FAKE + 80, grad=FAKE + 96)
        a.update(over)
        return sd.LIB.specopd_e2etv_fwd_bwd_noalloc(
            ctypes.byref(desc), P(a["draft"]), P(a["target"]), P(None), P(a["parent"]), P(a["alpha"]),
            P(a["prefix"]), P(a["loss"]), P(a["grad"]), P(None))
    assert call(big) == sd.SPECOPD_ERR_WORKSPACE
    assert call(_edesc(), draft=0) == sd.SPECOPD_ERR_INVALID_ARGUMENT
    assert call(_edesc(), grad=FAKE) == sd.SPECOPD_ERR_INVALID_ARGUMENT  # grad aliases draft
    assert call(_edesc(Wn=65)) == sd.SPECOPD_ERR_UNSUPPORTED


def _gdesc(**kw):
    base = dict(T=2, L=300, B=4, Wn=7, H=4, D=128, C=64, dtype=sd.SPECOPD_BF16)
    base.update(kw)
    return sd.gdn_desc(**base)


def _gcall(desc, ws_bytes=256, **over):
    names = ("ckpt", "trunk_k", "trunk_v", "trunk_gate", "trunk_beta", "anchors", "parent", "q", "k",
             "v", "gate", "beta", "out", "ws")
    args = {n: FAKE + 16 * i for i, n in enumerate(names)}
    args.update(over)
    P = ctypes.c_void_p
    return sd.LIB.specopd_gdn_replay_fwd(
        ctypes.byref(desc), *[P(args[n]) for n in names[:-1]], P(args["ws"]), ctypes.c_size_t(ws_bytes),
        P(None))


@pytest.mark.parametrize("field,value,code", [
    ("D", 256, sd.SPECOPD_ERR_UNSUPPORTED),
    ("D", 0, sd.SPECOPD_ERR_INVALID_ARGUMENT),
    ("C", 0, sd.SPECOPD_ERR_INVALID_ARGUMENT),
    ("C", 65, sd.SPECOPD_ERR_UNSUPPORTED),       # longer replays than the work list holds
    ("Wn", 65, sd.SPECOPD_ERR_UNSUPPORTED),
    ("Wn", 0, sd.SPECOPD_ERR_INVALID_ARGUMENT),
    ("H", 0, sd.SPECOPD_ERR_INVALID_ARGUMENT),
    ("dtype", 5, sd.SPECOPD_ERR_INVALID_ARGUMENT),
    ("flags", 1, sd.SPECOPD_ERR_INVALID_ARGUMENT),
    ("L", 300_000_000, sd.SPECOPD_ERR_UNSUPPORTED),  # T * L beyond 2^28 tokens
])
def test_gdn_desc_errors(field, value, code):
    d = _gdesc()
    setattr(d, field, value)
    assert _gcall(d) == code
    n = ctypes.c_size_t(0)
    assert sd.LIB.specopd_gdn_workspace_size(ctypes.byref(d), ctypes.byref(n)) == code


@pytest.mark.parametrize("over,code", [
    (dict(ckpt=0), sd.SPECOPD_ERR_INVALID_ARGUMENT),              # L >= C: checkpoints needed
    (dict(parent=0), sd.SPECOPD_ERR_INVALID_ARGUMENT),
    (dict(gate=FAKE + 8), sd.SPECOPD_ERR_INVALID_ARGUMENT),       # misaligned
    (dict(out=FAKE + 16), sd.SPECOPD_ERR_INVALID_ARGUMENT),       # out aliases trunk_k
    (dict(ws=0), sd.SPECOPD_ERR_WORKSPACE),
])
def test_gdn_pointer_errors(over, code):
    assert _gcall(_gdesc(), **over) == code


def _cdesc(**kw):
    base = dict(T=2, L=300, B=4, Wn=7, H=4, D=128, K=4, dtype=sd.SPECOPD_BF16)
    base.update(kw)
    return sd.gdn_conv_desc(**base)


def _ccall(desc, **over):
    names = ("trunk_x", "x", "w", "anchors", "parent", "out")
    args = {n: FAKE + 16 * i for i, n in enumerate(names)}
    args.update(over)
    P = ctypes.c_void_p
    return sd.LIB.specopd_gdn_conv_fwd(ctypes.byref(desc), *[P(args[n]) for n in names], P(None))


@pytest.mark.parametrize("field,value,code", [
    ("D", 256, sd.SPECOPD_ERR_UNSUPPORTED),
    ("K", 0, sd.SPECOPD_ERR_INVALID_ARGUMENT),
    ("K", 9, sd.SPECOPD_ERR_UNSUPPORTED),
    ("Wn", 65, sd.SPECOPD_ERR_UNSUPPORTED),
    ("B", 0, sd.SPECOPD_ERR_INVALID_ARGUMENT),
    ("dtype", 5, sd.SPECOPD_ERR_INVALID_ARGUMENT),
    ("flags", 2, sd.SPECOPD_ERR_INVALID_ARGUMENT),   # only SPECOPD_GDN_CONV_L2NORM is defined
    ("L", 300_000_000, sd.SPECOPD_ERR_UNSUPPORTED),
])
def test_gdn_conv_desc_errors(field, value, code):
    d = _cdesc()
    setattr(d, field, value)
    assert _ccall(d) == code


@pytest.mark.parametrize("over", [dict(w=0), dict(parent=0), dict(out=0), dict(x=FAKE + 8),
                                  dict(out=FAKE + 16)])  # the last: out aliases x
def test_gdn_conv_pointer_errors(over):
    assert _ccall(_cdesc(), **over) == sd.SPECOPD_ERR_INVALID_ARGUMENT


def test_gdn_workspace_and_short_trunks():
    d = _gdesc()
    need = sd.specopd_gdn_workspace_size(d)
    assert _gcall(d, ws_bytes=need - 1) == sd.SPECOPD_ERR_WORKSPACE
    bad = ctypes.c_int32(0)
    assert sd.LIB.specopd_gdn_device_status(ctypes.byref(d), ctypes.c_void_p(None), 0, ctypes.byref(bad),
                                            None) == sd.SPECOPD_ERR_WORKSPACE


def _qdesc(**kw):
    base = dict(T=2, L=4096, B=8, Wn=10, Di=128, topk=64)
    base.update(kw)
    return sd.qsa_desc(**base)


_QNAMES = ("trunk_gk", "trunk_raw", "x", "y", "gamma", "anchors", "parent", "pos", "sel", "score", "bkey")


def _qcall(desc, ws_bytes=None, **over):
    args = {n: FAKE + 16 * i for i, n in enumerate(_QNAMES)}
    args["ws"] = FAKE + 4096
    args.update(over)
    if ws_bytes is None:
        try:
            ws_bytes = sd.specopd_qsa_workspace_size(desc)
        except sd.SpecopdError:
            ws_bytes = 1 << 40
    P = ctypes.c_void_p
    return sd.LIB.specopd_qsa_select_fwd(ctypes.byref(desc), *[P(args[n]) for n in _QNAMES], P(args["ws"]),
                                         ctypes.c_size_t(ws_bytes), P(None))


@pytest.mark.parametrize("field,value,code", [
    ("Di", 96, sd.SPECOPD_ERR_UNSUPPORTED),
    ("Di", 0, sd.SPECOPD_ERR_INVALID_ARGUMENT),
    ("topk", 0, sd.SPECOPD_ERR_INVALID_ARGUMENT),
    ("Wn", 65, sd.SPECOPD_ERR_UNSUPPORTED),
    ("B", 0, sd.SPECOPD_ERR_INVALID_ARGUMENT),
    ("L", 61_440 - 9, sd.SPECOPD_ERR_UNSUPPORTED),    # (L + Wn) / 4 above the LDS bound
    ("flags", 1, sd.SPECOPD_ERR_INVALID_ARGUMENT),
    ("rope_base", float("inf"), sd.SPECOPD_ERR_INVALID_ARGUMENT),
])
def test_qsa_desc_errors(field, value, code):
    d = _qdesc()
    setattr(d, field, value)
    assert _qcall(d) == code


def test_qsa_largest_supported_trunk():
    d = _qdesc(L=61_440 - 10, T=1, B=1)
    assert sd.specopd_qsa_workspace_size(d) > 0


@pytest.mark.parametrize("over,code", [
    (dict(trunk_gk=0), sd.SPECOPD_ERR_INVALID_ARGUMENT),
    (dict(gamma=0), sd.SPECOPD_ERR_INVALID_ARGUMENT),
    (dict(sel=0), sd.SPECOPD_ERR_INVALID_ARGUMENT),
    (dict(score=0), sd.SPECOPD_ERR_INVALID_ARGUMENT),
    (dict(y=FAKE + 8), sd.SPECOPD_ERR_INVALID_ARGUMENT),       # misaligned
    (dict(sel=FAKE + 16), sd.SPECOPD_ERR_INVALID_ARGUMENT),    # sel aliases trunk_raw
    (dict(bkey=FAKE + 16 * 9), sd.SPECOPD_ERR_INVALID_ARGUMENT),  # bkey aliases score
    (dict(ws=0), sd.SPECOPD_ERR_WORKSPACE),
    (dict(ws=FAKE + 4100), sd.SPECOPD_ERR_WORKSPACE),          # misaligned workspace
])
def test_qsa_pointer_errors(over, code):
    assert _qcall(_qdesc(), **over) == code


def test_qsa_workspace_and_status_errors():
    d = _qdesc()
    need = sd.specopd_qsa_workspace_size(d)
    # scores of every node's candidates: rows x (L + Wn) / 4 floats, plus counts
    assert need >= 2 * 8 * 10 * ((4096 + 10) // 4) * 4
    assert _qcall(d, ws_bytes=need - 1) == sd.SPECOPD_ERR_WORKSPACE
    bad = ctypes.c_int32(0)
    assert sd.LIB.specopd_qsa_device_status(ctypes.byref(d), ctypes.c_void_p(None), 0, ctypes.byref(bad),
                                            None) == sd.SPECOPD_ERR_WORKSPACE
    P = ctypes.c_void_p
    assert sd.LIB.specopd_qsa_trunk_groups_fwd(ctypes.byref(d), P(FAKE), P(0), P(FAKE + 32), P(None)) \
        == sd.SPECOPD_ERR_INVALID_ARGUMENT
    assert sd.LIB.specopd_qsa_trunk_groups_fwd(ctypes.byref(d), P(FAKE), P(FAKE + 16), P(FAKE), P(None)) \
        == sd.SPECOPD_ERR_INVALID_ARGUMENT  # out aliases the raw keys


def _ldesc(**kw):
    base = dict(R=64, Wn=8, V=151936, H=4096, M=4608)
    base.update(kw)
    return sd.lmhead_desc(**base)


_LNAMES = ("h_draft", "w_draft", "h_target", "w_target", "target_row", "parent", "alpha", "prefix", "loss", "grad")


def _lcall(desc, ws_bytes=None, **over):
    args = {n: FAKE + 16 * i for i, n in enumerate(_LNAMES)}
    args["ws"] = FAKE + 4096
    args.update(over)
    if ws_bytes is None:
        try:
            ws_bytes = sd.specopd_lmhead_e2etv_workspace_size(desc)
        except sd.SpecopdError:
            ws_bytes = 1 << 40
    P = ctypes.c_void_p
    return sd.LIB.specopd_lmhead_e2etv_fwd_bwd(ctypes.byref(desc), *[P(args[n]) for n in _LNAMES], P(args["ws"]),
                                               ctypes.c_size_t(ws_bytes), P(None))


@pytest.mark.parametrize("field,value,code", [
    ("H", 4100, sd.SPECOPD_ERR_UNSUPPORTED),       # not a multiple of 16
    ("H", 8, sd.SPECOPD_ERR_INVALID_ARGUMENT),
    ("V", 0, sd.SPECOPD_ERR_INVALID_ARGUMENT),
    ("M", 0, sd.SPECOPD_ERR_INVALID_ARGUMENT),
    ("Wn", 65, sd.SPECOPD_ERR_UNSUPPORTED),
    ("R", 0, sd.SPECOPD_ERR_INVALID_ARGUMENT),
    ("flags", 1, sd.SPECOPD_ERR_INVALID_ARGUMENT),
    ("norm_count", float("nan"), sd.SPECOPD_ERR_INVALID_ARGUMENT),
    ("V", 2_000_000_000, sd.SPECOPD_ERR_UNSUPPORTED),
])
def test_lmhead_desc_errors(field, value, code):
    d = _ldesc()
    setattr(d, field, value)
    assert _lcall(d) == code


@pytest.mark.parametrize("over,code", [
    (dict(h_draft=0), sd.SPECOPD_ERR_INVALID_ARGUMENT),
    (dict(target_row=0), sd.SPECOPD_ERR_INVALID_ARGUMENT),
    (dict(loss=0), sd.SPECOPD_ERR_INVALID_ARGUMENT),           # the loss is always written
    (dict(w_target=FAKE + 8), sd.SPECOPD_ERR_INVALID_ARGUMENT),  # misaligned
    (dict(grad=FAKE), sd.SPECOPD_ERR_INVALID_ARGUMENT),         # grad aliases h_draft
    (dict(prefix=FAKE + 16 * 6), sd.SPECOPD_ERR_INVALID_ARGUMENT),  # prefix aliases alpha
    (dict(ws=0), sd.SPECOPD_ERR_WORKSPACE),
])
def test_lmhead_pointer_errors(over, code):
    assert _lcall(_ldesc(), **over) == code


def test_lmhead_workspace_and_status_errors():
    d = _ldesc()
    need = sd.specopd_lmhead_e2etv_workspace_size(d)
    # per row and 64-entry chunk: 16 bytes of log-sum-exp partials and 8 of overlap partials
    assert need >= 512 * ((151936 + 63) // 64) * 24
    assert _lcall(d, ws_bytes=need - 1) == sd.SPECOPD_ERR_WORKSPACE
    bad = ctypes.c_int32(0)
    assert sd.LIB.specopd_lmhead_e2etv_device_status(ctypes.byref(d), ctypes.c_void_p(None), 0,
                                                     ctypes.byref(bad), None) == sd.SPECOPD_ERR_WORKSPACE
