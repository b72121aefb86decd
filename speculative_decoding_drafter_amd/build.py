"""Builds libspecopd.so in-tree with hipcc for gfx950.

    python speculative_decoding_drafter_amd/build.py

Every source is compiled on every call (the caller wants a fresh check that
the tree builds); objects go to ``_build/`` next to this file.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libspecopd.so")

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

# Packed fp32 VALU instructions are switched off: the compiler would otherwise
# form them from ordinary float code, and some of their forms are not trusted
# on this hardware.
COMMON = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(HERE, "..", "include"),
]

SOURCES = ["specopd_api.cpp", "e2etv.hip", "tree_attn.hip", "tree_attn_mfma.hip", "prefill.hip", "gdn.hip", "gdn_conv.hip", "qsa.hip", "lmhead.hip"]

# Matrix-core accumulators live in ordinary VGPRs (the AGPR half of the file
# serves as extra room): with one wave per SIMD the attention kernel's
# softmax works on the same registers the matrix core writes, and the
# default form would shuttle them between the two halves every tile.
EXTRA = {"tree_attn_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src: str) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, *EXTRA.get(src, []), "-c", path, "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if warn and os.environ.get("SPECOPD_BUILD_VERBOSE"):
        print(warn, file=sys.stderr)
    return obj


def build(jobs: int = 4) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
