"""Build libkpool.so (the gfx950 kernels and their C ABI) in-tree with hipcc.

    python -m sparse_attention_kpool_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build", "kpool")
LIB = os.path.join(PKG, "libkpool.so")
SOURCES = ["api.cpp", "pool.hip", "score.hip", "topk.hip", "fused_topk.hip", "sparse_mla.hip", "sparse_mla_bwd.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
# selection switched off (v_pk_*_f32 stay out of the code objects).
COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-munsafe-fp-atomics",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-result", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]


# Per-file additions. The scoring kernel consumes each MFMA result in VALU
# code right away: asking for MFMA results in ordinary VGPRs (instead of the
# accumulation registers) lets the compiler keep eight MFMAs in flight. The
# attention kernel's QK scores are read by the softmax the same way (its O
# accumulators are pinned to AGPRs by inline assembly and unaffected).
EXTRA = {"score.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "sparse_mla.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"]
    cmd = [HIPCC, *COMMON, *EXTRA.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    return obj


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(min(jobs, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
