"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The oracle (plain C) is built with gcc's sanitizers together with
  tests/sanitize/oracle_drive.c, which walks every oracle function through small
  inputs and their edge cases; the run must end cleanly (leak checking on).
* The C ABI's host code (api.cpp: argument checks, workspace sizes, error
  text) is built with the sanitizers on its host side only and linked with the
  library's kernel objects; the host-side rejection tests of test_abi.py then
  run against that library in a child process that preloads the sanitizer
  runtime. No call reaches the device.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_attention_kpool_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"
KERNEL_OBJS = ["pool.o", "score.o", "topk.o", "fused_topk.o", "sparse_mla.o", "sparse_mla_bwd.o"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\nrc={r.returncode}\n{r.stdout[-3000:]}\n{r.stderr[-6000:]}"
    return r


def test_oracle_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc missing")
    exe = str(tmp_path / "oracle_drive")
    _run(["gcc", "-std=c11", "-g", "-O1", "-fopenmp", "-ffp-contract=off", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "oracle"),
          os.path.join(ROOT, "tests", "sanitize", "oracle_drive.c"), os.path.join(ROOT, "oracle", "kpool_oracle.c"),
          "-o", exe, "-lm"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1",
               OMP_NUM_THREADS="2")
    r = _run([exe], env=env, timeout=300)
    assert "oracle drive ok" in r.stdout


def test_abi_host_code_under_sanitizers(tmp_path):
    asan = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not (os.path.exists(HIPCC) and os.path.exists(CLANGXX) and asan):
        pytest.skip("hipcc, clang++ or the sanitizer runtime missing")
    objdir = os.path.join(ROOT, "_build", "kpool")
    if not all(os.path.exists(os.path.join(objdir, o)) for o in KERNEL_OBJS):
        from sparse_attention_kpool_amd import build
        build.build()
    api_o = str(tmp_path / "api.o")
    # sanitizers on the host side of api.cpp only (its device part is one scratch array)
    _run([HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-x", "hip", "-c", os.path.join(CSRC, "api.cpp"),
          "-o", api_o])
    lib = str(tmp_path / "libkpool_san.so")
    _run([CLANGXX, "-shared", "-fPIC", "-fsanitize=address,undefined", "-shared-libsan", api_o,
          *[os.path.join(objdir, o) for o in KERNEL_OBJS], "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib", "-o", lib])
    nm = _run(["nm", "-u", lib]).stdout
    assert "__asan_report" in nm, "api.cpp was not instrumented"
    child = (
        "import ctypes as C, sys\n"
        f"sys.path.insert(0, {ROOT!r})\n"
        "from sparse_attention_kpool_amd import _lib\n"
        f"L = C.CDLL({lib!r})\n"
        "for name, res, args in _lib.SIGNATURES:\n"
        "    f = getattr(L, name); f.restype = res; f.argtypes = args\n"
        "import tests.test_abi as T\n"
        "T.test_row_width(L)\n"
        "T.test_workspace_size(L)\n"
        "T.test_invalid_args_rejected_on_host(L)\n"
        "T.test_paged_args_rejected_on_host(L)\n"
        "print('abi host checks ok')\n")
    env = dict(os.environ, LD_PRELOAD=asan[-1], ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = _run([sys.executable, "-c", child], env=env, timeout=300, cwd=ROOT)
    assert "abi host checks ok" in r.stdout
