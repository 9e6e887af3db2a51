"""Builds libjano.so (HIP for gfx950) in-tree with hipcc, and beside it
libjano_calib.so, the calibration kernels that measurements use to find the
matrix-core rate and the streaming HBM rates the part sustains (not part of
the Jano path), and
libjano_asan.so, the same library with its host code (argument checks,
launch set-up) built with AddressSanitizer for host-only ABI tests. The
device code of the ASan build is compiled as usual; only the host pass is
instrumented.

    python -m token_sparse_attention_block_amd.build [-v]

Objects go to token_sparse_attention_block_amd/_build/, the libraries to
token_sparse_attention_block_amd/lib/ (each replaced atomically).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libjano.so")
SOURCES = ["capi.hip", "analyze.hip", "schedule.hip", "rows.hip", "attention.hip", "proj.hip"]
CALIB_LIB = os.path.join(LIBDIR, "libjano_calib.so")
CALIB_SOURCES = ["calib/mfma_loop.hip", "calib/stream.hip"]
ASAN_LIB = os.path.join(LIBDIR, "libjano_asan.so")
ASAN_OBJ = os.path.join(OBJ, "asan")
# host pass only: each sanitizer flag goes to the host compiler alone
ASAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.
COMMON = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]

# Per-source extras. attention.hip: its inputs are finite by contract (the
# scores are finite products of finite bf16 values), so the max reductions of
# the online softmax need no NaN canonicalisation; the ILP-first machine
# scheduler interleaves its MFMA, exp and LDS streams better than the default
# occupancy-first one (the kernel's occupancy is fixed by its LDS use anyway).
EXTRA = {"attention.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-sched-strategy=max-ilp"]}


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libjano)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("command failed: %s\n%s" % (" ".join(cmd), out))
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False, jobs: int = 8, asan: bool = True) -> str:
    cc = hipcc()
    os.makedirs(OBJ, exist_ok=True)
    os.makedirs(ASAN_OBJ, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    # (library, sources, object dir, extra compile flags, extra link flags)
    libs = [(LIB, SOURCES, OBJ, [], []), (CALIB_LIB, CALIB_SOURCES, OBJ, [], [])]
    if asan:
        libs.append((ASAN_LIB, SOURCES, ASAN_OBJ, ["-g"] + ASAN_HOST,
                     ["-Xarch_host", "-fsanitize=address", "-shared-libsan"]))

    def obj(d, s):
        return os.path.join(d, s.replace("/", "_").replace(".hip", ".o"))

    cmds = []
    for _, sources, d, cflags, _ in libs:
        for s in sources:
            cmds.append([cc] + COMMON + EXTRA.get(s, []) + cflags + ["-c", os.path.join(SRC, s), "-o", obj(d, s)])
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(cmds)))) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    for lib, sources, d, _, lflags in libs:
        tmp = lib + ".tmp"
        _run([cc, "--offload-arch=" + ARCH, "-shared", "-fPIC"] + lflags + ["-o", tmp] +
             [obj(d, s) for s in sources], verbose)
        os.replace(tmp, lib)
    return LIB


def asan_runtime() -> str:
    """Path of the ASan runtime that libjano_asan.so needs preloaded (the
    Python interpreter itself is not instrumented)."""
    cc = os.path.realpath(hipcc())
    out = subprocess.run([os.path.join(os.path.dirname(os.path.dirname(cc)), "llvm", "bin", "clang"),
                          "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = out.stdout.strip()
    if out.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("ASan runtime not found")
    return path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
