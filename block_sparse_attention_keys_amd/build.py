"""Compile the QSA HIP sources into the in-tree shared library ``libqsa.so``.

    python -m block_sparse_attention_keys_amd.build

hipcc for gfx950 only.  Packed fp32 instructions are disabled on the device
(``-packed-fp32-ops``) and floating-point contraction is off, so every fmaf
in the kernels is one the source writes.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libqsa.so")
# debug build for tests: counts the K/V rows the attention kernels load
PROBE_LIB = os.path.join(PKG, "libqsa_probe.so")
PROBE_FLAGS = ["-DQSA_COUNT_KEYS"]
SOURCES = ["qsa_api.hip", "qsa_kernels.hip", "qsa_block.hip", "qsa_prefill_ks.hip", "qsa_blas.hip"]
ARCH = "gfx950"
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-result", "-I", INCLUDE, "-I", CSRC]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.isabs(c) and os.path.exists(c) or not os.path.isabs(c)):
            return c
    return "hipcc"


def build(out: str = LIB, extra=(), verbose: bool = False) -> str:
    """Compile every source to an object (in parallel), then link ``out``."""
    hipcc = _hipcc()
    bdir = os.path.join(PKG, "_build", "probe" if extra else "lib")
    os.makedirs(bdir, exist_ok=True)

    def comp(src):
        obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        p = subprocess.run(cmd, capture_output=True, text=True)
        if p.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{p.stderr}")
        return obj

    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(comp, SOURCES))
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-ldl", "-o", tmp]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed:\n{p.stderr}")
    os.replace(tmp, out)
    return out


# Host AddressSanitizer build of the C-ABI layer (host code only; the device
# code is built as usual): for the CPU tests that drive argument validation
# under ASan.  Load it with the compiler's ASan runtime preloaded.
ASAN_LIB = os.path.join(PKG, "_build", "asan", "libqsa_asan.so")
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def build_asan() -> str:
    """libqsa_asan.so: qsa_api.hip with host ASan, the kernels' objects as
    built for the product library (built first if missing)."""
    hipcc = _hipcc()
    lib_dir = os.path.join(PKG, "_build", "lib")
    objs = [os.path.join(lib_dir, os.path.splitext(x)[0] + ".o") for x in SOURCES
            if x != "qsa_api.hip"]
    if not all(os.path.exists(o) for o in objs):
        build(LIB)
    adir = os.path.dirname(ASAN_LIB)
    os.makedirs(adir, exist_ok=True)
    api = os.path.join(adir, "qsa_api.o")
    cmd = [hipcc, *FLAGS, *ASAN_FLAGS, "-c", os.path.join(CSRC, "qsa_api.hip"), "-o", api]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed on the ASan build:\n{p.stderr}")
    tmp = ASAN_LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", *ASAN_FLAGS, api, *objs, "-ldl",
           "-o", tmp]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed (ASan build):\n{p.stderr}")
    os.replace(tmp, ASAN_LIB)
    return ASAN_LIB


def asan_runtime() -> str:
    """The ASan runtime of the compiler that builds the library."""
    clang = os.path.join(os.path.dirname(os.path.realpath(_hipcc())), "..", "lib", "llvm", "bin",
                         "clang")
    for c in (clang, "/opt/rocm/llvm/bin/clang"):
        if os.path.exists(c):
            p = subprocess.run([c, "-print-file-name=libclang_rt.asan-x86_64.so"],
                               capture_output=True, text=True)
            path = p.stdout.strip()
            if p.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
                return path
    raise RuntimeError("the compiler's ASan runtime was not found")


def build_all(verbose: bool = False) -> list:
    """The product library and the probe build."""
    return [build(LIB, verbose=verbose), build(PROBE_LIB, PROBE_FLAGS, verbose=verbose)]


if __name__ == "__main__":
    print(build_all(verbose="-v" in sys.argv))
