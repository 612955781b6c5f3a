"""Build the CPU oracle shared library (test infrastructure only).

    python oracle/build.py [--out PATH] [--src PATH]

gcc, C99, no floating-point contraction and no fast-math, so every fp32
rounding is the one the source writes; OpenMP spreads independent queries.
"""
import argparse
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qsa_oracle.c")
LIB = os.path.join(HERE, "libqsa_oracle.so")
FLAGS = ["-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
         "-shared", "-fPIC", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(out: str = LIB, src: str = SRC, extra=()) -> str:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", *FLAGS, *extra, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build_asan(out: str = os.path.join(HERE, "_asan", "libqsa_oracle_asan.so")) -> str:
    """The oracle with host AddressSanitizer (gcc's runtime: load it with
    asan_runtime() preloaded)."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    return build(out, extra=("-fsanitize=address", "-fno-omit-frame-pointer", "-g"))


def asan_runtime() -> str:
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                       check=True)
    return os.path.realpath(p.stdout.strip())


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=LIB)
    ap.add_argument("--src", default=SRC)
    a = ap.parse_args()
    print(build(a.out, a.src))
    sys.exit(0)
