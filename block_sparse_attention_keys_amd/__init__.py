"""Qwen Sparse Attention (QSA) hot path for AMD Instinct MI355X (gfx950).

Submodules:
  qsa        ctypes binding of the C-ABI library ``libqsa.so`` (HIP kernels)
  workloads  seeded synthetic inputs (random draws only, no method arithmetic)
  build      compiles ``csrc/`` into ``libqsa.so`` with hipcc for gfx950

Importing the package loads nothing; ``qsa`` loads the library on first use.
"""
__all__ = ["qsa", "workloads"]
