"""MI355X (gfx950) fused GEMM + ordered epilogue library.

The compute lives in libcoda.so (HIP kernels behind the C ABI of
include/coda.h).  Submodules:

  coda    - ctypes binding with the C ABI's function names
  runner  - marshalling of torch device tensors into a coda_epi_desc
  build   - compiles libcoda.so in-tree with hipcc for gfx950

Importing ``coda`` (or ``runner``) raises if libcoda.so has not been built.
"""
__all__ = ["coda", "runner", "build"]
