"""bit_exact_speculative_amd -- batch-invariant speculative-decoding verify step on MI355X.

Submodules:
  xv      ctypes binding of libxv.so (the C-ABI library of HIP kernels for gfx950)
  layer   one hybrid layer's verify step and its sequential-decode counterpart
  inputs  seeded synthetic inputs (shared with the CPU oracle used by the tests)
  build   ahead-of-time hipcc build of libxv.so

Importing the package loads nothing; ``import bit_exact_speculative_amd.xv``
loads the library and fails loudly if it has not been built.
"""
__all__ = ["xv", "layer", "inputs", "build"]
