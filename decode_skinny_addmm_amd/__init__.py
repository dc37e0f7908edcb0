"""MI355X-native skinny residual GEMM  Y = X * W^T + R  (bf16 in, fp32 accumulate, bf16 out).

The compute runs in hand-written HIP kernels for gfx950 behind the C ABI in
``include/skinny.h`` (library ``libskinny.so``); this package only marshals
arguments to it. Importing the package does not load the library; the first
call into it does, and raises if the library has not been built.
"""
from . import synth  # noqa: F401  (input generators; no arithmetic of the operation)

__all__ = ["synth"]
