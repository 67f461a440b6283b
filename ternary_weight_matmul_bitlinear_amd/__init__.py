"""MatMul-free LM block forward (ternary BitLinear -> MLGRU -> GLU) on MI355X (gfx950).

The compute runs in libmmf.so (hand-written HIP kernels behind the C ABI of
include/mmf.h); `api` is the Python binding.  Importing the package does not load the
library; the first call does, and fails loudly if it has not been built.
"""
__all__ = ["api", "synth"]
