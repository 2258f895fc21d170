"""MI355X (gfx950) W4A4 dual-branch linear: Y = Q(X_J / s_J) Q(s_J * W_J) + X_O W_O.

The compute lives in libw4a4.so (hand-written HIP kernels behind a C ABI, declared in
include/w4a4.h); ``bit_quantized_dit_amd.w4a4`` is its ctypes binding.  Importing the
package loads nothing; the first library call loads the .so and raises if it is missing.
"""
