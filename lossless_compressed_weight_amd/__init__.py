"""W12 lossless 12-bit weights and their skinny GEMM on MI355X (gfx950).

The compute lives in libw12.so (hand-written HIP kernels behind a C ABI,
include/w12.h); ``lossless_compressed_weight_amd.w12`` is its Python binding,
which loads the library on first use and raises if it is missing.
"""
