"""Tiled block-32 quantized matmul (Q4_0 / Q8_0 / IQ4_NL / MXFP4 / Q4_1 / Q4_K 32x32 tiles) on MI355X.

The computation lives in libtiledq.so (HIP kernels for gfx950 behind a C ABI
declared in include/tiledq.h); this package is its thin torch binding.
"""
from .ops import (BF16, F16, F32, IQ4_NL, MXFP4, PATH_GEMM, Q4_1, Q4_K, PATH_GEMV, Q4_0, Q8_0,  # noqa: F401
                  block_bytes, block_dots, flat_bytes, matmul, qgemm, qgemv, qgemv_x, quantize_act,
                  repack_tiles, supported, tile_bytes, tiled_bytes)
from ._lib import TiledqError, lib  # noqa: F401
