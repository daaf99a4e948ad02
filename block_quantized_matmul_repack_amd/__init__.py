"""Tiled block-32 quantized matmul (Q4_0 / Q8_0 / IQ4_NL / MXFP4 / Q4_1 / Q4_K 32x32 tiles) on MI355X.

The computation lives in libtiledq.so (HIP kernels for gfx950 behind a C ABI
declared in include/tiledq.h); this package is its thin torch binding.
"""
from .ops import (BF16, F16, F32, IQ4_NL, MXFP4, PATH_GEMM, PATH_GEMM_FLAT, PATH_GEMM_MX, PATH_GEMM_SPLIT, PATH_GEMV,  # noqa: F401
                  PATH_GEMV_FLAT, Q4_0, Q4_1, Q4_K, Q8_0, block_bytes, block_dots, flat_bytes,
                  matmul, matmul_flat, matmul_mx, matmul_path, matmul_x, qgemm, qgemm_flat, qgemm_mx, qgemv, qgemv_flat, qgemv_noalloc, qgemv_x,
                  quantize_act, quantize_act_mx, repack_tiles, stream_read, supported, tile_bytes, tiled_bytes,
                  unpack_tiles)
from ._lib import TiledqError, lib  # noqa: F401
