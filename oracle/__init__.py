"""Plain CPU oracle for tiled block-32 quantized matmul (ctypes shim over oracle.c).

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the benchmark's
CPU-baseline leg may import this package.  It shares no code with the HIP
library or its binding, and neither imports the other.

Every function follows the page "Hexagon backend developer details", section
"Tiled Weight Formats" (subsections "Tile Dimensions and Grid Layout" and
"Block-32 Quantized Formats") and section "Memory buffers"; the C source states
the reading taken wherever the page is silent.  Arrays are numpy, C-contiguous.

Parity pins: see tests/test_oracle_*.py.  The flat GGML block nibble order
(flat_decode, and through it the input side of repack) is "parity unpinned":
the page does not print the flat layout; for MXFP4 the flat block (one E8M0
byte, then 16 nibble bytes) and for Q4_1 (fp16 d, fp16 m, then 16 nibble
bytes) and for Q4_K (the 144-byte super-block with 6-bit scales and mins) are
unpinned for the same reason.
"""
import ctypes
import os

import numpy as np

from . import build as _build

Q4_0, Q8_0, IQ4_NL, MXFP4, Q4_1, Q4_K = 0, 1, 2, 3, 4, 5
F32, BF16, F16 = 0, 1, 2

_lib = None


def lib():
    global _lib
    if _lib is None:
        path = _build.LIB
        _build.build(force=False)
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        l = ctypes.c_long
        L.or_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.or_f16_to_f32.restype = ctypes.c_float
        L.or_f32_to_f16.argtypes = [ctypes.c_float]
        L.or_f32_to_f16.restype = ctypes.c_uint16
        L.or_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.or_bf16_to_f32.restype = ctypes.c_float
        for f in ("or_tile_bytes", "or_block_bytes", "or_scale_count", "or_block_elems"):
            getattr(L, f).argtypes = [ctypes.c_int]
            getattr(L, f).restype = l
        for f in ("or_tiled_bytes", "or_flat_bytes"):
            getattr(L, f).argtypes = [ctypes.c_int, l, l]
            getattr(L, f).restype = l
        L.or_flat_decode.argtypes = [ctypes.c_int, P, l, l, P, P]
        L.or_flat_decode.restype = None
        L.or_repack.argtypes = [ctypes.c_int, P, l, l, P]
        L.or_repack.restype = None
        L.or_unpack.argtypes = [ctypes.c_int, P, l, l, P, P]
        L.or_unpack.restype = None
        L.or_quantize_act.argtypes = [ctypes.c_int, P, l, l, l, P, P]
        L.or_quantize_act.restype = ctypes.c_int
        L.or_block_dots.argtypes = [ctypes.c_int, P, l, l, P, l, P, P]
        L.or_block_dots.restype = ctypes.c_int
        L.or_matmul.argtypes = [ctypes.c_int, P, l, l, P, P, l, P, l, l, P, P, l]
        L.or_matmul.restype = None
        L.or_block_dots_flat.argtypes = [ctypes.c_int, P, l, l, P, l, P, P]
        L.or_block_dots_flat.restype = ctypes.c_int
        L.or_matmul_flat.argtypes = [ctypes.c_int, P, l, l, P, P, l, P, l, l, P, P, l]
        L.or_matmul_flat.restype = None
        L.or_e4m3_value.argtypes = [ctypes.c_uint8]
        L.or_e4m3_value.restype = ctypes.c_double
        L.or_quantize_act_mx.argtypes = [ctypes.c_int, P, l, l, l, P, P]
        L.or_quantize_act_mx.restype = None
        L.or_matmul_mx.argtypes = [P, l, l, P, P, l, l, l, P, P, l]
        L.or_matmul_mx.restype = None
        L.or_row_scale.argtypes = [ctypes.c_int, ctypes.c_uint16]
        L.or_row_scale.restype = ctypes.c_double
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def f16_to_f32(bits):
    return lib().or_f16_to_f32(int(bits))


def f32_to_f16(x):
    return lib().or_f32_to_f16(float(np.float32(x)))


def bf16_to_f32(bits):
    return lib().or_bf16_to_f32(int(bits))


def f16_to_f32_array(bits):
    bits = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([lib().or_f16_to_f32(int(b)) for b in bits], dtype=np.float32)


def f32_to_f16_array(x):
    x = np.asarray(x, dtype=np.float32).ravel()
    return np.array([lib().or_f32_to_f16(float(v)) for v in x], dtype=np.uint16)


def tile_bytes(t):
    return lib().or_tile_bytes(t)


def block_bytes(t):
    return lib().or_block_bytes(t)


def tiled_bytes(t, K, N):
    return lib().or_tiled_bytes(t, K, N)


def flat_bytes(t, K, N):
    return lib().or_flat_bytes(t, K, N)


def row_scale(t, s):
    """The factor one tile row scale s contributes to y (fp64): the fp16 value
    of s, or for MXFP4 half the power of two the E8M0 byte s stands for."""
    return lib().or_row_scale(t, int(s))


def scale_count(t):
    return lib().or_scale_count(t)


def block_elems(t):
    return lib().or_block_elems(t)


def _scales_array(t, N, nb):
    ns = scale_count(t)
    return np.zeros((N, nb) if ns == 1 else (N, nb, ns), np.uint16)


def flat_decode(t, flat, K, N):
    """Flat GGML blocks -> (codes uint8 [N,K], scale bits uint16 [N,K/32]);
    for Q4_1 the scales are [N,K/32,2] (d, m)."""
    flat = _c(flat, np.uint8)
    assert flat.size == flat_bytes(t, K, N)
    codes = np.zeros((N, K), np.uint8)
    scales = _scales_array(t, N, K // 32)
    lib().or_flat_decode(t, _p(flat), K, N, _p(codes), _p(scales))
    return codes, scales


def repack(t, flat, K, N):
    """Flat GGML blocks -> tiled bytes (uint8, tiled_bytes(t, K, N))."""
    flat = _c(flat, np.uint8)
    assert flat.size == flat_bytes(t, K, N)
    tiles = np.empty(tiled_bytes(t, K, N), np.uint8)
    lib().or_repack(t, _p(flat), K, N, _p(tiles))
    return tiles


def unpack(t, tiles, K, N):
    """Tiled bytes -> (codes uint8 [N,K], scale bits as flat_decode)."""
    tiles = _c(tiles, np.uint8)
    assert tiles.size == tiled_bytes(t, K, N)
    codes = np.zeros((N, K), np.uint8)
    scales = _scales_array(t, N, K // 32)
    lib().or_unpack(t, _p(tiles), K, N, _p(codes), _p(scales))
    return codes, scales


def quantize_act(x, dtype=F32, K=None):
    """x: [M, K] float32 (dtype F32) or uint16 bit patterns (BF16 / F16).

    Returns (q int8 [M,K], d uint16 fp16 bits [M,K/32])."""
    x = np.ascontiguousarray(x, dtype=np.float32 if dtype == F32 else np.uint16)
    M, Kx = x.shape
    K = Kx if K is None else K
    q = np.zeros((M, K), np.int8)
    d = np.zeros((M, K // 32), np.uint16)
    rc = lib().or_quantize_act(dtype, _p(x), M, K, Kx, _p(q), _p(d))
    if rc != 0:
        raise ValueError("quantize_act: |q| > 127")
    return q, d


def block_dots(t, tiles, K, N, q, lut=None):
    """Integer block dots isum int32 [M, N, K/32]."""
    tiles = _c(tiles, np.uint8)
    q = _c(q, np.int8)
    M = q.shape[0]
    lut = None if lut is None else _c(lut, np.int8)
    isum = np.zeros((M, N, K // 32), np.int32)
    rc = lib().or_block_dots(t, _p(tiles), K, N, _p(q), M, _p(lut), _p(isum))
    if rc != 0:
        raise ValueError("block_dots: int32 overflow")
    return isum


def matmul(t, tiles, K, N, q, d, lut=None, n0=0, n1=None):
    """y[m, n] (fp64) and acond[m, n] = sum |W*A| for n0 <= n < n1."""
    tiles = _c(tiles, np.uint8)
    q = _c(q, np.int8)
    d = _c(d, np.uint16)
    M = q.shape[0]
    n1 = N if n1 is None else min(n1, N)
    lut = None if lut is None else _c(lut, np.int8)
    y = np.zeros((M, N), np.float64)
    acond = np.zeros((M, N), np.float64)
    lib().or_matmul(t, _p(tiles), K, N, _p(q), _p(d), M, _p(lut), n0, n1,
                    _p(y), _p(acond), N)
    return y, acond


def block_dots_flat(t, flat, K, N, q, lut=None):
    """Integer block dots int32 [M, N, K/32] over flat GGML blocks."""
    flat = _c(flat, np.uint8)
    assert flat.size == flat_bytes(t, K, N)
    q = _c(q, np.int8)
    M = q.shape[0]
    lut = None if lut is None else _c(lut, np.int8)
    isum = np.zeros((M, N, K // 32), np.int32)
    if lib().or_block_dots_flat(t, _p(flat), K, N, _p(q), M, _p(lut), _p(isum)) != 0:
        raise ValueError("block_dots_flat: int32 overflow")
    return isum


def matmul_flat(t, flat, K, N, q, d, lut=None, n0=0, n1=None):
    """As matmul, over flat GGML blocks."""
    flat = _c(flat, np.uint8)
    assert flat.size == flat_bytes(t, K, N)
    q = _c(q, np.int8)
    d = _c(d, np.uint16)
    M = q.shape[0]
    n1 = N if n1 is None else min(n1, N)
    lut = None if lut is None else _c(lut, np.int8)
    y = np.zeros((M, N), np.float64)
    acond = np.zeros((M, N), np.float64)
    lib().or_matmul_flat(t, _p(flat), K, N, _p(q), _p(d), M, _p(lut), n0, n1, _p(y), _p(acond), N)
    return y, acond



def e4m3_value(code):
    """Value of an OCP FP8 E4M3 code (0x7F / 0xFF, NaN, excluded)."""
    return lib().or_e4m3_value(int(code))


def quantize_act_mx(x, dtype=F32, K=None):
    """MXFP8 activations: x [M, K] float32 (F32) or uint16 bits (BF16 / F16).

    Returns (q uint8 E4M3 codes [M,K], e uint8 E8M0 scales [M,K/32])."""
    x = np.ascontiguousarray(x, dtype=np.float32 if dtype == F32 else np.uint16)
    M, Kx = x.shape
    K = Kx if K is None else K
    q = np.zeros((M, K), np.uint8)
    e = np.zeros((M, K // 32), np.uint8)
    lib().or_quantize_act_mx(dtype, _p(x), M, K, Kx, _p(q), _p(e))
    return q, e


def matmul_mx(tiles, K, N, q, e, n0=0, n1=None):
    """MXFP4 tiles x MXFP8 activations: y[m, n] (fp64) and acond[m, n] =
    sum |W*A| for n0 <= n < n1."""
    tiles = _c(tiles, np.uint8)
    q = _c(q, np.uint8)
    e = _c(e, np.uint8)
    M = q.shape[0]
    n1 = N if n1 is None else min(n1, N)
    y = np.zeros((M, N), np.float64)
    acond = np.zeros((M, N), np.float64)
    lib().or_matmul_mx(_p(tiles), K, N, _p(q), _p(e), M, n0, n1, _p(y), _p(acond), N)
    return y, acond
