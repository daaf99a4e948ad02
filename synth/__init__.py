"""Seeded synthetic inputs for tiled block-32 quantized matmul.

This module only draws random numbers and lays them out in the flat GGML
block-32 source format; it holds none of the method's arithmetic (no repack,
no activation quantization, no dot products).  Both the CPU oracle tests and
the HIP path's tests and benchmark take their inputs from here.

Generator: numpy.random.default_rng(seed) (PCG64).  Draw order per workload:
weight codes, then weight scales, then activations.

Flat layout written here (GGML block-32, little-endian): row n holds K/32
consecutive blocks; a Q4_0 / IQ4_NL block is 2 bytes of fp16 scale followed by
16 bytes whose low nibbles are elements 0..15 and high nibbles elements
16..31; a Q8_0 block is 2 bytes of fp16 scale followed by 32 int8 elements;
an MXFP4 block is 1 byte of E8M0 scale followed by 16 nibble bytes ordered
as in Q4_0; a Q4_1 block is 2 bytes of fp16 scale d, 2 bytes of fp16 min m,
then 16 nibble bytes ordered as in Q4_0.  A Q4_K super-block (256 elements)
is fp16 d, fp16 dmin, 12 bytes packing eight 6-bit scales and eight 6-bit
mins, then 128 bytes in which 64-element chunk c owns bytes 32c..32c+31
(element 64c + i in the low nibble of byte 32c + i, element 64c + 32 + i in
its high nibble).
"""
import collections
import dataclasses

import numpy as np

Q4_0, Q8_0, IQ4_NL, MXFP4, Q4_1, Q4_K = 0, 1, 2, 3, 4, 5
TYPE_NAMES = {Q4_0: "q4_0", Q8_0: "q8_0", IQ4_NL: "iq4_nl", MXFP4: "mxfp4", Q4_1: "q4_1",
              Q4_K: "q4_k"}
BLOCK_BYTES = {Q4_0: 18, Q8_0: 34, IQ4_NL: 18, MXFP4: 17, Q4_1: 20, Q4_K: 144}
BLOCK_ELEMS = {Q4_K: 256}          # elements per flat block; 32 for the others
TILE_BYTES = {Q4_0: 576, Q8_0: 1088, IQ4_NL: 576, MXFP4: 544, Q4_1: 640, Q4_K: 640}

# Q4_K super-block parameters: fp16 bits of d and dmin [N, K/256], 6-bit
# scale and min of each 32-element sub-block [N, K/32].
Q4KScales = collections.namedtuple("Q4KScales", "d dmin sc m")

# Stand-in for the 16-entry non-linear IQ4_NL table.  The page names the table
# but does not print its values; any 16 int8 entries keep the integer path
# exact.  These are round(127 * sign(u) * |u|**1.5) for u = (2i - 15) / 15,
# a symmetric, denser-near-zero codebook of our own construction.
IQ4_NL_STANDIN_LUT = np.array(
    [-127, -102, -80, -59, -40, -24, -11, -2, 2, 11, 24, 40, 59, 80, 102, 127],
    dtype=np.int8)


def _standin_lut_formula():
    u = (2 * np.arange(16) - 15) / 15.0
    v = 127.0 * np.sign(u) * np.abs(u) ** 1.5
    return (np.sign(v) * np.floor(np.abs(v) + 0.5)).astype(np.int8)


assert np.array_equal(_standin_lut_formula(), IQ4_NL_STANDIN_LUT)


def draw_codes(rng, qtype, N, K):
    """Weight codes [N, K]: 0..15 (Q4_0, IQ4_NL) or int8 in [-127, 127] (Q8_0)."""
    if qtype == Q8_0:
        return rng.integers(-127, 128, size=(N, K), dtype=np.int8)
    return rng.integers(0, 16, size=(N, K), dtype=np.uint8)


def draw_scales(rng, dist, N, K):
    """Scale bits [N, K/32] (uint16).  dist: 'uniform' -> fp16 of U[1e-3, 1e-2);
    'absnormal' -> fp16 of |N(0,1)| * 0.01 (drawn in float64, cast to float32,
    then to fp16 by numpy, round to nearest even); 'e8m0' -> MXFP4 E8M0 bytes
    uniform in [118, 124], power-of-two scales 2^-9 .. 2^-3 (with E2M1 values
    up to 6, weights of magnitude up to about 0.75); 'minmax' -> Q4_1 pairs
    [N, K/32, 2]: d = fp16 of U[1e-3, 1e-2), m = fp16 of -d * U[6, 10] (a
    block min below zero, codes 0..15 spanning [m, m + 15 d]); 'q4k' -> a
    Q4KScales of d, dmin = fp16 of U[1e-4, 1e-3) per super-block and 6-bit
    scales and mins uniform 0..63 per sub-block; 'edge' -> fp16 scale bits
    mixing +0, subnormals, the smallest normals, U[1e-3, 1e-2) and 1..8."""
    shape = (N, K // 32)
    if dist == "e8m0":
        return rng.integers(118, 125, size=shape).astype(np.uint16)
    if dist == "q4k":
        nsb = K // 256
        d = rng.uniform(1e-4, 1e-3, size=(N, nsb)).astype(np.float32).astype(np.float16)
        dmin = rng.uniform(1e-4, 1e-3, size=(N, nsb)).astype(np.float32).astype(np.float16)
        sc = rng.integers(0, 64, size=shape).astype(np.uint8)
        m = rng.integers(0, 64, size=shape).astype(np.uint8)
        return Q4KScales(d.view(np.uint16), dmin.view(np.uint16), sc, m)
    if dist == "minmax":
        d = rng.uniform(1e-3, 1e-2, size=shape)
        m = -d * rng.uniform(6.0, 10.0, size=shape)
        pair = np.stack([d, m], axis=-1)
        return pair.astype(np.float32).astype(np.float16).view(np.uint16)
    if dist == "edge":
        # fp16 scale bits at the ends of the range: +0, subnormals (bits
        # 1..1023), the smallest normals (1024..1279), U[1e-3, 1e-2), and
        # magnitudes 1..8
        kind = rng.integers(0, 5, size=shape)
        b = np.where(kind == 0, 0, 0).astype(np.int64)
        b = np.where(kind == 1, rng.integers(1, 1024, size=shape), b)
        b = np.where(kind == 2, rng.integers(1024, 1280, size=shape), b)
        mid = rng.uniform(1e-3, 1e-2, size=shape).astype(np.float32).astype(np.float16)
        big = rng.uniform(1.0, 8.0, size=shape).astype(np.float32).astype(np.float16)
        b = np.where(kind == 3, mid.view(np.uint16).astype(np.int64), b)
        b = np.where(kind == 4, big.view(np.uint16).astype(np.int64), b)
        return b.astype(np.uint16)
    if dist == "uniform":
        s = rng.uniform(1e-3, 1e-2, size=shape)
    elif dist == "absnormal":
        s = np.abs(rng.standard_normal(size=shape)) * 0.01
    else:
        raise ValueError(dist)
    return s.astype(np.float32).astype(np.float16).view(np.uint16)


def _pack_q4k(codes, p):
    """GGML Q4_K super-blocks from codes [N, K] and a Q4KScales."""
    N, K = codes.shape
    nsb = K // 256
    out = np.zeros((N, nsb, 144), np.uint8)
    d = np.ascontiguousarray(p.d, dtype=np.uint16).reshape(N, nsb)
    dmin = np.ascontiguousarray(p.dmin, dtype=np.uint16).reshape(N, nsb)
    out[:, :, 0], out[:, :, 1] = d & 0xFF, d >> 8
    out[:, :, 2], out[:, :, 3] = dmin & 0xFF, dmin >> 8
    sc = np.asarray(p.sc, dtype=np.uint8).reshape(N, nsb, 8)
    m = np.asarray(p.m, dtype=np.uint8).reshape(N, nsb, 8)
    sb = out[:, :, 4:16]
    for j in range(8):
        if j < 4:
            sb[:, :, j] |= sc[:, :, j]
            sb[:, :, j + 4] |= m[:, :, j]
        else:
            sb[:, :, j + 4] = (sc[:, :, j] & 0xF) | ((m[:, :, j] & 0xF) << 4)
            sb[:, :, j - 4] |= (sc[:, :, j] >> 4) << 6
            sb[:, :, j] |= (m[:, :, j] >> 4) << 6
    c = codes.astype(np.uint8).reshape(N, nsb, 4, 64)
    out[:, :, 16:] = (c[:, :, :, :32] | (c[:, :, :, 32:] << 4)).reshape(N, nsb, 128)
    return out.reshape(-1)


def pack_flat(qtype, codes, scale_bits):
    """Write codes [N, K] and scale bits [N, K/32] (fp16, E8M0 bytes for
    MXFP4, [N, K/32, 2] fp16 (d, m) pairs for Q4_1, a Q4KScales for Q4_K) as
    flat GGML blocks."""
    if qtype == Q4_K:
        return _pack_q4k(codes, scale_bits)
    N, K = codes.shape
    nb = K // 32
    bb = BLOCK_BYTES[qtype]
    ns = 2 if qtype == Q4_1 else 1
    out = np.empty((N, nb, bb), np.uint8)
    sb = np.ascontiguousarray(scale_bits, dtype=np.uint16).reshape(N, nb, ns)
    for i in range(ns):
        out[:, :, 2 * i] = (sb[:, :, i] & 0xFF).astype(np.uint8)
        if qtype != MXFP4:
            out[:, :, 2 * i + 1] = (sb[:, :, i] >> 8).astype(np.uint8)
    q0 = {MXFP4: 1, Q4_1: 4}.get(qtype, 2)
    c = codes.reshape(N, nb, 32)
    if qtype == Q8_0:
        out[:, :, q0:] = c.view(np.uint8)
    else:
        c = c.astype(np.uint8)
        out[:, :, q0:] = c[:, :, :16] | (c[:, :, 16:] << 4)
    return out.reshape(-1)


def draw_activations(rng, M, K, dtype="f32"):
    """Activations N(0,1) [M, K]: float32, or bf16 / fp16 bit patterns (uint16)
    rounded to nearest even from the float32 draw."""
    x = rng.standard_normal(size=(M, K), dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        u = x.view(np.uint32).astype(np.uint64)
        # round to nearest even on the upper 16 bits (finite inputs only)
        r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
        return r.astype(np.uint16)
    raise ValueError(dtype)


@dataclasses.dataclass
class Workload:
    name: str
    qtype: int
    K: int
    N: int
    M: int
    scale_dist: str
    act_dtype: str = "f32"
    seed: int = 0
    path: str = "qgemv"     # qgemv (M <= 8) or qgemm

    @property
    def n_col_tiles(self):
        return (self.N + 31) // 32

    @property
    def tile_bytes(self):
        return TILE_BYTES[self.qtype]

    @property
    def weight_bytes(self):
        return (self.K // 32) * self.n_col_tiles * self.tile_bytes


@dataclasses.dataclass
class Inputs:
    codes: np.ndarray
    scale_bits: np.ndarray
    flat: np.ndarray
    x: np.ndarray
    lut: np.ndarray


def make_inputs(w: Workload, M=None):
    """Draw one workload's inputs: codes, then scales, then activations."""
    rng = np.random.default_rng(w.seed)
    codes = draw_codes(rng, w.qtype, w.N, w.K)
    sb = draw_scales(rng, w.scale_dist, w.N, w.K)
    flat = pack_flat(w.qtype, codes, sb)
    x = draw_activations(rng, w.M if M is None else M, w.K, w.act_dtype)
    return Inputs(codes, sb, flat, x, IQ4_NL_STANDIN_LUT.copy())


# The synthetic workloads: shapes and value distributions of the pages'
# setting (a Q4_0 FFN up-projection 4096 -> 14336, a 128001-entry lm-head).
WORKLOADS = {
    "q4_0_gemv_k256_n64_m1": Workload("q4_0_gemv_k256_n64_m1", Q4_0, 256, 64, 1, "uniform"),
    "q8_0_gemv_k4096_n4096_m1": Workload("q8_0_gemv_k4096_n4096_m1", Q8_0, 4096, 4096, 1, "absnormal"),
    "q4_0_gemv_k4096_n14336_m1": Workload("q4_0_gemv_k4096_n14336_m1", Q4_0, 4096, 14336, 1, "uniform"),
    "q4_0_gemv_k4096_n14336_m4": Workload("q4_0_gemv_k4096_n14336_m4", Q4_0, 4096, 14336, 4, "uniform"),
    "q4_0_gemv_k4096_n14336_m8": Workload("q4_0_gemv_k4096_n14336_m8", Q4_0, 4096, 14336, 8, "uniform"),
    "iq4_nl_gemm_m512_k4096_n4096": Workload("iq4_nl_gemm_m512_k4096_n4096", IQ4_NL, 4096, 4096, 512,
                                             "uniform", act_dtype="bf16", path="qgemm"),
    "q8_0_lmhead_k4096_n128001_m1": Workload("q8_0_lmhead_k4096_n128001_m1", Q8_0, 4096, 128001, 1, "absnormal"),
    "q8_0_lmhead_k4096_n128001_m128": Workload("q8_0_lmhead_k4096_n128001_m128", Q8_0, 4096, 128001, 128,
                                               "absnormal", path="qgemm"),
    "mxfp4_gemv_k4096_n14336_m1": Workload("mxfp4_gemv_k4096_n14336_m1", MXFP4, 4096, 14336, 1, "e8m0"),
    "mxfp4_gemm_m512_k4096_n4096": Workload("mxfp4_gemm_m512_k4096_n4096", MXFP4, 4096, 4096, 512,
                                            "e8m0", act_dtype="bf16", path="qgemm"),
    "q4_1_gemv_k4096_n14336_m1": Workload("q4_1_gemv_k4096_n14336_m1", Q4_1, 4096, 14336, 1, "minmax"),
    "q4_1_gemm_m512_k4096_n4096": Workload("q4_1_gemm_m512_k4096_n4096", Q4_1, 4096, 4096, 512,
                                           "minmax", act_dtype="bf16", path="qgemm"),
    "q4_k_gemv_k4096_n14336_m1": Workload("q4_k_gemv_k4096_n14336_m1", Q4_K, 4096, 14336, 1, "q4k"),
}


# ---------------------------------------------------------------------------
# Edge-case inputs: the ends of the documented domains.  Like everything in
# this module they are draws and constants only; no quantization arithmetic.

# Block maxima |x| for the activation edge cases, per input dtype.  f32 and
# bf16 share fp32's exponent range: the domain's lower end 2^-120 and just
# above it, the amax whose d = amax/127 is the smallest normal fp32
# (127 * 2^-126) and one just below (a subnormal fp32 d), maxima whose fp16 d
# is near the fp16 normal / subnormal boundary (about 7.75e-3), an fp16
# subnormal d (1e-5) and one that rounds to +0 (3e-6), plain magnitudes, and
# the domain's upper end 65504 * 127.  fp16 inputs cannot go below 2^-24 or
# above 65504.
EDGE_AMAX = {
    "f32": [2.0 ** -120, 2.0 ** -119, 127 * 2.0 ** -126, 126 * 2.0 ** -126, 7.75e-3, 7e-3,
            1e-5, 3e-6, 1.0, 3.5, 65504.0 * 127],
    "bf16": [2.0 ** -120, 2.0 ** -119, 127 * 2.0 ** -126, 126 * 2.0 ** -126, 7.75e-3, 7e-3,
             1e-5, 3e-6, 1.0, 3.5, 65280.0 * 127],
    "f16": [2.0 ** -24, 2.0 ** -20, 6.1e-5, 7.75e-3, 7e-3, 1e-5, 3e-6, 1.0, 3.5, 65504.0],
}


def _round_bf16_bits(x):
    u = x.astype(np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def draw_edge_activations(rng, M, K, dtype="f32"):
    """Activations [M, K] (float32, or bf16 / fp16 bit patterns) built block
    by block to reach the quantizer's edges.  Each 32-element block is one
    of: a maximum from EDGE_AMAX[dtype] placed on one element (random sign)
    with the others uniform in (-amax, amax) -- which puts fp32 / bf16 / fp16
    subnormal elements into the tiny-maximum blocks; a block with some
    elements below the fp32 normal range (f32 / bf16: |x| < 2^-126) beside a
    maximum of 2^-118; an all-zero block (signed zeros); a constant block
    +c or -c (every code +-127: with weights of -128 the integer dot reaches
    its extreme 32 * 128 * 127); exact half-way products (x = (k + 1/2) *
    amax / 127 with amax = 127, where x / d is k + 1/2 exactly); or N(0,1).
    The kind of block b of row m is (m * 7 + b) mod the number of kinds, so
    every row and every K range see them all."""
    amaxes = EDGE_AMAX[dtype]
    kinds = len(amaxes) + 5
    nb = K // 32
    x = np.zeros((M, K), dtype=np.float64)
    for m in range(M):
        for b in range(nb):
            k = (m * 7 + b) % kinds
            blk = np.zeros(32)
            if k < len(amaxes):
                a = amaxes[k]
                blk = rng.uniform(-a, a, size=32)
                blk[rng.integers(0, 32)] = a * (1 if rng.integers(0, 2) else -1)
            elif k == len(amaxes):
                if dtype == "f16":
                    blk = rng.integers(-1023, 1024, size=32) * 2.0 ** -24   # fp16 subnormals
                    blk[rng.integers(0, 32)] = 2.0 ** -14
                else:
                    blk = rng.uniform(-1, 1, size=32) * 2.0 ** -130          # fp32 subnormals
                    blk[rng.integers(0, 32)] = -(2.0 ** -118)
            elif k == len(amaxes) + 1:
                blk = np.where(rng.integers(0, 2, size=32) == 1, 0.0, -0.0)
            elif k == len(amaxes) + 2:
                c = float(rng.uniform(0.1, 2.0)) * (1 if (m + b) % 2 else -1)
                blk[:] = c
            elif k == len(amaxes) + 3:
                # amax = 127 on one element, so d = 1 and x / d = x exactly;
                # the others sit on exact halves k + 1/2
                blk = rng.integers(-126, 126, size=32) + 0.5
                blk[rng.integers(0, 32)] = 127.0 * (1 if rng.integers(0, 2) else -1)
            else:
                blk = rng.standard_normal(32)
            x[m, 32 * b:32 * b + 32] = blk
    if dtype == "f32":
        return x.astype(np.float32)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    return _round_bf16_bits(x)


def draw_codes_q8_full(rng, N, K):
    """Q8_0 codes [N, K] over the whole int8 range [-128, 127], with -128
    planted: every third row is all -128, every other block of the other rows
    holds -128 in half its elements, and the rest is uniform in [-128, 127]."""
    c = rng.integers(-128, 128, size=(N, K), dtype=np.int16)
    for n in range(N):
        if n % 3 == 0:
            c[n, :] = -128
        else:
            for b in range(0, K // 32, 2):
                sel = rng.permutation(32)[:16]
                c[n, 32 * b + sel] = -128
    return c.astype(np.int8)
