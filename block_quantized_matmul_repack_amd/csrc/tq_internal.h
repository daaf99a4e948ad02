// Internal declarations of the tiledq HIP library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tiledq.h"

namespace tq {

// Tile geometry ("Block-32 Quantized Formats"): quant bytes, then 32 row
// scales at scale_off: fp16 at scale_off + 2*row, for MXFP4 one E8M0 byte at
// scale_off + row, for Q4_1 the fp16 pair (d, m) at scale_off + 4*row.
// block = bytes of one flat GGML block.
template <int QT> struct Fmt;
template <> struct Fmt<TQ_Q4_0> {
    static constexpr int tile = 576, scale_off = 512, block = 18;
};
template <> struct Fmt<TQ_IQ4_NL> {
    static constexpr int tile = 576, scale_off = 512, block = 18;
};
template <> struct Fmt<TQ_Q8_0> {
    static constexpr int tile = 1088, scale_off = 1024, block = 34;
};
template <> struct Fmt<TQ_MXFP4> {
    static constexpr int tile = 544, scale_off = 512, block = 17;
};
template <> struct Fmt<TQ_Q4_1> {
    static constexpr int tile = 640, scale_off = 512, block = 20;
};
// Q4_K: Q4_1 tiles; `block` is one 256-element flat super-block
template <> struct Fmt<TQ_Q4_K> {
    static constexpr int tile = 640, scale_off = 512, block = 144;
};

// Raw buffer loads (CDNA buffer resource descriptor, stride 0): a load whose
// byte offset lies outside [0, bytes) returns zero, so out-of-range operands
// are zeroed without branches and every path issues the same loads.  The
// offset checked is the whole one, vector plus scalar operand, and a load of
// several dwords is checked dword by dword: a dword with any byte at or past
// `bytes` reads zero, the dwords wholly inside are returned (checked on
// gfx950).  Ranges stay below 2^31 bytes; BUF_OOB is an offset past all of
// them.
constexpr int64_t BUF_MAX_BYTES = 0x7E000000;
constexpr int BUF_OOB = 0x7F000000;  // + any in-tile offset stays positive
constexpr int BUF_NT = 2;                 // aux bits: nontemporal (stream past the caches)

// `base` and `bytes` must be the same in every lane of the wave (they are
// read from the first active lane so the descriptor lives in scalar registers).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes)
{
    const int64_t n = bytes < 0 ? 0 : (bytes < BUF_MAX_BYTES ? bytes : BUF_MAX_BYTES);
    const uint64_t a = (uint64_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const int nr = __builtin_amdgcn_readfirstlane((int)n);
    // descriptor word 3: 32-bit data format, required by gfx9-family raw buffers
    return __builtin_amdgcn_make_buffer_rsrc((void *)(((uint64_t)hi << 32) | lo), (short)0, nr,
                                             0x00020000);
}

// 16-entry int8 table of a 4-bit type (IQ4_NL: the caller's; MXFP4: 2 *
// E2M1) as four little-endian dwords (entries 4i..4i+3 in dword i).
struct Lut {
    uint32_t w[4];
};

__device__ __forceinline__ float f16_bits_to_f32(uint16_t b)
{
    return (float)__builtin_bit_cast(_Float16, b);
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float f)
{
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// fp16 bits of the product a * b, formed in fp32 and rounded once to nearest
// even, with IEEE signed zeros.  The empty asm keeps the product an fp32
// value: otherwise the compiler fuses multiply and conversion into a mixed
// fma with a +0 addend (v_fma_mixlo_f16), which turns a -0 product into +0.
__device__ __forceinline__ uint16_t f16_of_product(float a, float b)
{
    float p = a * b;
    asm volatile("" : "+v"(p));
    return f32_to_f16_bits(p);
}

// Eight consecutive activation elements of dtype DT from index i, converted
// exactly to fp32.  x needs only element alignment: the wide loads are
// unaligned-capable on this target.
typedef float f32x4u __attribute__((ext_vector_type(4), aligned(4)));
typedef uint16_t u16x8u __attribute__((ext_vector_type(8), aligned(2)));
template <int DT>
__device__ __forceinline__ void load_x8(float (&v)[8], const void *x, int64_t i)
{
    if constexpr (DT == TQ_F32) {
        const f32x4u a = *(const f32x4u *)((const float *)x + i);
        const f32x4u b = *(const f32x4u *)((const float *)x + i + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
        const u16x8u h = *(const u16x8u *)((const uint16_t *)x + i);
#pragma unroll
        for (int e = 0; e < 8; e++) {
            if constexpr (DT == TQ_BF16)
                v[e] = __builtin_bit_cast(float, (uint32_t)h[e] << 16);
            else
                v[e] = f16_bits_to_f32(h[e]);
        }
    }
}

// Max over the 4 lanes of a quad (DPP quad permutations, no LDS).
__device__ __forceinline__ float quad_max(float v)
{
    const int b = __builtin_bit_cast(int, v);
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, b, 0xB1, 0xF, 0xF, true)));
    const int c = __builtin_bit_cast(int, v);
    return fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, c, 0x4E, 0xF, 0xF, true)));
}

// MXFP4 ("MXFP4", Dequantization): the E8M0 row byte e as the fp16 power of
// two whose exponent bits are clamp(e - 112, 0, 30) (field 0: +0.0).
__device__ __forceinline__ uint16_t e8m0_f16_bits(uint32_t e)
{
    return (uint16_t)(min(max((int)e - 112, 0), 30) << 10);
}

// fp16 bits of tile row l's scale, read from the tile (LDS or global).
template <int QT>
__device__ __forceinline__ uint16_t tile_scale_bits(const uint8_t *tile, int l)
{
    if constexpr (QT == TQ_MXFP4)
        return e8m0_f16_bits(tile[Fmt<QT>::scale_off + l]);
    else if constexpr (QT == TQ_Q4_1)
        return ((const uint16_t *)(tile + Fmt<QT>::scale_off))[2 * l];
    else
        return ((const uint16_t *)(tile + Fmt<QT>::scale_off))[l];
}

// fp16 bits of tile row l's min (Q4_1 only).
__device__ __forceinline__ uint16_t tile_min_bits(const uint8_t *tile, int l)
{
    return ((const uint16_t *)(tile + Fmt<TQ_Q4_1>::scale_off))[2 * l + 1];
}

// acc + the sum of the 4 int8 of a (activation block sums for Q4_1's min).
__device__ __forceinline__ int byte_sum(uint32_t a, int acc)
{
    return __builtin_amdgcn_sdot4((int)a, 0x01010101, acc, false);
}

// The kernels multiply integer weights that are a fixed power of two times
// the format's: Q4_0 as 16 (code - 8) (the nibble in the high half of a
// byte), MXFP4 as 2 * E2M1 (integers).  This factor undoes it, exactly.
template <int QT>
constexpr float weight_unscale()
{
    return QT == TQ_Q4_0 ? 0.0625f : (QT == TQ_MXFP4 ? 0.5f : 1.0f);
}

// Dynamic activation quantization of one 32-element K block ("Memory
// buffers": dynamically quantized activations; used as Q8_0 activation
// tiles): d = amax / 127 (IEEE fp32 divide), q = round-half-away-from-zero(
// v * (1 / d)), the scale stored as fp16 nearest-even.  The block is held by
// a quad of lanes, lane c holding elements 8c..8c+7; every lane of the quad
// must be active.  Returns this lane's 8 int8 codes (element 8c + e in byte
// e) and, in every lane, the fp16 scale bits.  Every kernel that quantizes
// activations calls this, so they all produce the same bits.
//
// Rounding half away from zero is done as a truncating conversion of y +
// copysign(0.5 - 2^-25, y), the addition in fp32: the two agree for every
// fp32 |y| < 2^23 (tests/test_host_rounding.py checks every value below 256);
// here |y| <= 127.  The product y
// must be rounded on its own, so contraction into a fused multiply-add is
// off in this function.
__device__ __forceinline__ void quant_quad(const float (&v)[8], uint2 &q, uint16_t &dbits)
{
#pragma clang fp contract(off)
    float amax = fabsf(v[0]);
#pragma unroll
    for (int e = 1; e < 8; e++)
        amax = fmaxf(amax, fabsf(v[e]));
    amax = quad_max(amax);
    const float dd = amax / 127.0f;
    const float id = (dd != 0.0f) ? 1.0f / dd : 0.0f;
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; e++) {
        const float y = v[e] * id;
        const int c = (int)(y + copysignf(0.49999997f, y));
        w[e >> 2] |= ((uint32_t)c & 0xFFu) << (8 * (e & 3));
    }
    q = make_uint2(w[0], w[1]);
    dbits = f32_to_f16_bits(dd);
}

typedef uint32_t u32x2u __attribute__((ext_vector_type(2), aligned(4)));

// 0xFF in each byte of v whose bit 7 is set, else 0x00: v_perm_b32's sign
// selectors (8, 9: bits 15, 31 of the second operand; 10, 11: of the first)
// read bytes 1 and 3 only, so v << 8 brings bytes 0 and 2 there.
__device__ __forceinline__ uint32_t byte_sign_mask(uint32_t v)
{
    return __builtin_amdgcn_perm(v, v << 8, 0x0B090A08u);
}

// Table lookups of the 8 nibbles of x at once: ev gets the int8 table entries
// of the low nibbles (byte b: entry of bits 4b..4b+3), od those of the high
// nibbles.  v_perm_b32 picks any byte of an 8-byte pair, so each half of the
// table is looked up with the nibble's low 3 bits and the two results are
// merged on its bit 3 (bit 7 of the byte for a high nibble, bit 3 shifted
// there for a low one).  14 VALU operations for 8 lookups.
__device__ __forceinline__ void lut16x2(uint32_t x, const Lut &t, uint32_t &ev, uint32_t &od)
{
    const uint32_t se = x & 0x07070707u;
    const uint32_t so = (x >> 4) & 0x07070707u;
    const uint32_t me = byte_sign_mask(x << 4);
    const uint32_t mo = byte_sign_mask(x);
    const uint32_t le = __builtin_amdgcn_perm(t.w[1], t.w[0], se);
    const uint32_t he = __builtin_amdgcn_perm(t.w[3], t.w[2], se);
    const uint32_t lo = __builtin_amdgcn_perm(t.w[1], t.w[0], so);
    const uint32_t ho = __builtin_amdgcn_perm(t.w[3], t.w[2], so);
    ev = (he & me) | (le & ~me);
    od = (ho & mo) | (lo & ~mo);
}

// The MXFP4 block at byte a of the flat buffer (total bytes long): its E8M0
// byte and its 8 quant halfwords.  The 5 covering dwords start at a & ~3;
// the first four end before a + 16, inside the block; the fifth can pass the
// end of the buffer only for its last block, and is then read bytewise.
__device__ __forceinline__ void load_mx_block(const uint8_t *__restrict__ flat, int64_t a,
                                              int64_t total, uint16_t (&q)[8], uint16_t &e)
{
    const int64_t A = a & ~int64_t(3);
    const int sh = (int)(a - A);
    uint32_t w[5];
#pragma unroll
    for (int i = 0; i < 4; i++)
        w[i] = *(const uint32_t *)(flat + A + 4 * i);
    if (A + 20 <= total) {
        w[4] = *(const uint32_t *)(flat + A + 16);
    } else {
        w[4] = 0;
        for (int j = 0; j < 4 && A + 16 + j < total; j++)
            w[4] |= (uint32_t)flat[A + 16 + j] << (8 * j);
    }
    e = (uint16_t)((w[0] >> (8 * sh)) & 0xFFu);
    const int s1 = 8 * (sh + 1);                  // quants start 1..4 bytes into w[0]
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const uint32_t v = (uint32_t)((((uint64_t)w[k + 1] << 32) | w[k]) >> s1);
        q[2 * k] = (uint16_t)v;
        q[2 * k + 1] = (uint16_t)(v >> 16);
    }
}

// Q4_K: 6-bit scale and min of sub-block j from the 12 scale bytes (three
// dwords), as the repack decodes them (Q4_K layout in tiledq.h).
__device__ __forceinline__ void q4k_scale_min(const uint32_t (&s3)[3], int j, uint32_t &sc,
                                              uint32_t &m)
{
    auto sb = [&](int k) {
        const uint32_t v = k < 4 ? s3[0] : (k < 8 ? s3[1] : s3[2]);
        return (v >> (8 * (k & 3))) & 0xFFu;
    };
    if (j < 4) {
        sc = sb(j) & 63u;
        m = sb(j + 4) & 63u;
    } else {
        sc = (sb(j + 4) & 15u) | ((sb(j - 4) >> 6) << 4);
        m = (sb(j + 4) >> 4) | ((sb(j) >> 6) << 4);
    }
}

// A dispatch counts work-items in 32 bits per grid dimension.  The shape
// limits of the entry points keep every grid of the library below 2^31
// work-items; each launcher still checks its grid (`blocks` workgroups of
// `threads`) before converting it, and refuses an oversized one.
inline bool grid_fits(int64_t blocks, int threads)
{
    return blocks >= 0 && blocks * threads < (int64_t(1) << 32);
}

// K-split of the decode GEMV: S workgroups per stripe (a power of two),
// `chunk` k-tiles each; slots points into the caller's workspace when S > 1.
struct Split {
    int S, chunk;
    uint64_t *slots;
};
Split gemv_split(int64_t K, int64_t N);
size_t gemv_workspace_bytes(int64_t K, int64_t N, int64_t M);

hipError_t launch_repack(int type, const void *flat, int64_t K, int64_t N, void *tiles,
                         hipStream_t s);
hipError_t launch_quantize(int dtype, const void *x, int64_t M, int64_t K, int64_t ldx,
                           int8_t *q, uint16_t *d, hipStream_t s);
// Activations of the decode GEMV: either quantized already (q, d) or raw
// (x of dtype xt, row stride ldx, quantized inside the GEMV kernel).
struct Act {
    const int8_t *q;
    const uint16_t *d;
    const void *x;
    int xt;          // -1: use q, d
    int64_t ldx;
};

hipError_t launch_qgemv(int type, const void *tiles, int64_t K, int64_t N, const Act &act,
                        int64_t M, const Lut &lut, float *y, int64_t ldy, int32_t *isum,
                        void *ws, size_t ws_bytes, hipStream_t s);
hipError_t launch_qgemm(int type, const void *tiles, int64_t K, int64_t N, const int8_t *q,
                        const uint16_t *d, int64_t M, const Lut &lut, float *y, int64_t ldy,
                        int32_t *isum, hipStream_t s);
// The GEMM with K split into S ranges (S >= 2), for output grids too small
// to fill the chip: partial planes of M x N fp32 in part (S * M * N floats),
// then summed in a fixed order into y.
hipError_t launch_qgemm_split(int type, const void *tiles, int64_t K, int64_t N, const int8_t *q,
                              const uint16_t *d, int64_t M, const Lut &lut, float *y, int64_t ldy,
                              int S, float *part, hipStream_t s);
// y[m * ldy + n] = the sum of S partial planes (M x N fp32 each, contiguous
// in part) in the order 0, 1, ..., S - 1.
hipError_t launch_sum_planes(const float *part, int64_t M, int64_t N, int S, float *y,
                             int64_t ldy, hipStream_t s);
// Flat (un-repacked) GGML blocks: unpack of tiles, and the two products.
hipError_t launch_unpack(int type, const void *tiles, int64_t K, int64_t N, void *flat,
                         hipStream_t s);
hipError_t launch_qgemv_flat(int type, const void *flat, int64_t K, int64_t N, const int8_t *q,
                             const uint16_t *d, int64_t M, const Lut &lut, float *y,
                             int64_t ldy, int32_t *isum, hipStream_t s);
hipError_t launch_qgemm_flat(int type, const void *flat, int64_t K, int64_t N, const int8_t *q,
                             const uint16_t *d, int64_t M, const Lut &lut, float *y,
                             int64_t ldy, int32_t *isum, hipStream_t s);
// MXFP4 tiles x MXFP8 activations on the block-scaled matrix cores.
hipError_t launch_quantize_mx(int dtype, const void *x, int64_t M, int64_t K, int64_t ldx,
                              uint8_t *q, uint8_t *e, hipStream_t s);
// S >= 2 splits K into S ranges, their partial planes in part (S * M * N
// floats), summed into y as launch_sum_planes.
hipError_t launch_qgemm_mx(const void *tiles, int64_t K, int64_t N, const uint8_t *q,
                           const uint8_t *e, int64_t M, float *y, int64_t ldy, int S, float *part,
                           hipStream_t s);

}  // namespace tq
