// Internal declarations of the tiledq HIP library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tiledq.h"

namespace tq {

// Tile geometry ("Block-32 Quantized Formats"): quant bytes, then 32 fp16
// row scales at scale_off + 2*row.
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

// IQ4_NL table as four little-endian dwords (entries 4i..4i+3 in dword i).
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

// 4 table lookups at once: idx holds four byte indices 0..15; returns the four
// int8 table entries in the same byte positions.  v_perm_b32 selects any byte
// of an 8-byte pair, so the two table halves are looked up separately and
// merged on bit 3 of each index.
__device__ __forceinline__ uint32_t lut16(uint32_t idx, const Lut &t)
{
    uint32_t sel = idx & 0x07070707u;
    uint32_t lo = __builtin_amdgcn_perm(t.w[1], t.w[0], sel);
    uint32_t hi = __builtin_amdgcn_perm(t.w[3], t.w[2], sel);
    uint32_t m = ((idx >> 3) & 0x01010101u) * 0xFFu;
    return (hi & m) | (lo & ~m);
}

hipError_t launch_repack(int type, const void *flat, int64_t K, int64_t N, void *tiles,
                         hipStream_t s);
hipError_t launch_quantize(int dtype, const void *x, int64_t M, int64_t K, int64_t ldx,
                           int8_t *q, uint16_t *d, hipStream_t s);
hipError_t launch_qgemv(int type, const void *tiles, int64_t K, int64_t N, const int8_t *q,
                        const uint16_t *d, int64_t M, const Lut &lut, float *y, int64_t ldy,
                        int32_t *isum, hipStream_t s);
hipError_t launch_qgemm(int type, const void *tiles, int64_t K, int64_t N, const int8_t *q,
                        const uint16_t *d, int64_t M, const Lut &lut, float *y, int64_t ldy,
                        int32_t *isum, hipStream_t s);

}  // namespace tq
