// Unpack 32x32 tiles back into flat GGML blocks: the inverse of the repack
// ("Tiled Weight Formats"; tensors also exist flat, "supports_op
// Independence from Buffer and Repack State").  Rows n >= N (the padding of
// the last stripe) are dropped.  Q4_K is not invertible (its tiles keep the
// products d * sc and -dmin * m, not the super-block's fields) and is
// rejected by the caller.
//
// One workgroup takes one 32-row stripe and KT consecutive k-tiles: the
// tiles (contiguous) are copied to LDS with 16-byte loads, then each work
// item assembles one flat block (row r, tile t) from LDS bytes:
//   4-bit: flat byte 2h = low nibbles of tile bytes (h, r) and (h + 8, r),
//          flat byte 2h + 1 = their high nibbles (elements 2h, 2h + 1 of the
//          tile's column pair h; elements 2h + 16, 2h + 17 of pair h + 8);
//   Q8_0:  flat halfword cp = tile halfword (cp, r), the row's two columns.
// Items with consecutive t write consecutive blocks of one row.
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int KT = 16;
constexpr int THREADS = 256;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int QT>
__global__ __launch_bounds__(THREADS) void k_unpack(const uint8_t *__restrict__ tiles,
                                                    int64_t nb, int64_t N,
                                                    uint8_t *__restrict__ flat)
{
    constexpr int TS = Fmt<QT>::tile;
    constexpr int BB = Fmt<QT>::block;
    __shared__ __attribute__((aligned(16))) uint8_t lt[KT * TS];

    const int64_t ct = blockIdx.x;
    const int64_t kt0 = (int64_t)blockIdx.y * KT;
    const int te = (int)min<int64_t>(KT, nb - kt0);
    const u32x4 *src = (const u32x4 *)(tiles + (ct * nb + kt0) * TS);
    for (int i = threadIdx.x; i < te * TS / 16; i += THREADS)
        ((u32x4 *)lt)[i] = src[i];
    __syncthreads();

    for (int i = threadIdx.x; i < te * 32; i += THREADS) {
        const int r = i / te, t = i - r * te;
        const int64_t n = 32 * ct + r;
        if (n >= N)
            continue;
        const uint8_t *tile = lt + t * TS;
        uint8_t *blk = flat + (n * nb + kt0 + t) * BB;
        if constexpr (QT == TQ_Q8_0) {
            u16x8u h0, h1;
#pragma unroll
            for (int cp = 0; cp < 8; cp++) {
                h0[cp] = *(const uint16_t *)(tile + cp * 64 + 2 * r);
                h1[cp] = *(const uint16_t *)(tile + (cp + 8) * 64 + 2 * r);
            }
            *(uint16_t *)blk = *(const uint16_t *)(tile + 1024 + 2 * r);
            *(u16x8u *)(blk + 2) = h0;
            *(u16x8u *)(blk + 18) = h1;
        } else {
            u16x8u qh;
#pragma unroll
            for (int h = 0; h < 8; h++) {
                const uint32_t b1 = tile[h * 32 + r], b2 = tile[(h + 8) * 32 + r];
                const uint32_t lo = (b1 & 0x0Fu) | ((b2 & 0x0Fu) << 4);
                const uint32_t hi = (b1 >> 4) | (b2 & 0xF0u);
                qh[h] = (uint16_t)(lo | (hi << 8));
            }
            if constexpr (QT == TQ_MXFP4) {
                // 17-byte blocks start at any byte: byte stores only
                blk[0] = tile[512 + r];
#pragma unroll
                for (int h = 0; h < 8; h++) {
                    blk[1 + 2 * h] = (uint8_t)qh[h];
                    blk[2 + 2 * h] = (uint8_t)(qh[h] >> 8);
                }
            } else if constexpr (QT == TQ_Q4_1) {
                *(uint32_t *)blk = *(const uint32_t *)(tile + 512 + 4 * r);   // (d, m)
                *(u16x8u *)(blk + 4) = qh;
            } else {
                *(uint16_t *)blk = *(const uint16_t *)(tile + 512 + 2 * r);
                *(u16x8u *)(blk + 2) = qh;
            }
        }
    }
}

}  // namespace

hipError_t launch_unpack(int type, const void *tiles, int64_t K, int64_t N, void *flat,
                         hipStream_t s)
{
    const int64_t nb = K / 32;
    if (!grid_fits((N + 31) / 32, THREADS))
        return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)((N + 31) / 32), (unsigned)((nb + KT - 1) / KT));
    const uint8_t *t = (const uint8_t *)tiles;
    uint8_t *f = (uint8_t *)flat;
    switch (type) {
    case TQ_Q4_0: k_unpack<TQ_Q4_0><<<grid, THREADS, 0, s>>>(t, nb, N, f); break;
    case TQ_IQ4_NL: k_unpack<TQ_IQ4_NL><<<grid, THREADS, 0, s>>>(t, nb, N, f); break;
    case TQ_Q8_0: k_unpack<TQ_Q8_0><<<grid, THREADS, 0, s>>>(t, nb, N, f); break;
    case TQ_MXFP4: k_unpack<TQ_MXFP4><<<grid, THREADS, 0, s>>>(t, nb, N, f); break;
    case TQ_Q4_1: k_unpack<TQ_Q4_1><<<grid, THREADS, 0, s>>>(t, nb, N, f); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace tq
