// Repack flat GGML block-32 rows into 32x32 tiles ("Tiled Weight Formats",
// subsections "Tile Dimensions and Grid Layout" and "Block-32 Quantized
// Formats").  One workgroup takes one 32-row stripe (ct) and KT consecutive
// k-tiles, which are contiguous in the output.
//
// Load: one flat block (row r, k-tile t) per work item, its quant bytes read
// as 16-byte vectors; the quants go to LDS transposed, as halfword columns
// qs[t][32 h + r] (halfword h = quant bytes 2h, 2h+1 of row r), the scales
// to sc[t][r].  In that layout the 32 rows of one halfword are contiguous, which
// is what both tile formats need:
//   Q8_0: tile dword (cp, rp) = halfword cp of rows 2rp and 2rp+1, so a
//         16-byte tile chunk is a 16-byte LDS read, stored as is;
//   Q4_0 / IQ4_NL / MXFP4 / Q4_1: tile byte (cp, r) = one nibble of each of quant
//         bytes 2h, 2h+1 of row r (h = cp mod 8; low nibbles for cp < 8,
//         high for cp >= 8), built two rows at a time with shifts and masks.
// Store: every thread writes whole 16-byte chunks of the tiles.
//
// MXFP4 blocks are 17 bytes (one E8M0 byte, then the 16 quant bytes), so
// most of them start at odd addresses: a block is read as the 5 aligned
// dwords that cover it (the flat buffer is 4-byte aligned) and shifted into
// place.
#include <type_traits>

#include "tq_internal.h"

namespace tq {
namespace {

constexpr int KT = 16;         // k-tiles per workgroup
constexpr int THREADS = 256;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// One Q4_K super-block of row r (16-byte aligned, 144 bytes) into the 8
// tiles' LDS staging of k_repack: for sub-block j, the 16 bytes of a flat
// 32-element block (element e low, e + 16 high nibble, as Q4_0) and the pair
// (fp16 d * sc_j, fp16 -(dmin * m_j)), products exact in fp32, rounded to
// nearest even.  valid = false stages zeros.
template <int TP>
__device__ __forceinline__ void stage_q4k(const uint8_t *__restrict__ blk, bool valid, int r,
                                          uint16_t (*qs)[TP], uint32_t (*sc)[32])
{
    uint32_t w[36];
#pragma unroll
    for (int v = 0; v < 9; v++) {
        const u32x4 x = valid ? *(const u32x4 *)(blk + 16 * v) : u32x4{0, 0, 0, 0};
        w[4 * v] = x.x;
        w[4 * v + 1] = x.y;
        w[4 * v + 2] = x.z;
        w[4 * v + 3] = x.w;
    }
    const float d = f16_bits_to_f32((uint16_t)w[0]);
    const float dmin = f16_bits_to_f32((uint16_t)(w[0] >> 16));
    auto sbyte = [&](int k) { return (w[1 + k / 4] >> (8 * (k % 4))) & 0xFFu; };   // scales[k]
#pragma unroll
    for (int j = 0; j < 8; j++) {
        uint32_t s6, m6;
        if (j < 4) {
            s6 = sbyte(j) & 63u;
            m6 = sbyte(j + 4) & 63u;
        } else {
            s6 = (sbyte(j + 4) & 15u) | ((sbyte(j - 4) >> 6) << 4);
            m6 = (sbyte(j + 4) >> 4) | ((sbyte(j) >> 6) << 4);
        }
        // -dmin * m is -(dmin * m) bit for bit, signed zeros included
        const uint32_t a = f16_of_product(d, (float)s6);
        const uint32_t b = f16_of_product(-dmin, (float)m6);
        sc[j][r] = valid ? (a | (b << 16)) : 0u;
        // sub-block j = nibble j % 2 of 64-element chunk j / 2
        const int c = j >> 1;
#pragma unroll
        for (int v = 0; v < 4; v++) {
            const uint32_t lo = w[4 + 8 * c + v], hi = w[4 + 8 * c + 4 + v];   // elements v.., 16 + v..
            const uint32_t o = (j & 1) ? (((lo >> 4) & 0x0F0F0F0Fu) | (hi & 0xF0F0F0F0u))
                                       : ((lo & 0x0F0F0F0Fu) | ((hi & 0x0F0F0F0Fu) << 4));
            qs[j][32 * (2 * v) + r] = (uint16_t)o;
            qs[j][32 * (2 * v + 1) + r] = (uint16_t)(o >> 16);
        }
    }
}

template <int QT>
__global__ __launch_bounds__(THREADS) void k_repack(const uint8_t *__restrict__ flat,
                                                    int64_t nb, int64_t N,
                                                    uint8_t *__restrict__ tiles)
{
    constexpr bool MX = QT == TQ_MXFP4;
    constexpr bool Q41 = QT == TQ_Q4_1;
    constexpr bool Q4K = QT == TQ_Q4_K;
    constexpr int BB = Fmt<QT>::block;          // flat block bytes (scales + quants)
    constexpr int QOFF = MX ? 1 : (Q41 ? 4 : 2);// offset of the quants in a block
    constexpr int QH = Q4K ? 8 : (BB - QOFF) / 2;   // quant halfwords per tile row: 8 or 16
    constexpr int TS = Fmt<QT>::tile;
    constexpr int CH = TS / 16;                 // 16-byte chunks per tile: 36, 68 or 34
    constexpr int QCH = Fmt<QT>::scale_off / 16;// chunks of quants (the rest hold scales)
    // a row's scale bytes in the tile: E8M0 byte, fp16 d, or fp16 pair (d, m)
    using Scale =
        std::conditional_t<MX, uint8_t, std::conditional_t<Q41 || Q4K, uint32_t, uint16_t>>;
    constexpr int SPC = 16 / (int)sizeof(Scale);// row scales per 16-byte chunk
    // each tile's halfword columns padded by 16 bytes: the lanes of a store
    // differ in t, and a tile stride of 16 mod 256 bytes spreads them over
    // the LDS banks
    constexpr int TP = QH * 32 + 8;
    __shared__ __attribute__((aligned(16))) uint16_t qs[KT][TP];
    __shared__ __attribute__((aligned(16))) Scale sc[KT][32];

    const int64_t ct = blockIdx.x;
    const int64_t kt0 = (int64_t)blockIdx.y * KT;
    const int te = (int)min<int64_t>(KT, nb - kt0);

    if constexpr (Q4K) {
        // item = (row r, super-block): 8 tiles at once (te is a multiple of 8)
        const int nsb = te / 8;
        for (int i = threadIdx.x; i < nsb * 32; i += THREADS) {
            const int r = i / nsb, sb = i - r * nsb;
            const int64_t n = 32 * ct + r;
            const uint8_t *blk = flat + ((n < N ? n : 0) * (nb / 8) + kt0 / 8 + sb) * BB;
            stage_q4k<TP>(blk, n < N, r, &qs[8 * sb], &sc[8 * sb]);
        }
    }
    // Load: item i = (row r = i / te, tile t = i % te), so a wave reads a few
    // contiguous runs of blocks; rows past N are zero.
    for (int i = threadIdx.x; i < (Q4K ? 0 : te * 32); i += THREADS) {
        const int r = i / te, t = i - r * te;
        const int64_t n = 32 * ct + r;
        uint16_t q[QH];
        Scale d = 0;
        if (n < N) {
            if constexpr (MX) {
                uint16_t e;
                load_mx_block(flat, (n * nb + kt0 + t) * BB, N * nb * BB, q, e);
                d = (Scale)e;
            } else {
                // Q4_1 blocks are 20 bytes and the flat buffer 4-byte aligned,
                // so (d, m) is one aligned dword
                const uint8_t *blk = flat + (n * nb + kt0 + t) * BB;
                d = *(const Scale *)blk;
#pragma unroll
                for (int v = 0; v < QH / 8; v++) {
                    const u16x8u w = *(const u16x8u *)(blk + QOFF + 16 * v);
#pragma unroll
                    for (int e = 0; e < 8; e++)
                        q[8 * v + e] = w[e];
                }
            }
        } else {
#pragma unroll
            for (int h = 0; h < QH; h++)
                q[h] = 0;
        }
#pragma unroll
        for (int h = 0; h < QH; h++)
            qs[t][32 * h + r] = q[h];
        sc[t][r] = d;
    }
    __syncthreads();

    uint8_t *dst = tiles + (ct * nb + kt0) * TS;
    for (int i = threadIdx.x; i < te * CH; i += THREADS) {
        const int t = i / CH, c = i - t * CH;
        u32x4 out;
        if (c >= QCH) {
            // scale chunk: rows SPC j .. SPC j + SPC - 1
            out = *(const u32x4 *)&sc[t][SPC * (c - QCH)];
        } else if constexpr (QT == TQ_Q8_0) {
            // dwords (cp, rp .. rp + 3): halfword cp of rows 8j .. 8j + 7
            out = *(const u32x4 *)&qs[t][32 * (c >> 2) + 8 * (c & 3)];
        } else {
            // dwords (cp, g .. g + 3), g = 4 (c & 1): rows 16 (c & 1) .. + 15
            const int cp = c >> 1, h = cp & 7;
            const u32x4 *src = (const u32x4 *)&qs[t][32 * h + 16 * (c & 1)];
            const u32x4 a = src[0], b = src[1];     // rows +0..+7, +8..+15
            const uint32_t v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
            uint32_t o[4];
#pragma unroll
            for (int j = 0; j < 4; j++) {
                // v holds two rows (low / high halfword); per row the tile
                // byte takes one nibble of each quant byte of the halfword
                uint32_t p[2];
#pragma unroll
                for (int k = 0; k < 2; k++) {
                    const uint32_t x = v[2 * j + k];
                    p[k] = cp < 8 ? ((x & 0x000F000Fu) | ((x >> 4) & 0x00F000F0u))
                                  : (((x >> 4) & 0x000F000Fu) | ((x >> 8) & 0x00F000F0u));
                }
                o[j] = __builtin_amdgcn_perm(p[1], p[0], 0x06040200u);
            }
            out = u32x4{o[0], o[1], o[2], o[3]};
        }
        *(u32x4 *)(dst + (int64_t)t * TS + 16 * c) = out;
    }
}

}  // namespace

hipError_t launch_repack(int type, const void *flat, int64_t K, int64_t N, void *tiles,
                         hipStream_t s)
{
    const int64_t nb = K / 32;
    if (!grid_fits((N + 31) / 32, THREADS))
        return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)((N + 31) / 32), (unsigned)((nb + KT - 1) / KT));
    const uint8_t *f = (const uint8_t *)flat;
    uint8_t *t = (uint8_t *)tiles;
    switch (type) {
    case TQ_Q4_0: k_repack<TQ_Q4_0><<<grid, THREADS, 0, s>>>(f, nb, N, t); break;
    case TQ_IQ4_NL: k_repack<TQ_IQ4_NL><<<grid, THREADS, 0, s>>>(f, nb, N, t); break;
    case TQ_Q8_0: k_repack<TQ_Q8_0><<<grid, THREADS, 0, s>>>(f, nb, N, t); break;
    case TQ_MXFP4: k_repack<TQ_MXFP4><<<grid, THREADS, 0, s>>>(f, nb, N, t); break;
    case TQ_Q4_1: k_repack<TQ_Q4_1><<<grid, THREADS, 0, s>>>(f, nb, N, t); break;
    case TQ_Q4_K: k_repack<TQ_Q4_K><<<grid, THREADS, 0, s>>>(f, nb, N, t); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace tq
