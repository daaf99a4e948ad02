// Repack flat GGML block-32 rows into 32x32 tiles ("Tiled Weight Formats",
// subsections "Tile Dimensions and Grid Layout" and "Block-32 Quantized
// Formats").  One workgroup takes one 32-row stripe (ct) and KT consecutive
// k-tiles: it stages the 32 rows' flat blocks in LDS with coalesced loads
// (each row's blocks for consecutive kt are contiguous), then writes the KT
// tiles, which are contiguous in the output, one dword per thread per step.
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int KT = 8;          // k-tiles per workgroup
constexpr int THREADS = 256;

template <int QT>
__global__ __launch_bounds__(THREADS) void k_repack(const uint16_t *__restrict__ flat,
                                                    int64_t nb, int64_t N,
                                                    uint32_t *__restrict__ tiles)
{
    constexpr int BH = Fmt<QT>::block / 2;      // halfwords per flat block
    constexpr int TD = Fmt<QT>::tile / 4;       // dwords per tile
    constexpr int RL = KT * BH;                 // halfwords per staged row
    __shared__ uint16_t lds[32][RL];

    const int64_t ct = blockIdx.x;
    const int64_t kt0 = (int64_t)blockIdx.y * KT;
    const int te = (int)min<int64_t>(KT, nb - kt0);
    const int rl = te * BH;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

    for (int r = wave; r < 32; r += THREADS / 64) {
        const int64_t n = 32 * ct + r;
        const uint16_t *src = flat + (n * nb + kt0) * BH;
        for (int j = lane; j < rl; j += 64)
            lds[r][j] = (n < N) ? src[j] : (uint16_t)0;
    }
    __syncthreads();

    uint32_t *dst = tiles + (ct * nb + kt0) * TD;
    for (int i = threadIdx.x; i < te * TD; i += THREADS) {
        const int t = i / TD, w = i - t * TD;
        const uint16_t *blk0 = &lds[0][t * BH];
        uint32_t out;
        if constexpr (QT == TQ_Q8_0) {
            if (w < 256) {
                // dword (cp, rp): rows 2rp and 2rp+1, columns 2cp and 2cp+1;
                // the flat halfword qs[2cp..2cp+1] is exactly that byte pair.
                const int cp = w >> 4, rp = w & 15;
                out = (uint32_t)blk0[(2 * rp) * RL + 1 + cp] |
                      ((uint32_t)blk0[(2 * rp + 1) * RL + 1 + cp] << 16);
            } else {
                const int s = w - 256;
                out = (uint32_t)blk0[(2 * s) * RL] | ((uint32_t)blk0[(2 * s + 1) * RL] << 16);
            }
        } else {
            if (w < 128) {
                // dword (cp, g): rows 4g..4g+3 of column pair cp.  Columns
                // 2cp, 2cp+1 live in the flat halfword qs[2h..2h+1], h = cp mod
                // 8: low nibbles for cp < 8, high nibbles for cp >= 8.
                const int cp = w >> 3, g = w & 7, h = cp & 7;
                out = 0;
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const uint32_t v = blk0[(4 * g + j) * RL + 1 + h];
                    const uint32_t b = (cp < 8) ? ((v & 0x0Fu) | ((v >> 4) & 0xF0u))
                                                : (((v >> 4) & 0x0Fu) | ((v >> 8) & 0xF0u));
                    out |= b << (8 * j);
                }
            } else {
                const int s = w - 128;
                out = (uint32_t)blk0[(2 * s) * RL] | ((uint32_t)blk0[(2 * s + 1) * RL] << 16);
            }
        }
        dst[i] = out;
    }
}

}  // namespace

hipError_t launch_repack(int type, const void *flat, int64_t K, int64_t N, void *tiles,
                         hipStream_t s)
{
    const int64_t nb = K / 32;
    dim3 grid((unsigned)((N + 31) / 32), (unsigned)((nb + KT - 1) / KT));
    const uint16_t *f = (const uint16_t *)flat;
    uint32_t *t = (uint32_t *)tiles;
    switch (type) {
    case TQ_Q4_0: k_repack<TQ_Q4_0><<<grid, THREADS, 0, s>>>(f, nb, N, t); break;
    case TQ_IQ4_NL: k_repack<TQ_IQ4_NL><<<grid, THREADS, 0, s>>>(f, nb, N, t); break;
    case TQ_Q8_0: k_repack<TQ_Q8_0><<<grid, THREADS, 0, s>>>(f, nb, N, t); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace tq
