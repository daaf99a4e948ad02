// Prefill matrix-matrix product over 32x32 tiles with int8 MFMA.
//
// A workgroup of 8 waves owns a BM x BN = 128 x 64 output block (M rows of
// activations x N output features).  Per 32-element K block kt it stages in
// LDS: the activation block (128 rows x 32 int8, natural K order) with its
// fp16 scales, and the two weight tiles of its two stripes decoded to int8
// in [row][K] order (the tile's [column pair][row] byte order is transposed
// on the way in: "Block-32 Quantized Formats") with their fp16 row scales.
// Each wave then runs one v_mfma_i32_32x32x32_i8 on its 32 x 32 sub-block;
// the instruction's K depth equals the block size, so its int32 output is
// exactly the per-block integer dot, which is scaled by (row scale x
// activation scale, exact in fp32) and accumulated in fp32.  The next
// block's global loads are issued before the current block's MFMA.
#include "tq_internal.h"

namespace tq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 64, THREADS = 512;
constexpr int LDS_ROW = 48;    // bytes per staged 32-byte row (padding spreads LDS banks)

template <int QT>
struct Stage {
    uint4 a;          // 16 bytes of activations (threads 0..255)
    uint16_t da;      // activation scale (threads 256..383)
    uint32_t w[2];    // weight quant dwords
    uint16_t dw;      // weight row scale (threads 448..511)
};

template <int QT, bool DOTS>
__device__ __forceinline__ void load_stage(Stage<QT> &s, const uint8_t *tiles, int64_t nkt,
                                           int64_t nct, int64_t ct0, const int8_t *q,
                                           const uint16_t *d, int64_t M, int64_t K, int64_t m0,
                                           int64_t kt, int tid)
{
    constexpr int TS = Fmt<QT>::tile;
    if (tid < 256) {
        const int64_t m = m0 + (tid >> 1);
        if (m < M)
            s.a = *(const uint4 *)(q + m * K + kt * 32 + 16 * (tid & 1));
        else
            s.a = make_uint4(0, 0, 0, 0);
    } else if (tid < 384) {
        const int64_t m = m0 + (tid - 256);
        s.da = (!DOTS && m < M) ? d[m * nkt + kt] : (uint16_t)0;   // no scales in block-dot mode
    }
    // weight quants: Q8_0 512 dwords over 2 tiles (1 per thread);
    // 4-bit 256 dwords (threads 256..511, 1 each)
    if constexpr (QT == TQ_Q8_0) {
        const int tt = tid >> 8, w = tid & 255;
        const int64_t ct = ct0 + tt;
        s.w[0] = (ct < nct) ? __builtin_nontemporal_load(
                                  (const uint32_t *)(tiles + (ct * nkt + kt) * TS) + w)
                            : 0u;
    } else if (tid >= 256) {
        const int i = tid - 256, tt = i >> 7, w = i & 127;
        const int64_t ct = ct0 + tt;
        s.w[0] = (ct < nct) ? __builtin_nontemporal_load(
                                  (const uint32_t *)(tiles + (ct * nkt + kt) * TS) + w)
                            : 0u;
    }
    if (tid >= 448) {
        const int i = tid - 448, tt = i >> 5, r = i & 31;
        const int64_t ct = ct0 + tt;
        s.dw = (ct < nct) ? ((const uint16_t *)(tiles + (ct * nkt + kt) * TS +
                                                Fmt<QT>::scale_off))[r]
                          : (uint16_t)0;
    }
}

template <int QT>
__device__ __forceinline__ void store_stage(const Stage<QT> &s, uint8_t *As, uint8_t *Bs,
                                            float *das, float *dws, const Lut &lut, int tid)
{
    if (tid < 256)
        *(uint4 *)(As + (tid >> 1) * LDS_ROW + 16 * (tid & 1)) = s.a;
    else if (tid < 384)
        das[tid - 256] = f16_bits_to_f32(s.da);
    if constexpr (QT == TQ_Q8_0) {
        // dword w = cp*16 + p: [row 2p: col 2cp, 2cp+1][row 2p+1: col 2cp, 2cp+1]
        const int tt = tid >> 8, w = tid & 255, cp = w >> 4, p = w & 15;
        uint8_t *b = Bs + (32 * tt + 2 * p) * LDS_ROW + 2 * cp;
        *(uint16_t *)b = (uint16_t)(s.w[0] & 0xFFFFu);
        *(uint16_t *)(b + LDS_ROW) = (uint16_t)(s.w[0] >> 16);
    } else if (tid >= 256) {
        // dword w = cp*8 + g: byte j = row 4g+j, low nibble col 2cp, high col 2cp+1
        const int i = tid - 256, tt = i >> 7, w = i & 127, cp = w >> 3, g = w & 7;
        const uint32_t v = s.w[0];
        uint32_t lo, hi;
        if constexpr (QT == TQ_Q4_0) {
            // code - 8 for 4-bit codes, bytewise: (c ^ 8) is c - 8 in 4-bit two's
            // complement; sign-extend it to 8 bits
            const uint32_t tl = (v & 0x0F0F0F0Fu) ^ 0x08080808u;
            const uint32_t th = ((v >> 4) & 0x0F0F0F0Fu) ^ 0x08080808u;
            lo = tl | (((tl >> 3) & 0x01010101u) * 0xF0u);
            hi = th | (((th >> 3) & 0x01010101u) * 0xF0u);
        } else {
            lo = lut16(v & 0x0F0F0F0Fu, lut);
            hi = lut16((v >> 4) & 0x0F0F0F0Fu, lut);
        }
        // interleave: row j gets (lo byte j, hi byte j)
        const uint32_t p01 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);  // [lo0, hi0, lo1, hi1]
        const uint32_t p23 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);  // [lo2, hi2, lo3, hi3]
        uint8_t *b = Bs + (32 * tt + 4 * g) * LDS_ROW + 2 * cp;
        *(uint16_t *)b = (uint16_t)(p01 & 0xFFFFu);
        *(uint16_t *)(b + LDS_ROW) = (uint16_t)(p01 >> 16);
        *(uint16_t *)(b + 2 * LDS_ROW) = (uint16_t)(p23 & 0xFFFFu);
        *(uint16_t *)(b + 3 * LDS_ROW) = (uint16_t)(p23 >> 16);
    }
    if (tid >= 448)
        dws[tid - 448] = f16_bits_to_f32(s.dw);
}

template <int QT, bool DOTS>
__global__ __launch_bounds__(THREADS) void k_qgemm(const uint8_t *__restrict__ tiles,
                                                   int64_t nkt, int64_t N,
                                                   const int8_t *__restrict__ q,
                                                   const uint16_t *__restrict__ d, int64_t M,
                                                   int64_t K, Lut lut, float *__restrict__ y,
                                                   int64_t ldy, int32_t *__restrict__ isum)
{
    __shared__ __attribute__((aligned(16))) uint8_t As[BM * LDS_ROW];
    __shared__ __attribute__((aligned(16))) uint8_t Bs[BN * LDS_ROW];
    __shared__ __attribute__((aligned(16))) float das[BM];
    __shared__ float dws[BN];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 3, wn = wave >> 2;
    const int64_t nct = (N + 31) / 32;
    const int64_t ct0 = (int64_t)blockIdx.x * (BN / 32);
    const int64_t m0 = (int64_t)blockIdx.y * BM;

    float acc[16];
#pragma unroll
    for (int r = 0; r < 16; r++)
        acc[r] = 0.0f;

    const int li = lane & 31, lk = lane >> 5;
    Stage<QT> st;
    load_stage<QT, DOTS>(st, tiles, nkt, nct, ct0, q, d, M, K, m0, 0, tid);
    for (int64_t kt = 0; kt < nkt; kt++) {
        __syncthreads();                 // previous block's LDS reads are done
        store_stage<QT>(st, As, Bs, das, dws, lut, tid);
        __syncthreads();
        if (kt + 1 < nkt)
            load_stage<QT, DOTS>(st, tiles, nkt, nct, ct0, q, d, M, K, m0, kt + 1, tid);

        const v4i a = *(const v4i *)(As + (32 * wm + li) * LDS_ROW + 16 * lk);
        const v4i b = *(const v4i *)(Bs + (32 * wn + li) * LDS_ROW + 16 * lk);
        v16i z = {};
        const v16i dot = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, z, 0, 0, 0);
        // output layout: lane holds column li, rows 8*(r/4) + 4*lk + (r%4)
        if constexpr (DOTS) {
            const int64_t n = 32 * (ct0 + wn) + li;
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int64_t m = m0 + 32 * wm + 8 * (r >> 2) + 4 * lk + (r & 3);
                if (m < M && n < N)
                    isum[(m * N + n) * nkt + kt] = dot[r];
            }
        } else {
            const float dw = dws[32 * wn + li];
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const float4 da = *(const float4 *)(das + 32 * wm + 8 * g + 4 * lk);
                acc[4 * g + 0] = fmaf((float)dot[4 * g + 0], da.x * dw, acc[4 * g + 0]);
                acc[4 * g + 1] = fmaf((float)dot[4 * g + 1], da.y * dw, acc[4 * g + 1]);
                acc[4 * g + 2] = fmaf((float)dot[4 * g + 2], da.z * dw, acc[4 * g + 2]);
                acc[4 * g + 3] = fmaf((float)dot[4 * g + 3], da.w * dw, acc[4 * g + 3]);
            }
        }
    }
    if constexpr (DOTS)
        return;
    const int64_t n = 32 * (ct0 + wn) + li;
    if (n < N) {
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const int64_t m = m0 + 32 * wm + 8 * (r >> 2) + 4 * lk + (r & 3);
            if (m < M)
                y[m * ldy + n] = acc[r];
        }
    }
}

template <int QT>
hipError_t launch_t(const void *tiles, int64_t K, int64_t N, const int8_t *q, const uint16_t *d,
                    int64_t M, const Lut &lut, float *y, int64_t ldy, int32_t *isum,
                    hipStream_t s)
{
    const int64_t nkt = K / 32;
    const int64_t nct = (N + 31) / 32;
    dim3 grid((unsigned)((nct + BN / 32 - 1) / (BN / 32)), (unsigned)((M + BM - 1) / BM));
    if (isum)
        k_qgemm<QT, true><<<grid, THREADS, 0, s>>>((const uint8_t *)tiles, nkt, N, q, d, M, K,
                                                   lut, y, ldy, isum);
    else
        k_qgemm<QT, false><<<grid, THREADS, 0, s>>>((const uint8_t *)tiles, nkt, N, q, d, M, K,
                                                    lut, y, ldy, isum);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_qgemm(int type, const void *tiles, int64_t K, int64_t N, const int8_t *q,
                        const uint16_t *d, int64_t M, const Lut &lut, float *y, int64_t ldy,
                        int32_t *isum, hipStream_t s)
{
    switch (type) {
    case TQ_Q4_0: return launch_t<TQ_Q4_0>(tiles, K, N, q, d, M, lut, y, ldy, isum, s);
    case TQ_Q8_0: return launch_t<TQ_Q8_0>(tiles, K, N, q, d, M, lut, y, ldy, isum, s);
    case TQ_IQ4_NL: return launch_t<TQ_IQ4_NL>(tiles, K, N, q, d, M, lut, y, ldy, isum, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace tq
