// Decode matrix-vector product (M <= 8 activation rows) over flat,
// un-repacked GGML blocks ("supports_op Independence from Buffer and Repack
// State": a supported type must also work when stored flat).  Results equal
// those over the tiles of the same data (the same integer block dots, the
// same per-block scaling).
//
// Layout facts used: row n of the weights is K/32 consecutive blocks
// (Q4_K: K/256 super-blocks); in a 4-bit block the low nibbles of quant
// bytes 0..15 are elements 0..15 and the high nibbles elements 16..31, so a
// quant dword's low nibbles are 4 consecutive K and v_dot4_i32_i8 needs no
// transposes.  Each lane therefore owns whole blocks: it loads one block
// (16-byte vector loads at the block's 2-byte alignment), decodes it into 8
// int8 dwords in K order and forms the exact block dot against the staged
// activations alone; lanes are summed only once per output, at the end.
//
// Work split: a workgroup of 4 waves takes 16 consecutive rows, 4 per wave;
// a wave takes its 4 rows together (4 blocks in flight per lane).  The
// activations of all M rows are staged in LDS per pass over K, as in the
// tiled kernel, with their fp32 scales and, for Q4_1 / Q4_K, block sums.
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int WAVES = 4, RW = 4, ROWS = WAVES * RW;   // rows per wave / workgroup

template <int MM>
constexpr int flat_act_lds_bytes()
{
    return MM <= 4 ? 32768 : 40960;
}

// One weight block decoded for the dot: dword k holds the int8 weights of K
// 4k .. 4k + 3 of the block; dw (and for Q4_1 / Q4_K mw) the row's scale.
struct WBlock {
    uint32_t w[8];
    float dw, mw;
};

// Load and decode block kb (32-element index) of row n.
template <int QT>
__device__ __forceinline__ void load_block(WBlock &b, const uint8_t *__restrict__ flat,
                                           int64_t n, int64_t nb, int64_t kb, int64_t total,
                                           const Lut &lut)
{
    constexpr int BB = Fmt<QT>::block;
    b.mw = 0.0f;
    if constexpr (QT == TQ_Q4_K) {
        const uint8_t *sb = flat + (n * (nb / 8) + kb / 8) * BB;   // 16-byte aligned
        const int s = (int)(kb & 7), c = s >> 1;
        const uint4 h = *(const uint4 *)sb;
        const uint4 q0 = *(const uint4 *)(sb + 16 + 32 * c);
        const uint4 q1 = *(const uint4 *)(sb + 32 + 32 * c);
        const uint32_t qd[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
        for (int k = 0; k < 8; k++)
            b.w[k] = (s & 1) ? ((qd[k] >> 4) & 0x0F0F0F0Fu) : (qd[k] & 0x0F0F0F0Fu);
        const uint32_t s3[3] = {h.y, h.z, h.w};
        uint32_t sc, m;
        q4k_scale_min(s3, s, sc, m);
        const float d = f16_bits_to_f32((uint16_t)h.x);
        const float dmin = f16_bits_to_f32((uint16_t)(h.x >> 16));
        b.dw = f16_bits_to_f32(f16_of_product(d, (float)sc));
        b.mw = f16_bits_to_f32(f16_of_product(-dmin, (float)m));
        return;
    } else if constexpr (QT == TQ_Q8_0) {
        const uint8_t *blk = flat + (n * nb + kb) * BB;
        const u16x8u a0 = *(const u16x8u *)(blk + 2);
        const u16x8u a1 = *(const u16x8u *)(blk + 18);
#pragma unroll
        for (int k = 0; k < 4; k++) {
            b.w[k] = a0[2 * k] | ((uint32_t)a0[2 * k + 1] << 16);
            b.w[4 + k] = a1[2 * k] | ((uint32_t)a1[2 * k + 1] << 16);
        }
        b.dw = f16_bits_to_f32(*(const uint16_t *)blk);
        return;
    } else {
        uint32_t q[4];
        if constexpr (QT == TQ_MXFP4) {
            uint16_t qh[8], e;
            load_mx_block(flat, (n * nb + kb) * BB, total, qh, e);
#pragma unroll
            for (int k = 0; k < 4; k++)
                q[k] = qh[2 * k] | ((uint32_t)qh[2 * k + 1] << 16);
            b.dw = f16_bits_to_f32(e8m0_f16_bits(e)) * weight_unscale<QT>();
        } else {
            const uint8_t *blk = flat + (n * nb + kb) * BB;
            constexpr int QOFF = QT == TQ_Q4_1 ? 4 : 2;
            const u16x8u a = *(const u16x8u *)(blk + QOFF);
#pragma unroll
            for (int k = 0; k < 4; k++)
                q[k] = a[2 * k] | ((uint32_t)a[2 * k + 1] << 16);
            if constexpr (QT == TQ_Q4_1) {
                const uint32_t dm = *(const uint32_t *)blk;      // 20-byte blocks: aligned
                b.dw = f16_bits_to_f32((uint16_t)dm);
                b.mw = f16_bits_to_f32((uint16_t)(dm >> 16));
            } else {
                b.dw = f16_bits_to_f32(*(const uint16_t *)blk) * weight_unscale<QT>();
            }
        }
        // low nibbles: K 4k .. 4k + 3; high nibbles: K 16 + 4k ..
#pragma unroll
        for (int k = 0; k < 4; k++) {
            if constexpr (QT == TQ_Q4_0) {
                const uint32_t t = q[k] ^ 0x88888888u;
                b.w[k] = (t << 4) & 0xF0F0F0F0u;        // 16 (code - 8), as the tiled path
                b.w[4 + k] = t & 0xF0F0F0F0u;
            } else if constexpr (QT == TQ_Q4_1) {
                b.w[k] = q[k] & 0x0F0F0F0Fu;
                b.w[4 + k] = (q[k] >> 4) & 0x0F0F0F0Fu;
            } else {
                lut16x2(q[k], lut, b.w[k], b.w[4 + k]);
            }
        }
    }
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        v += __shfl_xor(v, o);
    return v;
}

template <int QT, int MM, bool DOTS>
__global__ __launch_bounds__(WAVES * 64) void k_qgemv_flat(
    const uint8_t *__restrict__ flat, int64_t nb, int64_t N, const int8_t *__restrict__ q,
    const uint16_t *__restrict__ d, int64_t K, Lut lut, float *__restrict__ y, int64_t ldy,
    int32_t *__restrict__ isum, int64_t total)
{
    constexpr bool MIN = QT == TQ_Q4_1 || QT == TQ_Q4_K;
    constexpr int PB = MIN ? 40 : 36;                     // LDS bytes per block and row
    constexpr int P = flat_act_lds_bytes<MM>() / (MM * PB);
    __shared__ __attribute__((aligned(16))) uint8_t act[flat_act_lds_bytes<MM>()];
    int8_t *qs = (int8_t *)act;                           // [block][row][32]
    float *ds = (float *)(act + MM * P * 32);             // [block][row]
    float *ss = ds + MM * P;                              // block sums (Q4_1, Q4_K)

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t nw0 = (int64_t)blockIdx.x * ROWS + wave * RW;    // this wave's first row
    float acc[RW][MM];
#pragma unroll
    for (int r = 0; r < RW; r++)
#pragma unroll
        for (int m = 0; m < MM; m++)
            acc[r][m] = 0.0f;

    for (int64_t pb = 0; pb < nb; pb += P) {
        const int pn = (int)min<int64_t>(P, nb - pb);
        __syncthreads();                                  // previous pass done with the LDS
        // stage: 16-byte chunk o (block o / 2, half o % 2) of each row m
        for (int o = threadIdx.x; o < 2 * pn; o += WAVES * 64) {
#pragma unroll
            for (int m = 0; m < MM; m++) {
                const uint4 v = *(const uint4 *)(q + m * K + (pb * 32 + 16 * o));
                *(uint4 *)(qs + ((o >> 1) * MM + m) * 32 + 16 * (o & 1)) = v;
                if (o < pn)
                    ds[o * MM + m] = DOTS ? 0.0f : f16_bits_to_f32(d[m * nb + pb + o]);
                if constexpr (MIN && !DOTS) {
                    // pairs (o, o ^ 1) are in range together: 2 pn is even
                    int s = byte_sum(v.x, byte_sum(v.y, byte_sum(v.z, byte_sum(v.w, 0))));
                    s += __shfl_xor(s, 1);
                    if ((o & 1) == 0)
                        ss[(o >> 1) * MM + m] = (float)s;
                }
            }
        }
        __syncthreads();

        for (int jp = lane; jp < pn; jp += 64) {
            WBlock b[RW];
#pragma unroll
            for (int r = 0; r < RW; r++)
                if (nw0 + r < N)
                    load_block<QT>(b[r], flat, nw0 + r, nb, pb + jp, total, lut);
#pragma unroll
            for (int m = 0; m < MM; m++) {
                const uint4 xa = *(const uint4 *)(qs + (jp * MM + m) * 32);
                const uint4 xb = *(const uint4 *)(qs + (jp * MM + m) * 32 + 16);
                const uint32_t x[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
                const float da = ds[jp * MM + m];
#pragma unroll
                for (int r = 0; r < RW; r++) {
                    if (nw0 + r >= N)
                        continue;
                    int s = 0;
#pragma unroll
                    for (int k = 0; k < 8; k++)
                        s = __builtin_amdgcn_sdot4((int)b[r].w[k], (int)x[k], s, false);
                    if constexpr (DOTS) {
                        isum[((int64_t)m * N + nw0 + r) * nb + pb + jp] =
                            (QT == TQ_Q4_0) ? (s >> 4) : s;
                    } else {
                        acc[r][m] = fmaf((float)s, b[r].dw * da, acc[r][m]);
                        if constexpr (MIN)
                            acc[r][m] = fmaf(b[r].mw, da * ss[jp * MM + m], acc[r][m]);
                    }
                }
            }
        }
    }
    if constexpr (DOTS)
        return;
#pragma unroll
    for (int r = 0; r < RW; r++) {
#pragma unroll
        for (int m = 0; m < MM; m++) {
            const float v = wave_sum(acc[r][m]);
            if (lane == 0 && nw0 + r < N)
                y[m * ldy + nw0 + r] = v;
        }
    }
}

template <int QT, int MM>
hipError_t launch_m(const void *flat, int64_t K, int64_t N, const int8_t *q, const uint16_t *d,
                    const Lut &lut, float *y, int64_t ldy, int32_t *isum, hipStream_t s)
{
    const int64_t nb = K / 32;
    const int64_t total = N * (K / (QT == TQ_Q4_K ? 256 : 32)) * Fmt<QT>::block;
    if (!grid_fits((N + ROWS - 1) / ROWS, WAVES * 64))
        return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)((N + ROWS - 1) / ROWS));
    if (isum)
        k_qgemv_flat<QT, MM, true><<<grid, WAVES * 64, 0, s>>>(
            (const uint8_t *)flat, nb, N, q, d, K, lut, y, ldy, isum, total);
    else
        k_qgemv_flat<QT, MM, false><<<grid, WAVES * 64, 0, s>>>(
            (const uint8_t *)flat, nb, N, q, d, K, lut, y, ldy, isum, total);
    return hipGetLastError();
}

template <int QT>
hipError_t launch_t(const void *flat, int64_t K, int64_t N, const int8_t *q, const uint16_t *d,
                    int64_t M, const Lut &lut, float *y, int64_t ldy, int32_t *isum,
                    hipStream_t s)
{
    switch (M) {
    case 1: return launch_m<QT, 1>(flat, K, N, q, d, lut, y, ldy, isum, s);
    case 2: return launch_m<QT, 2>(flat, K, N, q, d, lut, y, ldy, isum, s);
    case 3: return launch_m<QT, 3>(flat, K, N, q, d, lut, y, ldy, isum, s);
    case 4: return launch_m<QT, 4>(flat, K, N, q, d, lut, y, ldy, isum, s);
    case 5: return launch_m<QT, 5>(flat, K, N, q, d, lut, y, ldy, isum, s);
    case 6: return launch_m<QT, 6>(flat, K, N, q, d, lut, y, ldy, isum, s);
    case 7: return launch_m<QT, 7>(flat, K, N, q, d, lut, y, ldy, isum, s);
    case 8: return launch_m<QT, 8>(flat, K, N, q, d, lut, y, ldy, isum, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_qgemv_flat(int type, const void *flat, int64_t K, int64_t N, const int8_t *q,
                             const uint16_t *d, int64_t M, const Lut &lut, float *y,
                             int64_t ldy, int32_t *isum, hipStream_t s)
{
    switch (type) {
    case TQ_Q4_0: return launch_t<TQ_Q4_0>(flat, K, N, q, d, M, lut, y, ldy, isum, s);
    case TQ_Q8_0: return launch_t<TQ_Q8_0>(flat, K, N, q, d, M, lut, y, ldy, isum, s);
    case TQ_IQ4_NL: return launch_t<TQ_IQ4_NL>(flat, K, N, q, d, M, lut, y, ldy, isum, s);
    case TQ_MXFP4: return launch_t<TQ_MXFP4>(flat, K, N, q, d, M, lut, y, ldy, isum, s);
    case TQ_Q4_1: return launch_t<TQ_Q4_1>(flat, K, N, q, d, M, lut, y, ldy, isum, s);
    case TQ_Q4_K: return launch_t<TQ_Q4_K>(flat, K, N, q, d, M, lut, y, ldy, isum, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace tq
