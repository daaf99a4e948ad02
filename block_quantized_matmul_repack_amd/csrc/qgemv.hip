// Decode matrix-vector product over 32x32 tiles, M <= 8 activation rows.
//
// Layout facts used ("Tiled Weight Formats" / "Block-32 Quantized Formats"):
// a 32-row stripe's K/32 tiles are contiguous; inside a tile the quant bytes
// are ordered [column pair][row], so one dword holds 4 rows (4-bit types) or
// 2 rows (Q8_0) of one column pair.  The integer dot wants one row's
// consecutive K values in a dword (v_dot4_i32_i8), so every lane transposes
// the bytes it loads with v_perm_b32 and finishes each row's 32-element
// block dot with one or two quad DPP adds.
//
// Mapping: one workgroup per stripe; each wave half (32 lanes) owns one tile
// per step, so a workgroup step reads 2*NW consecutive tiles.  After the
// in-quad reduction lane l of the half holds the exact int32 block dot of row
// l, scales it by its fp16 row scale times the fp16 activation scale (exact
// in fp32) and accumulates in fp32.  Partial sums of the 2*NW halves are added
// in a fixed order through LDS, so results are deterministic.
//
// 4-bit lanes: lane l = 4g + c loads the dwords of rows 4g..4g+3 for the
// column pairs 4c..4c+3 (K indices 8c..8c+7).  Q8_0 lanes: lane l = 2p + h
// loads rows 2p, 2p+1 for column pairs 8h..8h+7 (K indices 16h..16h+15).
// Each lane keeps its rows in "slots" rotated by its quad position, so the
// byte selectors differ per lane but the DPP reduction needs no selects.
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int DPP_XOR1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;   // quad_perm [2,3,0,1]

__device__ __forceinline__ int dpp_xor1(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, DPP_XOR1, 0xF, 0xF, true);
}
__device__ __forceinline__ int dpp_xor2(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, DPP_XOR2, 0xF, 0xF, true);
}

template <int QT>
struct TileRegs;

// 4-bit tiles: 4 dwords (rows 4g..4g+3 at column pairs 4c+i) and the row scale.
template <>
struct TileRegs<TQ_Q4_0> {
    uint32_t a[4];
    uint16_t sc;
};
template <>
struct TileRegs<TQ_IQ4_NL> : TileRegs<TQ_Q4_0> {};
// Q8_0 tiles: 8 dwords (rows 2p, 2p+1 at column pairs 8h+i) and the row scale.
template <>
struct TileRegs<TQ_Q8_0> {
    uint32_t a[8];
    uint16_t sc;
};

template <int QT>
__device__ __forceinline__ void load_tile(TileRegs<QT> &r, const uint8_t *tile, int l)
{
    if constexpr (QT == TQ_Q8_0) {
        const int p = l >> 1, h = l & 1;
        const uint32_t *t = (const uint32_t *)tile;
#pragma unroll
        for (int i = 0; i < 8; i++)
            r.a[i] = __builtin_nontemporal_load(t + (8 * h + i) * 16 + p);
    } else {
        const int g = l >> 2, c = l & 3;
        const uint32_t *t = (const uint32_t *)tile;
#pragma unroll
        for (int i = 0; i < 4; i++)
            r.a[i] = __builtin_nontemporal_load(t + (4 * c + i) * 8 + g);
    }
    r.sc = ((const uint16_t *)(tile + Fmt<QT>::scale_off))[l];
}

template <int QT, int MM>
struct ActRegs;
template <int MM>
struct ActRegs<TQ_Q4_0, MM> {
    uint32_t e[MM], o[MM];   // even / odd K of this lane's 8 activations
    uint16_t d[MM];
};
template <int MM>
struct ActRegs<TQ_IQ4_NL, MM> : ActRegs<TQ_Q4_0, MM> {};
template <int MM>
struct ActRegs<TQ_Q8_0, MM> {
    uint32_t v[MM][4];       // 16 consecutive K
    uint16_t d[MM];
};

template <int QT, int MM, bool DOTS>
__device__ __forceinline__ void load_act(ActRegs<QT, MM> &r, const int8_t *q, const uint16_t *d,
                                         int64_t K, int64_t nb, int t, int l)
{
#pragma unroll
    for (int m = 0; m < MM; m++) {
        const int8_t *qb = q + m * K + (int64_t)t * 32;
        if constexpr (QT == TQ_Q8_0) {
            const uint4 v = *(const uint4 *)(qb + 16 * (l & 1));
            r.v[m][0] = v.x;
            r.v[m][1] = v.y;
            r.v[m][2] = v.z;
            r.v[m][3] = v.w;
        } else {
            const uint2 v = *(const uint2 *)(qb + 8 * (l & 3));
            r.e[m] = __builtin_amdgcn_perm(v.y, v.x, 0x06040200u);
            r.o[m] = __builtin_amdgcn_perm(v.y, v.x, 0x07050301u);
        }
        r.d[m] = DOTS ? (uint16_t)0 : d[m * nb + t];   // no scales in block-dot mode
    }
}

// Exact block dots of this lane's row for every m.  For Q4_0 the result is
// 16x the block dot (nibbles are used as 16*(code-8) in the high half of a
// byte); the caller folds the 1/16 into the row scale, which is exact.
template <int QT, int MM>
__device__ __forceinline__ void block_dots(int (&s)[MM], const TileRegs<QT> &w,
                                           const ActRegs<QT, MM> &x, uint32_t sel0,
                                           uint32_t sel1, const Lut &lut)
{
    if constexpr (QT == TQ_Q8_0) {
        // slot j: row 2p + (j ^ h); word pair i: K 16h+4i .. 16h+4i+3
        uint32_t wd[2][4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            wd[0][i] = __builtin_amdgcn_perm(w.a[2 * i + 1], w.a[2 * i], sel0);
            wd[1][i] = __builtin_amdgcn_perm(w.a[2 * i + 1], w.a[2 * i], sel1);
        }
#pragma unroll
        for (int m = 0; m < MM; m++) {
            int p0 = 0, p1 = 0;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                p0 = __builtin_amdgcn_sdot4((int)wd[0][i], (int)x.v[m][i], p0, false);
                p1 = __builtin_amdgcn_sdot4((int)wd[1][i], (int)x.v[m][i], p1, false);
            }
            s[m] = p0 + dpp_xor1(p1);
        }
    } else {
        // 4x4 byte transpose: slot j gets [a0, a1, a2, a3] byte (j ^ c),
        // i.e. row 4g + (j ^ c) at column pairs 4c..4c+3.
        const uint32_t u0 = __builtin_amdgcn_perm(w.a[1], w.a[0], sel0);
        const uint32_t v0 = __builtin_amdgcn_perm(w.a[1], w.a[0], sel1);
        const uint32_t u1 = __builtin_amdgcn_perm(w.a[3], w.a[2], sel0);
        const uint32_t v1 = __builtin_amdgcn_perm(w.a[3], w.a[2], sel1);
        uint32_t tr[4];
        tr[0] = __builtin_amdgcn_perm(u1, u0, 0x05040100u);
        tr[1] = __builtin_amdgcn_perm(u1, u0, 0x07060302u);
        tr[2] = __builtin_amdgcn_perm(v1, v0, 0x05040100u);
        tr[3] = __builtin_amdgcn_perm(v1, v0, 0x07060302u);
        uint32_t ev[4], od[4];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            if constexpr (QT == TQ_Q4_0) {
                const uint32_t t = tr[j] ^ 0x88888888u;       // nibble c -> c - 8 (4-bit two's complement)
                ev[j] = (t << 4) & 0xF0F0F0F0u;               // 16 * (even-column code - 8)
                od[j] = t & 0xF0F0F0F0u;                      // 16 * (odd-column code - 8)
            } else {
                ev[j] = lut16(tr[j] & 0x0F0F0F0Fu, lut);
                od[j] = lut16((tr[j] >> 4) & 0x0F0F0F0Fu, lut);
            }
        }
#pragma unroll
        for (int m = 0; m < MM; m++) {
            int p[4];
#pragma unroll
            for (int j = 0; j < 4; j++)
                p[j] = __builtin_amdgcn_sdot4((int)od[j], (int)x.o[m],
                                              __builtin_amdgcn_sdot4((int)ev[j], (int)x.e[m], 0, false),
                                              false);
            const int r0 = p[0] + dpp_xor2(p[2]);
            const int r1 = p[1] + dpp_xor2(p[3]);
            s[m] = r0 + dpp_xor1(r1);
        }
    }
}

template <int QT, int MM, int NW, bool DOTS>
__global__ __launch_bounds__(NW * 64) void k_qgemv(const uint8_t *__restrict__ tiles, int nkt,
                                                   int64_t N, const int8_t *__restrict__ q,
                                                   const uint16_t *__restrict__ d, int64_t K,
                                                   Lut lut, float *__restrict__ y, int64_t ldy,
                                                   int32_t *__restrict__ isum)
{
    constexpr int TS = Fmt<QT>::tile;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int half = lane >> 5, l = lane & 31;
    const int64_t ct = blockIdx.x;
    const uint8_t *stripe = tiles + ct * (int64_t)nkt * TS;
    const int64_t nb = nkt;

    // lane-dependent byte selectors of the row slots
    uint32_t sel0, sel1;
    if constexpr (QT == TQ_Q8_0) {
        const int h = l & 1;
        sel0 = h ? 0x07060302u : 0x05040100u;
        sel1 = h ? 0x05040100u : 0x07060302u;
    } else {
        const uint32_t c = l & 3;
        const uint32_t b0 = c, b1 = 1 ^ c, b2 = 2 ^ c, b3 = 3 ^ c;
        sel0 = b0 | ((4 + b0) << 8) | (b1 << 16) | ((4 + b1) << 24);
        sel1 = b2 | ((4 + b2) << 8) | (b3 << 16) | ((4 + b3) << 24);
    }

    float acc[MM];
#pragma unroll
    for (int m = 0; m < MM; m++)
        acc[m] = 0.0f;

    const int step = 2 * NW;
    int t = 2 * wave + half;
    TileRegs<QT> wc;
    ActRegs<QT, MM> xc;
    if (t < nkt) {
        load_tile<QT>(wc, stripe + (int64_t)t * TS, l);
        load_act<QT, MM, DOTS>(xc, q, d, K, nb, t, l);
    }
    for (; t < nkt; t += step) {
        TileRegs<QT> wn;
        ActRegs<QT, MM> xn;
        const int tn = t + step;
        if (tn < nkt) {
            load_tile<QT>(wn, stripe + (int64_t)tn * TS, l);
            load_act<QT, MM, DOTS>(xn, q, d, K, nb, tn, l);
        }
        int s[MM];
        block_dots<QT, MM>(s, wc, xc, sel0, sel1, lut);
        if constexpr (DOTS) {
            const int64_t n = 32 * ct + l;
            if (n < N) {
#pragma unroll
                for (int m = 0; m < MM; m++)
                    isum[((int64_t)m * N + n) * nb + t] = (QT == TQ_Q4_0) ? (s[m] >> 4) : s[m];
            }
        } else {
            float dw = f16_bits_to_f32(wc.sc);
            if constexpr (QT == TQ_Q4_0)
                dw *= 0.0625f;
#pragma unroll
            for (int m = 0; m < MM; m++)
                acc[m] = fmaf((float)s[m], dw * f16_bits_to_f32(xc.d[m]), acc[m]);
        }
        wc = wn;
        xc = xn;
    }
    if constexpr (DOTS)
        return;

    __shared__ float red[2 * NW][MM][32];
#pragma unroll
    for (int m = 0; m < MM; m++)
        red[2 * wave + half][m][l] = acc[m];
    __syncthreads();
    for (int i = threadIdx.x; i < MM * 32; i += NW * 64) {
        const int m = i >> 5, r = i & 31;
        float sum = 0.0f;
#pragma unroll
        for (int c = 0; c < 2 * NW; c++)
            sum += red[c][m][r];
        const int64_t n = 32 * ct + r;
        if (n < N)
            y[m * ldy + n] = sum;
    }
}

constexpr int NW = 8;

template <int QT, int MM>
hipError_t launch_m(const void *tiles, int64_t K, int64_t N, const int8_t *q, const uint16_t *d,
                    const Lut &lut, float *y, int64_t ldy, int32_t *isum, hipStream_t s)
{
    const int nkt = (int)(K / 32);
    dim3 grid((unsigned)((N + 31) / 32));
    if (isum)
        k_qgemv<QT, MM, NW, true><<<grid, NW * 64, 0, s>>>((const uint8_t *)tiles, nkt, N, q, d,
                                                           K, lut, y, ldy, isum);
    else
        k_qgemv<QT, MM, NW, false><<<grid, NW * 64, 0, s>>>((const uint8_t *)tiles, nkt, N, q, d,
                                                            K, lut, y, ldy, isum);
    return hipGetLastError();
}

template <int QT>
hipError_t launch_t(const void *tiles, int64_t K, int64_t N, const int8_t *q, const uint16_t *d,
                    int64_t M, const Lut &lut, float *y, int64_t ldy, int32_t *isum,
                    hipStream_t s)
{
    switch (M) {
    case 1: return launch_m<QT, 1>(tiles, K, N, q, d, lut, y, ldy, isum, s);
    case 2: return launch_m<QT, 2>(tiles, K, N, q, d, lut, y, ldy, isum, s);
    case 3: return launch_m<QT, 3>(tiles, K, N, q, d, lut, y, ldy, isum, s);
    case 4: return launch_m<QT, 4>(tiles, K, N, q, d, lut, y, ldy, isum, s);
    case 5: return launch_m<QT, 5>(tiles, K, N, q, d, lut, y, ldy, isum, s);
    case 6: return launch_m<QT, 6>(tiles, K, N, q, d, lut, y, ldy, isum, s);
    case 7: return launch_m<QT, 7>(tiles, K, N, q, d, lut, y, ldy, isum, s);
    case 8: return launch_m<QT, 8>(tiles, K, N, q, d, lut, y, ldy, isum, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_qgemv(int type, const void *tiles, int64_t K, int64_t N, const int8_t *q,
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
