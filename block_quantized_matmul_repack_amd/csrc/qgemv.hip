// Decode matrix-vector product over 32x32 tiles, M <= 8 activation rows.
//
// Layout facts used ("Tiled Weight Formats" / "Block-32 Quantized Formats"):
// a 32-row stripe's K/32 tiles are contiguous; inside a tile the quant bytes
// are ordered [column pair][row], so one dword holds 4 rows (4-bit types) or
// 2 rows (Q8_0) of one column pair.  The integer dot wants one row's
// consecutive K values in a dword (v_dot4_i32_i8).
//
// Data path.  Each wave streams "units" of two consecutive tiles with
// contiguous 16-byte nontemporal loads (every load instruction covers 1 KB of
// HBM), stages the unit in its own slice of LDS, and reads it back in the
// transposing order the dot needs: half-wave h takes tile h of the unit.
// The next unit's loads are in flight while the current one is computed.
//
// Arithmetic.  A lane reads the dwords of 4 rows (4-bit) or 2 rows (Q8_0) for
// a quarter / half of the tile's column pairs, transposes bytes with
// v_perm_b32, forms partial dots with v_dot4_i32_i8 and finishes each row's
// 32-element block dot with quad DPP adds.  Lane l of the half then holds the
// exact int32 block dot of row l, scales it by its fp16 row scale times the
// fp16 activation scale (exact in fp32) and accumulates in fp32.
//   4-bit lanes: l = 4g + c reads rows 4g..4g+3 at column pairs 4c..4c+3
//   (K 8c..8c+7).  Q8_0 lanes: l = 2p + h reads rows 2p, 2p+1 at column
//   pairs 8h..8h+7 (K 16h..16h+15).  Each lane keeps its rows in slots
//   rotated by its quad position, so byte selectors differ per lane and the
//   DPP reduction needs no selects.
//
// Work split.  Workgroup (ct, ks) takes k-tiles [ks*C, (ks+1)*C) of stripe
// ct.  Its waves' partial sums are added in a fixed order through LDS.  With
// S > 1 workgroups per stripe the partials go to a workspace and the last
// workgroup to finish (atomic counter) adds the S partials in ks order, so
// results are deterministic for every S; it then zeroes the partials and the
// counter, so the workspace is all-zero again after every call.
#include <algorithm>

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

typedef unsigned v4u __attribute__((ext_vector_type(4)));

// Largest S * M * 32 of a split: the last workgroup gathers that many partials
// into LDS.
constexpr int MAX_SPLIT_OUT = 2048;
// LDS for one pass of staged activations (int8 q and fp16 scales, all M rows).
constexpr int ACT_LDS_BYTES = 32768;

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

// Read this lane's dwords of one tile from its LDS copy.
template <int QT>
__device__ __forceinline__ void lds_tile(TileRegs<QT> &r, const uint8_t *tile, int l)
{
    const uint32_t *t = (const uint32_t *)tile;
    if constexpr (QT == TQ_Q8_0) {
        const int p = l >> 1, h = l & 1;
#pragma unroll
        for (int i = 0; i < 8; i++)
            r.a[i] = t[(8 * h + i) * 16 + p];
    } else {
        const int g = l >> 2, c = l & 3;
#pragma unroll
        for (int i = 0; i < 4; i++)
            r.a[i] = t[(4 * c + i) * 8 + g];
    }
    r.sc = ((const uint16_t *)(tile + Fmt<QT>::scale_off))[l];
}

template <int QT, int MM>
struct ActRegs;
template <int MM>
struct ActRegs<TQ_Q4_0, MM> {
    uint2 v[MM];             // this lane's 8 consecutive K (split into even / odd K at use)
    uint16_t d[MM];
};
template <int MM>
struct ActRegs<TQ_IQ4_NL, MM> : ActRegs<TQ_Q4_0, MM> {};
template <int MM>
struct ActRegs<TQ_Q8_0, MM> {
    uint32_t v[MM][4];       // 16 consecutive K
    uint16_t d[MM];
};

// Activations of tile tp (pass-local) from the workgroup's LDS copy:
// qs[m][tp*32 + K], ds[m][tp].
template <int QT, int MM>
__device__ __forceinline__ void lds_act(ActRegs<QT, MM> &r, const int8_t *qs, const uint16_t *ds,
                                        int pstride, int tp, int l)
{
#pragma unroll
    for (int m = 0; m < MM; m++) {
        const int8_t *qb = qs + m * pstride * 32 + tp * 32;
        if constexpr (QT == TQ_Q8_0) {
            const uint4 v = *(const uint4 *)(qb + 16 * (l & 1));
            r.v[m][0] = v.x;
            r.v[m][1] = v.y;
            r.v[m][2] = v.z;
            r.v[m][3] = v.w;
        } else {
            r.v[m] = *(const uint2 *)(qb + 8 * (l & 3));
        }
        r.d[m] = ds[m * pstride + tp];
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
            const uint32_t xe = __builtin_amdgcn_perm(x.v[m].y, x.v[m].x, 0x06040200u);  // even K
            const uint32_t xo = __builtin_amdgcn_perm(x.v[m].y, x.v[m].x, 0x07050301u);  // odd K
            int p[4];
#pragma unroll
            for (int j = 0; j < 4; j++)
                p[j] = __builtin_amdgcn_sdot4((int)od[j], (int)xo,
                                              __builtin_amdgcn_sdot4((int)ev[j], (int)xe, 0, false),
                                              false);
            const int r0 = p[0] + dpp_xor2(p[2]);
            const int r1 = p[1] + dpp_xor2(p[3]);
            s[m] = r0 + dpp_xor1(r1);
        }
    }
}

// One unit = two consecutive tiles, loaded as 16-byte chunks: chunk i of the
// unit goes to lane i % 64, register slot i / 64.
template <int QT>
struct Unit {
    static constexpr int BYTES = 2 * Fmt<QT>::tile;       // 1152 (4-bit), 2176 (Q8_0)
    static constexpr int CHUNKS = BYTES / 16;             // 72, 136
    static constexpr int SLOTS = (CHUNKS + 63) / 64;      // 2, 3
    v4u c[SLOTS];
};

// Branch-free: lanes past the unit's valid bytes re-read its last chunk (and
// do not store it), so every path issues the same loads and the compiler can
// wait for exactly the loads it needs.
template <int QT>
__device__ __forceinline__ void load_unit(Unit<QT> &u, const uint8_t *src, int valid_chunks,
                                          int lane)
{
#pragma unroll
    for (int i = 0; i < Unit<QT>::SLOTS; i++) {
        const int ch = min(i * 64 + lane, valid_chunks - 1);
        u.c[i] = __builtin_nontemporal_load((const v4u *)src + ch);
    }
}

template <int QT>
__device__ __forceinline__ void store_unit(const Unit<QT> &u, uint8_t *dst, int valid_chunks,
                                           int lane)
{
#pragma unroll
    for (int i = 0; i < Unit<QT>::SLOTS; i++) {
        const int ch = i * 64 + lane;
        if (ch < valid_chunks)
            *((v4u *)dst + ch) = u.c[i];
    }
}

template <int QT, int MM, int NW, bool DOTS>
__global__ __launch_bounds__(NW * 64) void k_qgemv(const uint8_t *__restrict__ tiles, int nkt,
                                                   int64_t N, const int8_t *__restrict__ q,
                                                   const uint16_t *__restrict__ d, int64_t K,
                                                   Lut lut, float *__restrict__ y, int64_t ldy,
                                                   int32_t *__restrict__ isum, int chunk, int S,
                                                   float *__restrict__ ws_part,
                                                   uint32_t *__restrict__ ws_cnt)
{
    constexpr int TS = Fmt<QT>::tile;
    constexpr int UB = Unit<QT>::BYTES;
    static_assert(NW * 64 >= MM * 32, "one thread per output of the stripe");
    __shared__ __attribute__((aligned(16))) uint8_t stage[NW][UB];
    __shared__ __attribute__((aligned(16))) uint8_t act_lds[ACT_LDS_BYTES];
    __shared__ float red[2 * NW][MM][32];
    __shared__ float gath[MAX_SPLIT_OUT];
    __shared__ int last_flag;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int half = lane >> 5, l = lane & 31;
    const int64_t ct = blockIdx.x / S;
    const int ks = blockIdx.x - (int)(ct * S);
    const int kt0 = ks * chunk;
    const int nt = min(chunk, nkt - kt0);                 // tiles of this workgroup
    const uint8_t *cbase = tiles + (ct * (int64_t)nkt + kt0) * TS;
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

    uint8_t *my = stage[wave];
    // The chunk is processed in passes of up to P tiles.  Each pass first
    // copies the pass's int8 activations and fp16 scales into LDS (all M
    // rows), so the unit loop below has only weight loads in flight.
    constexpr int P = ACT_LDS_BYTES / (MM * 34) & ~1;
    int8_t *qs = (int8_t *)act_lds;
    uint16_t *ds = (uint16_t *)(act_lds + MM * P * 32);
    for (int pb = 0; pb < nt; pb += P) {
        const int pn = min(P, nt - pb);                   // tiles in this pass
        __syncthreads();                                  // previous pass done with qs / ds
        for (int c = threadIdx.x; c < MM * pn * 2; c += NW * 64) {
            const int m = c / (pn * 2), o = c - m * pn * 2;   // 16-byte chunk o of row m
            *(uint4 *)(qs + m * P * 32 + o * 16) =
                *(const uint4 *)(q + m * K + (int64_t)(kt0 + pb) * 32 + o * 16);
        }
        for (int c = threadIdx.x; c < MM * pn; c += NW * 64) {
            const int m = c / pn, o = c - m * pn;
            ds[m * P + o] = DOTS ? (uint16_t)0 : d[m * nb + kt0 + pb + o];
        }
        __syncthreads();

        // A stage is one unit of two weight tiles; all loads are unconditional
        // (indices clamped into range), the next stage is always issued before
        // the current one is used and the last is peeled, so one stage's
        // loads overlap the previous stage's compute.
        const int nunits = (pn + 1) >> 1;
        const uint8_t *pbase = cbase + (int64_t)pb * TS;
        auto load_stage = [&](Unit<QT> &u, int j) {
            load_unit<QT>(u, pbase + (int64_t)j * UB, min(2, pn - 2 * j) * (TS / 16), lane);
        };
        auto process = [&](const Unit<QT> &u, int j) {
            store_unit<QT>(u, my, min(2, pn - 2 * j) * (TS / 16), lane);
            const int tp = min(2 * j + half, pn - 1);         // this half's tile, pass-local
            const bool valid = 2 * j + half < pn;
            TileRegs<QT> w;
            lds_tile<QT>(w, my + half * TS, l);
            ActRegs<QT, MM> x;
            lds_act<QT, MM>(x, qs, ds, P, tp, l);
            int s[MM];
            block_dots<QT, MM>(s, w, x, sel0, sel1, lut);
            if constexpr (DOTS) {
                const int64_t n = 32 * ct + l;
                if (valid && n < N) {
#pragma unroll
                    for (int m = 0; m < MM; m++)
                        isum[((int64_t)m * N + n) * nb + kt0 + pb + tp] =
                            (QT == TQ_Q4_0) ? (s[m] >> 4) : s[m];
                }
            } else {
                float dw = f16_bits_to_f32(w.sc);
                if constexpr (QT == TQ_Q4_0)
                    dw *= 0.0625f;
                dw = valid ? dw : 0.0f;                       // a missing second tile adds 0
#pragma unroll
                for (int m = 0; m < MM; m++)
                    acc[m] = fmaf((float)s[m], dw * f16_bits_to_f32(x.d[m]), acc[m]);
            }
        };
        const int count = wave < nunits ? (nunits - 1 - wave) / NW + 1 : 0;   // units of this wave
        if (count > 0) {
            // two unit buffers used in turn (no register copies, which would
            // wait for the prefetch); every loop iteration prefetches
            Unit<QT> ua, ub;
            load_stage(ua, wave);
            int it = 0;
            for (; it + 2 < count; it += 2) {
                load_stage(ub, wave + (it + 1) * NW);
                process(ua, wave + it * NW);
                load_stage(ua, wave + (it + 2) * NW);
                process(ub, wave + (it + 1) * NW);
            }
            if (it + 2 == count) {
                load_stage(ub, wave + (it + 1) * NW);
                process(ua, wave + it * NW);
                process(ub, wave + (it + 1) * NW);
            } else {
                process(ua, wave + it * NW);
            }
        }
    }
    if constexpr (DOTS)
        return;

#pragma unroll
    for (int m = 0; m < MM; m++)
        red[2 * wave + half][m][l] = acc[m];
    __syncthreads();
    const int i = threadIdx.x;
    const int m = i >> 5, r = i & 31;
    float part = 0.0f;
    if (i < MM * 32) {
#pragma unroll
        for (int c = 0; c < 2 * NW; c++)
            part += red[c][m][r];
    }
    const int64_t n = 32 * ct + r;
    if (S == 1) {
        if (i < MM * 32 && n < N)
            y[m * ldy + n] = part;
        return;
    }
    // Cross-workgroup reduction.  Partials are published and collected with
    // relaxed agent-scope atomic exchanges, which are coherent across the
    // XCDs' L2 caches without a cache write-back.  Each publishing lane waits
    // for its exchange to return (the asm consumes the value) before the
    // workgroup increments the stripe's counter, so the last workgroup to
    // arrive finds every partial in place.  It adds them in ks order and
    // exchanges zeros back, leaving the workspace zero for the next call of
    // any shape (counter and partial offsets depend on the shape).
    if (i < MM * 32) {
        const float old = __hip_atomic_exchange(&ws_part[((ct * S + ks) * MM + m) * 32 + r], part,
                                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        asm volatile("" ::"v"(old));
    }
    __syncthreads();
    if (i == 0)
        last_flag = (atomicAdd(&ws_cnt[ct], 1u) == (uint32_t)(S - 1));
    __syncthreads();
    if (!last_flag)
        return;
    // gather all S * MM * 32 partials at once (one round trip), then add them
    // in ks order
    for (int g = i; g < S * MM * 32; g += NW * 64)
        gath[g] = __hip_atomic_exchange(&ws_part[(ct * S) * MM * 32 + g], 0.0f, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (i < MM * 32) {
        float sum = 0.0f;
        for (int k = 0; k < S; k++)
            sum += gath[(k * MM + m) * 32 + r];
        if (n < N)
            y[m * ldy + n] = sum;
    }
    if (i == 0)
        __hip_atomic_store(&ws_cnt[ct], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

#ifndef TQ_GEMV_NW
#define TQ_GEMV_NW 8
#endif
#ifndef TQ_GEMV_TARGET_WG
#define TQ_GEMV_TARGET_WG 256
#endif
constexpr int NW = TQ_GEMV_NW;                   // waves per workgroup
constexpr int64_t TARGET_WG = TQ_GEMV_TARGET_WG; // workgroups wanted for a full chip

template <int QT, int MM>
hipError_t launch_m(const void *tiles, int64_t K, int64_t N, const int8_t *q, const uint16_t *d,
                    const Lut &lut, float *y, int64_t ldy, int32_t *isum, const Split &sp,
                    hipStream_t s)
{
    const int nkt = (int)(K / 32);
    const int64_t nct = (N + 31) / 32;
    dim3 grid((unsigned)(nct * sp.S));
    if (isum)
        k_qgemv<QT, MM, NW, true><<<grid, NW * 64, 0, s>>>((const uint8_t *)tiles, nkt, N, q, d,
                                                           K, lut, y, ldy, isum, sp.chunk, sp.S,
                                                           sp.part, sp.cnt);
    else
        k_qgemv<QT, MM, NW, false><<<grid, NW * 64, 0, s>>>((const uint8_t *)tiles, nkt, N, q, d,
                                                            K, lut, y, ldy, isum, sp.chunk, sp.S,
                                                            sp.part, sp.cnt);
    return hipGetLastError();
}

template <int QT>
hipError_t launch_t(const void *tiles, int64_t K, int64_t N, const int8_t *q, const uint16_t *d,
                    int64_t M, const Lut &lut, float *y, int64_t ldy, int32_t *isum,
                    const Split &sp, hipStream_t s)
{
    switch (M) {
    case 1: return launch_m<QT, 1>(tiles, K, N, q, d, lut, y, ldy, isum, sp, s);
    case 2: return launch_m<QT, 2>(tiles, K, N, q, d, lut, y, ldy, isum, sp, s);
    case 3: return launch_m<QT, 3>(tiles, K, N, q, d, lut, y, ldy, isum, sp, s);
    case 4: return launch_m<QT, 4>(tiles, K, N, q, d, lut, y, ldy, isum, sp, s);
    case 5: return launch_m<QT, 5>(tiles, K, N, q, d, lut, y, ldy, isum, sp, s);
    case 6: return launch_m<QT, 6>(tiles, K, N, q, d, lut, y, ldy, isum, sp, s);
    case 7: return launch_m<QT, 7>(tiles, K, N, q, d, lut, y, ldy, isum, sp, s);
    case 8: return launch_m<QT, 8>(tiles, K, N, q, d, lut, y, ldy, isum, sp, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

// K-split geometry: enough workgroups to fill the chip (TARGET_WG), chunks of
// an even number of k-tiles (whole units), never more splits than units.
Split gemv_split(int64_t K, int64_t N)
{
    Split sp{};
    const int64_t nkt = K / 32, nct = (N + 31) / 32;
    if (nkt < 1 || nct < 1) {
        sp.S = 1;
        sp.chunk = (int)std::max<int64_t>(nkt, 1);
        return sp;
    }
    int64_t S = (TARGET_WG + nct - 1) / nct;
    S = std::min<int64_t>(S, MAX_SPLIT_OUT / (32 * 8));
    S = std::max<int64_t>(1, std::min<int64_t>(S, (nkt + 1) / 2));
    int64_t chunk = (nkt + S - 1) / S;
    chunk += chunk & 1;
    S = (nkt + chunk - 1) / chunk;
    sp.S = (int)S;
    sp.chunk = (int)chunk;
    return sp;
}

// Workspace: one uint32 counter per stripe (padded to 256 bytes), then
// S * M * 32 fp32 partial sums per stripe.
size_t gemv_workspace_bytes(int64_t K, int64_t N, int64_t M)
{
    const Split sp = gemv_split(K, N);
    if (sp.S <= 1)
        return 0;
    const int64_t nct = (N + 31) / 32;
    const size_t cnt = ((size_t)nct * 4 + 255) & ~(size_t)255;
    return cnt + (size_t)nct * sp.S * M * 32 * 4;
}

hipError_t launch_qgemv(int type, const void *tiles, int64_t K, int64_t N, const int8_t *q,
                        const uint16_t *d, int64_t M, const Lut &lut, float *y, int64_t ldy,
                        int32_t *isum, void *ws, size_t ws_bytes, hipStream_t s)
{
    Split sp = gemv_split(K, N);
    if (!isum && sp.S > 1) {
        if (!ws || ws_bytes < gemv_workspace_bytes(K, N, M)) {
            // no room for the split: one workgroup per stripe
            sp.S = 1;
            sp.chunk = (int)(K / 32);
        } else {
            const int64_t nct = (N + 31) / 32;
            const size_t cnt = ((size_t)nct * 4 + 255) & ~(size_t)255;
            sp.cnt = (uint32_t *)ws;
            sp.part = (float *)((uint8_t *)ws + cnt);
        }
    }
    switch (type) {
    case TQ_Q4_0: return launch_t<TQ_Q4_0>(tiles, K, N, q, d, M, lut, y, ldy, isum, sp, s);
    case TQ_Q8_0: return launch_t<TQ_Q8_0>(tiles, K, N, q, d, M, lut, y, ldy, isum, sp, s);
    case TQ_IQ4_NL: return launch_t<TQ_IQ4_NL>(tiles, K, N, q, d, M, lut, y, ldy, isum, sp, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace tq
