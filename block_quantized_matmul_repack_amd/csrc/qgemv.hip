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
// exact int32 block dot of row l, scales it by its fp16 row scale (MXFP4:
// the power of two of its E8M0 byte) times the fp16 activation scale (exact
// in fp32) and accumulates in fp32.  IQ4_NL and MXFP4 codes become int8
// through a 16-entry table (MXFP4: 2 * E2M1, its half going to the scale).
//   4-bit lanes: l = 4g + c reads rows 4g..4g+3 at column pairs 4c..4c+3
//   (K 8c..8c+7).  Q8_0 lanes: l = 2p + h reads rows 2p, 2p+1 at column
//   pairs 8h..8h+7 (K 16h..16h+15).  Each lane keeps its rows in slots
//   rotated by its quad position, so byte selectors differ per lane and the
//   DPP reduction needs no selects.
//
// Work split.  Workgroup (ct, ks) takes k-tiles [ks*C, (ks+1)*C) of stripe
// ct.  Its waves' partial sums are added in a fixed order through LDS.  With
// S > 1 workgroups per stripe the S partials are added in a fixed pairwise
// tree through a workspace (see the end of k_qgemv), so results are
// deterministic for every S and the workspace is all-zero after every call.
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

// LDS for one pass of staged activations (int8 q and fp32 scales, all M rows).
// Up to 4 rows: 32 KB (three workgroups fit a CU's LDS); 5..8 rows: 40 KB,
// enough for one pass over K = 4096 at M = 8.
template <int MM>
constexpr int act_lds_bytes()
{
    return MM <= 4 ? 32768 : 40960;
}

// Weight units each wave keeps in flight (ring depth), per tile type.
#ifndef TQ_GEMV_DEPTH_Q8
#define TQ_GEMV_DEPTH_Q8 2
#endif
#ifndef TQ_GEMV_DEPTH_Q4
#define TQ_GEMV_DEPTH_Q4 2
#endif
template <int QT>
constexpr int ring_depth()
{
    return QT == TQ_Q8_0 ? TQ_GEMV_DEPTH_Q8 : TQ_GEMV_DEPTH_Q4;
}

// Activation batches (one 32-element block per quad of lanes) that the fused
// kernels load together before quantizing them.
#ifndef TQ_GEMV_XG
#define TQ_GEMV_XG 4
#endif

// Tiles with at least this many activation rows go through the int8 matrix
// cores (one v_mfma_i32_32x32x32_i8 per tile, rows past M zero) instead of
// v_dot4; fewer rows stay on v_dot4, where the matrix core would mostly
// multiply zeros.  Q8_0's v_dot4 path needs no nibble decode and stays
// ahead up to 4 rows (measured level at M = 4, the matrix cores 14-20 %
// faster at M = 8).
#ifndef TQ_GEMV_MMA_MIN_M
#define TQ_GEMV_MMA_MIN_M 2
#endif
#ifndef TQ_GEMV_MMA_MIN_M_Q8
#define TQ_GEMV_MMA_MIN_M_Q8 5
#endif
template <int QT, int MM>
constexpr bool use_mma()
{
    return MM >= (QT == TQ_Q8_0 ? TQ_GEMV_MMA_MIN_M_Q8 : TQ_GEMV_MMA_MIN_M);
}

typedef int v2i_t __attribute__((ext_vector_type(2)));
typedef int v4i_t __attribute__((ext_vector_type(4)));
typedef int v16i_t __attribute__((ext_vector_type(16)));

// Matrix-core operand of a staged 4-bit tile.  ds_read_b64_tr_b8 hands lane
// j of each 16-lane group byte j % 8 of the 8-byte rows that lanes 2i + (j
// >= 8) of the group point at (i = 0..7).  Pointing lane 2i + p of group G
// at the tile's 8 bytes (column pair 8 (G / 2) + i, rows 8 (2 (G % 2) + p)
// ..) gives lane l the column pairs 16 (l / 32) / 2 .. + 7 of row l % 32: its
// 16 K values K0 + 0 .. 15, K0 = 16 (l / 32), as nibbles.  The byte offset
// of that row in the tile:
__device__ __forceinline__ int tr8_offset(int lane)
{
    const int G = lane >> 4, s = lane & 15;
    return (8 * (G >> 1) + (s >> 1)) * 32 + 8 * (2 * (G & 1) + (s & 1));
}

// The 16 int8 of that operand, in the matrix-core K order used throughout:
// K0 + {0, 2, 4, 6}, {8, .., 14}, {1, .., 7}, {9, .., 15} (the activations
// are staged in the same order).  Q4_0 values are 16 (code - 8), like the
// v_dot4 path.
template <int QT>
__device__ __forceinline__ v4i_t tile_operand(const uint8_t *tile, int off, const Lut &lut)
{
    const v2i_t w = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
        (__attribute__((address_space(3))) v2i_t *)(tile + off));
    uint32_t lo[2], hi[2];
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const uint32_t x = (uint32_t)w[i];
        if constexpr (QT == TQ_Q4_0) {
            lo[i] = ((x << 4) ^ 0x80808080u) & 0xF0F0F0F0u;
            hi[i] = (x ^ 0x80808080u) & 0xF0F0F0F0u;
        } else if constexpr (QT == TQ_Q4_1) {
            lo[i] = x & 0x0F0F0F0Fu;
            hi[i] = (x >> 4) & 0x0F0F0F0Fu;
        } else {
            lut16x2(x, lut, lo[i], hi[i]);
        }
    }
    return v4i_t{(int)lo[0], (int)lo[1], (int)hi[0], (int)hi[1]};
}

// The same operand for a staged Q8_0 tile, whose byte cp * 64 + 2 r + e is
// element 2 cp + e of row r: lane l (row r = l % 32, K0 = 16 (l / 32)) reads
// the dwords holding column pairs 8 (l / 32) .. + 7 of its row pair and keeps
// its row's halfword of each, K0 + 0 .. 15 in natural order (the staged Q8_0
// activations are in natural order too).
__device__ __forceinline__ v4i_t tile_operand_q8(const uint8_t *tile, int lane)
{
    const int r = lane & 31, cp0 = 8 * (lane >> 5);
    const uint32_t *t = (const uint32_t *)tile + (r >> 1);
    const uint32_t sel = (r & 1) ? 0x07060302u : 0x05040100u;
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; i++)
        w[i] = t[(cp0 + i) * 16];
    return v4i_t{(int)__builtin_amdgcn_perm(w[1], w[0], sel), (int)__builtin_amdgcn_perm(w[3], w[2], sel),
                 (int)__builtin_amdgcn_perm(w[5], w[4], sel), (int)__builtin_amdgcn_perm(w[7], w[6], sel)};
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
template <>
struct TileRegs<TQ_MXFP4> : TileRegs<TQ_Q4_0> {};
template <>
struct TileRegs<TQ_Q4_1> : TileRegs<TQ_Q4_0> {
    uint16_t mn;             // the row's min
};
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
        // slot i holds column pair 4c + ((i + c) & 3): the 4 lanes of a quad
        // (c = 0..3) read 4 different bank groups instead of one address 32
        // dwords apart each, so the 32 lanes of a half read 32 banks; the
        // staged activations carry the same rotation (rot_act)
        const int g = l >> 2, c = l & 3;
#pragma unroll
        for (int i = 0; i < 4; i++)
            r.a[i] = t[(4 * c + ((i + c) & 3)) * 8 + g];
    }
    r.sc = tile_scale_bits<QT>(tile, l);
    if constexpr (QT == TQ_Q4_1)
        r.mn = tile_min_bits(tile, l);
}

template <int QT, int MM>
struct ActRegs;
template <int MM>
struct ActRegs<TQ_Q4_0, MM> {
    uint2 v[MM];             // this lane's 8 K: x = the even K, y = the odd K
    float d[MM];
};
template <int MM>
struct ActRegs<TQ_IQ4_NL, MM> : ActRegs<TQ_Q4_0, MM> {};
template <int MM>
struct ActRegs<TQ_MXFP4, MM> : ActRegs<TQ_Q4_0, MM> {};
template <int MM>
struct ActRegs<TQ_Q4_1, MM> : ActRegs<TQ_Q4_0, MM> {
    float s[MM];             // da * (sum of the block's 32 int8), exact
};
template <int MM>
struct ActRegs<TQ_Q8_0, MM> {
    uint32_t v[MM][4];       // 16 consecutive K
    float d[MM];
};

// Staged activations of one pass: tile tp's 32 int8 of row m at
// qs[(tp * MM + m) * 32] -- for 4-bit weights as the 16 even K then the 16
// odd K, each word c rotated by rot_act, so that a lane's even and odd words
// come out of LDS ready for the nibble dot products -- and its scale, as
// fp32, at ds[tp * MM + m]; for Q4_1 also da times the sum of its 32 int8
// at ss[tp * MM + m].
template <int QT, int MM>
__device__ __forceinline__ void lds_act(ActRegs<QT, MM> &r, const int8_t *qs, const float *ds,
                                        const float *ss, int tp, int l)
{
#pragma unroll
    for (int m = 0; m < MM; m++) {
        const int8_t *qb = qs + (tp * MM + m) * 32;
        if constexpr (QT == TQ_Q8_0) {
            const uint4 v = *(const uint4 *)(qb + 16 * (l & 1));
            r.v[m][0] = v.x;
            r.v[m][1] = v.y;
            r.v[m][2] = v.z;
            r.v[m][3] = v.w;
        } else {
            r.v[m].x = *(const uint32_t *)(qb + 4 * (l & 3));
            r.v[m].y = *(const uint32_t *)(qb + 16 + 4 * (l & 3));
        }
        r.d[m] = ds[tp * MM + m];
        if constexpr (QT == TQ_Q4_1)
            r.s[m] = ss[tp * MM + m];
    }
}

// Activation word c (4 even or 4 odd K of K 8c .. 8c + 7) of a tile, as the
// v_dot4 path stages it for 4-bit weights: rotated right by c bytes, so that
// its byte b meets the weights of column pair 4c + ((b + c) & 3), the order
// in which lds_tile reads them.
__device__ __forceinline__ uint32_t rot_act(uint32_t w, int c)
{
    return __builtin_amdgcn_alignbyte(w, w, (uint32_t)c);
}

// Even-K / odd-K split of 8 consecutive int8 (K 8c .. 8c + 7) into the two
// words the 4-bit layout of the staged activations keeps.
__device__ __forceinline__ uint2 split_even_odd(uint2 v)
{
    return make_uint2(__builtin_amdgcn_perm(v.y, v.x, 0x06040200u),
                      __builtin_amdgcn_perm(v.y, v.x, 0x07050301u));
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
                // nibble c in the high half of a byte, its top bit flipped:
                // the byte is 16 * (c - 8) (4-bit two's complement)
                ev[j] = ((tr[j] << 4) ^ 0x80808080u) & 0xF0F0F0F0u;   // even column
                od[j] = (tr[j] ^ 0x80808080u) & 0xF0F0F0F0u;          // odd column
            } else if constexpr (QT == TQ_Q4_1) {
                ev[j] = tr[j] & 0x0F0F0F0Fu;                  // the codes themselves
                od[j] = (tr[j] >> 4) & 0x0F0F0F0Fu;
            } else {
                lut16x2(tr[j], lut, ev[j], od[j]);
            }
        }
#pragma unroll
        for (int m = 0; m < MM; m++) {
            const uint32_t xe = x.v[m].x;                 // even K
            const uint32_t xo = x.v[m].y;                 // odd K
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
    static constexpr int BYTES = 2 * Fmt<QT>::tile;       // 1152 (4-bit), 2176 (Q8_0), 1088 (MXFP4), 1280 (Q4_1)
    static constexpr int CHUNKS = BYTES / 16;             // 72, 136, 68
    static constexpr int SLOTS = (CHUNKS + 63) / 64;      // 2, 3, 2
    v4u c[SLOTS];
};

// Every chunk of the unit is stored: a tile missing from the workgroup's
// range (the second of a last, odd unit) was loaded as zeros.
template <int QT>
__device__ __forceinline__ void store_unit(const Unit<QT> &u, uint8_t *dst, int lane)
{
#pragma unroll
    for (int i = 0; i < Unit<QT>::SLOTS; i++) {
        const int ch = i * 64 + lane;
        if (ch < Unit<QT>::CHUNKS)
            *((v4u *)dst + ch) = u.c[i];
    }
}

// XT < 0: activations arrive quantized (act.q, act.d).  XT = a tq_dtype: raw
// activations act.x are quantized here, per pass, straight into LDS with the
// same quant_quad() as tq_quantize_act, so q and d are bit-identical.
template <int QT, int MM, int NW, int XT, bool DOTS>
__global__ __launch_bounds__(NW * 64) void k_qgemv(const uint8_t *__restrict__ tiles, int nkt,
                                                   int64_t N, Act act, int64_t K, Lut lut,
                                                   float *__restrict__ y, int64_t ldy,
                                                   int32_t *__restrict__ isum, int chunk, int S,
                                                   uint64_t *__restrict__ ws_slots)
{
    constexpr int TS = Fmt<QT>::tile;
    constexpr int UB = Unit<QT>::BYTES;
    constexpr int D = ring_depth<QT>();
    constexpr bool MMA = use_mma<QT, MM>();
    constexpr int ACC = MMA ? 4 : MM;                     // fp32 sums per lane
    constexpr int NSLOT = MMA ? NW : 2 * NW;              // partial sums per output
    // staged 4-bit activations: the even K of a 16-K half at HS * h, the odd
    // K ODD bytes further (v_dot4: all even K, then all odd K; matrix cores:
    // each 16-K half as 8 even then 8 odd)
    constexpr int HS = MMA ? 16 : 8, ODD = MMA ? 8 : 16;
    static_assert(NW * 64 >= MM * 32, "one thread per output of the stripe");
    __shared__ __attribute__((aligned(16))) uint8_t stage[NW][UB];
    __shared__ __attribute__((aligned(16))) uint8_t act_lds[act_lds_bytes<MM>()];
    __shared__ float red[NSLOT][MM][32];
    __shared__ __attribute__((aligned(16))) uint32_t zero16[4];   // A rows past M
    // stores of staging work-items with nothing to stage land here, so that
    // their loads are used on every path (a load used only under a branch
    // gets sunk into it, behind the weight loads)
    __shared__ __attribute__((aligned(16))) uint8_t sink_lds[48];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int half = lane >> 5, l = lane & 31;
    const int hs = 2 * wave + half;                       // half-wave slot in the workgroup
    const int64_t ct = blockIdx.x / S;
    const int ks = blockIdx.x - (int)(ct * S);
    const int kt0 = ks * chunk;
    const int nt = max(0, min(chunk, nkt - kt0));         // tiles of this workgroup
    const int64_t nct = (N + 31) / 32;
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

    float acc[ACC];
#pragma unroll
    for (int m = 0; m < ACC; m++)
        acc[m] = 0.0f;
    if (threadIdx.x < 4)
        zero16[threadIdx.x] = 0;                          // read after the staging barrier

    uint8_t *my = stage[wave];
    const int tro = tr8_offset(lane);                     // matrix-core path only
    int row_clamped[4];                                   // matrix-core path: this lane's rows
#pragma unroll
    for (int r = 0; r < 4; r++)
        row_clamped[r] = min(4 * half + r, MM - 1);
    // Weight loads are raw buffer loads over this workgroup's tiles: an
    // offset at or past the range's end returns zeros and moves no data, so
    // every load is issued unconditionally.
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(cbase, (int64_t)nt * TS);
    int chunk_off[Unit<QT>::SLOTS];                       // this lane's chunk of a unit
#pragma unroll
    for (int s = 0; s < Unit<QT>::SLOTS; s++)
        chunk_off[s] = s * 64 + lane < Unit<QT>::CHUNKS ? 16 * (s * 64 + lane) : BUF_OOB;
    // The chunk is processed in passes of up to P tiles.  Each pass first
    // stages the pass's int8 activations and scales of all M rows in LDS
    // (layout at lds_act), so the unit loop has only weight loads in flight.
    // per tile and row: 32 int8, the fp32 scale and, for Q4_1, the block sum
    constexpr int PB = QT == TQ_Q4_1 ? 40 : 36;
    constexpr int P = act_lds_bytes<MM>() / (MM * PB) & ~1;
    int8_t *qs = (int8_t *)act_lds;
    float *ds = (float *)(act_lds + MM * P * 32);
    float *ss = ds + MM * P;                              // Q4_1 only
    // one 16-byte chunk (K 16 h .. 16 h + 15 of a tile) of row m into qs
    auto put_chunk = [&](int tp, int m, int h, uint4 v, bool in = true) {
        int8_t *qb = in ? qs + (tp * MM + m) * 32 : (int8_t *)sink_lds;
        if constexpr (QT == TQ_Q8_0) {
            *(uint4 *)(qb + 16 * h) = v;
        } else {
            uint2 a = split_even_odd(make_uint2(v.x, v.y));     // words 2h
            uint2 b = split_even_odd(make_uint2(v.z, v.w));     // and 2h + 1
            if constexpr (!MMA) {
                a = make_uint2(rot_act(a.x, 2 * h), rot_act(a.y, 2 * h));
                b = make_uint2(rot_act(b.x, 2 * h + 1), rot_act(b.y, 2 * h + 1));
            }
            *(uint2 *)(qb + HS * h) = make_uint2(a.x, b.x);
            *(uint2 *)(qb + HS * h + ODD) = make_uint2(a.y, b.y);
        }
    };
    for (int pb = 0; pb < nt; pb += P) {
        const int pn = min(P, nt - pb);                   // tiles in this pass
        const int nunits = (pn + 1) >> 1;
        const int count = wave < nunits ? (nunits - 1 - wave) / NW + 1 : 0;   // units of this wave
        // the wave's i-th unit of the pass (i >= count: nothing)
        // The unit's byte offset is wave-uniform; a lane adds its fixed
        // chunk offset (lanes past the unit's chunks: BUF_OOB).  A unit past
        // the wave's count starts at the end of the range, and a last unit
        // of one tile reads its second tile past the end: zeros either way.
        auto load_stage = [&](Unit<QT> &u, int i) {
            const int j = wave + i * NW;                  // pass-local unit index
            const int base = i < count ? (pb + 2 * j) * TS : nt * TS;
#pragma unroll
            for (int s = 0; s < Unit<QT>::SLOTS; s++)
                u.c[s] = __builtin_bit_cast(
                    v4u, __builtin_amdgcn_raw_buffer_load_b128(
                             wr, (int)((unsigned)chunk_off[s] + (unsigned)base), 0, BUF_NT));
        };
        __syncthreads();                                  // previous pass done with qs / ds

        // Activations: the first batch is loaded before the weight units, so
        // waiting for it does not wait for the weights; the D units of the
        // wave are then all in flight while the activations are staged.
        Unit<QT> u[D];
        if constexpr (XT < 0) {
            // The pass's 2 MM pn 16-byte chunks of q in staged order: chunk c
            // is half c % 2 of row (c / 2) % MM of tile c / (2 MM), and scale
            // s is row s % MM of tile s / MM (ds[s]).  Consecutive threads
            // take consecutive chunks: every load is a distinct 16 bytes (a
            // wave's load reads 32 / MM consecutive tiles of each row, runs
            // of 1024 / MM bytes, whole 128-byte lines) and the LDS stores
            // are contiguous.  The first batch, loaded before the weight
            // units, holds QB1 chunks and SB1 scales per thread: all of a
            // pass of up to NT / 4 tiles (NT / 2 at MM = 1); the rest of a
            // longer pass is loaded after it.
            const int64_t q0 = (int64_t)(kt0 + pb) * 32;
            const int nch = 2 * MM * pn, nsc = MM * pn;
            constexpr int NT = NW * 64;
            constexpr int QB1 = (MM + 1) / 2, SB1 = (MM + 3) / 4;
            auto qload = [&](int c) {
                c = min(c, nch - 1);
                const int tm = c >> 1, tp = tm / MM, m = tm - tp * MM;
                return *(const uint4 *)(act.q + m * K + q0 + 32 * tp + 16 * (c & 1));
            };
            auto dload = [&](int s) -> uint16_t {
                s = min(s, nsc - 1);
                const int tp = s / MM, m = s - tp * MM;
                return DOTS ? (uint16_t)0 : act.d[m * nb + kt0 + pb + tp];
            };
            const int o = threadIdx.x;
            uint4 qv[QB1];
            uint16_t dv[SB1];
#pragma unroll
            for (int i = 0; i < QB1; i++)
                qv[i] = qload(o + i * NT);
#pragma unroll
            for (int i = 0; i < SB1; i++)
                dv[i] = dload(o + i * NT);
#pragma unroll
            for (int r = 0; r < D; r++)
                load_stage(u[r], r);
            // Q4_1: the sum of a tile row's 32 int8 from its two chunks, held
            // by neighbouring threads (c, c ^ 1; NT is even, so pairs are in
            // range together)
            auto put_sum = [&](int c, const uint4 &v) {
                if constexpr (QT == TQ_Q4_1 && !DOTS) {
                    int p = byte_sum(v.x, byte_sum(v.y, byte_sum(v.z, byte_sum(v.w, 0))));
                    p += dpp_xor1(p);
                    if (c < nch && (c & 1) == 0)
                        ss[c >> 1] = (float)p;
                }
            };
            auto put = [&](int c, const uint4 &v, bool in) {
                const int tm = c >> 1, tp = tm / MM;
                put_chunk(tp, tm - tp * MM, c & 1, v, in);
            };
#pragma unroll
            for (int i = 0; i < QB1; i++) {
                const int c = o + i * NT;
                put(c, qv[i], c < nch);
                put_sum(c, qv[i]);
            }
#pragma unroll
            for (int i = 0; i < SB1; i++) {
                const int sc = o + i * NT;
                *(sc < nsc ? &ds[sc] : (float *)(sink_lds + 32)) = f16_bits_to_f32(dv[i]);
            }
            for (int c = o + QB1 * NT; c < nch; c += NT) {
                const uint4 v2 = qload(c);
                put(c, v2, true);
                put_sum(c, v2);
            }
            for (int sc = o + SB1 * NT; sc < nsc; sc += NT)
                ds[sc] = f16_bits_to_f32(dload(sc));
        } else {
            // one 32-element block per quad of lanes, 8 elements per lane
            // (quant_quad); block b = tp * MM + m, QB blocks per batch
            constexpr int QB = NW * 16;
            const int nblk = MM * pn;
            const int c = lane & 3, bq = threadIdx.x >> 2;
            auto xload = [&](float (&v)[8], int b) {
                b = min(b, nblk - 1);
                const int tp = b / MM, m = b - tp * MM;
                load_x8<XT>(v, act.x, m * act.ldx + (int64_t)(kt0 + pb + tp) * 32 + 8 * c);
            };
            // quantized unconditionally (a branch here would let the compiler
            // sink the load below the weight loads); stored if in range
            auto xquant = [&](const float (&v)[8], int b) {
                uint2 qv;
                uint16_t db;
                quant_quad(v, qv, db);
                if constexpr (QT == TQ_Q4_1) {
                    int p = byte_sum(qv.x, byte_sum(qv.y, 0));
                    p += dpp_xor1(p);                     // the quad's 32 int8
                    p += dpp_xor2(p);
                    if (b < nblk && c == 0)
                        ss[b] = (float)p;
                }
                if (b < nblk) {
                    int8_t *qb = qs + b * 32;
                    if constexpr (QT == TQ_Q8_0) {
                        *(uint2 *)(qb + 8 * c) = qv;
                    } else {
                        uint2 eo = split_even_odd(qv);
                        if constexpr (!MMA)
                            eo = make_uint2(rot_act(eo.x, c), rot_act(eo.y, c));
                        *(uint32_t *)(qb + HS * (c >> 1) + 4 * (c & 1)) = eo.x;
                        *(uint32_t *)(qb + HS * (c >> 1) + 4 * (c & 1) + ODD) = eo.y;
                    }
                    if (c == 0)
                        ds[b] = f16_bits_to_f32(db);
                }
            };
            // XG batches in flight at once: with several rows the pass has
            // M batches, and loading them one after another would put a
            // cache round trip per batch in front of the weight stream
            constexpr int XG = MM < TQ_GEMV_XG ? MM : TQ_GEMV_XG;
            float v[XG][8];
#pragma unroll
            for (int g = 0; g < XG; g++)
                xload(v[g], bq + g * QB);
#pragma unroll
            for (int r = 0; r < D; r++)
                load_stage(u[r], r);
#pragma unroll
            for (int g = 0; g < XG; g++)
                xquant(v[g], bq + g * QB);
            for (int b = bq + XG * QB; b < nblk; b += XG * QB) {
#pragma unroll
                for (int g = 0; g < XG; g++)
                    xload(v[g], b + g * QB);
#pragma unroll
                for (int g = 0; g < XG; g++)
                    xquant(v[g], b + g * QB);
            }
        }
        __syncthreads();

        // the unit is already in this wave's LDS slice (the ring loop below)
        auto process = [&](int j) {
            if constexpr (MMA) {
                // the whole wave takes both tiles of the unit: lane l holds
                // output row n = l % 32 for activation rows 4 (l / 32) + r.
                // Both tiles' operands are read and both MFMAs issued before
                // either result is used, so the second tile's reads overlap
                // the first MFMA.
                v16i_t dot[2];
#pragma unroll
                for (int t = 0; t < 2; t++) {
                    const int tp = min(2 * j + t, pn - 1);
                    v4i_t b;
                    if constexpr (QT == TQ_Q8_0)
                        b = tile_operand_q8(my + t * TS, lane);
                    else
                        b = tile_operand<QT>(my + t * TS, tro, lut);
                    const int8_t *ap = l < MM ? qs + (tp * MM + l) * 32 + 16 * half
                                              : (const int8_t *)zero16;
                    const v4i_t a = *(const v4i_t *)ap;
                    dot[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, v16i_t{}, 0, 0, 0);
                }
                // Only dot[t][0..3] are used, but each MFMA writes all 16
                // registers.  Reading them all here keeps the compiler from
                // handing the unused ones to other values before the MFMAs
                // have finished writing them (a variant without this gave
                // wrong sums at M = 8).
                asm volatile("" ::"v"(dot[0]), "v"(dot[1]));
#pragma unroll
                for (int t = 0; t < 2; t++) {
                    const int tp = min(2 * j + t, pn - 1);
                    const bool valid = 2 * j + t < pn;
                    const uint8_t *tile = my + t * TS;
                    if constexpr (DOTS) {
                        const int64_t n = 32 * ct + l;
#pragma unroll
                        for (int r = 0; r < 4; r++) {
                            const int m = 4 * half + r;
                            if (valid && m < MM && n < N)
                                isum[((int64_t)m * N + n) * nb + kt0 + pb + tp] =
                                    (QT == TQ_Q4_0) ? (dot[t][r] >> 4) : dot[t][r];
                        }
                    } else {
                        // a missing second tile was staged as zeros: scale
                        // (and min) 0, adds 0; the weights' power-of-two
                        // factor is applied to the sums at the end (exact)
                        const float dw = f16_bits_to_f32(tile_scale_bits<QT>(tile, l));
                        float mw = 0.0f;
                        if constexpr (QT == TQ_Q4_1)
                            mw = f16_bits_to_f32(tile_min_bits(tile, l));
                        // rows past M read row M - 1's scale: their dots are
                        // 0 (zero A rows) and their sums are never stored.
                        // M = 4 / 8: the half's 4 rows are contiguous (16-byte
                        // aligned), one read; at M = 4 half 1 holds no row and
                        // takes half 0's scales
                        float da[4], sa[4];
                        if constexpr (MM == 4 || MM == 8) {
                            const int mi0 = tp * MM + (MM == 8 ? 4 * half : 0);
                            const float4 v = *(const float4 *)(ds + mi0);
                            da[0] = v.x, da[1] = v.y, da[2] = v.z, da[3] = v.w;
                            if constexpr (QT == TQ_Q4_1) {
                                const float4 w4 = *(const float4 *)(ss + mi0);
                                sa[0] = w4.x, sa[1] = w4.y, sa[2] = w4.z, sa[3] = w4.w;
                            }
                        } else {
#pragma unroll
                            for (int r = 0; r < 4; r++) {
                                const int mi = tp * MM + row_clamped[r];
                                da[r] = ds[mi];
                                if constexpr (QT == TQ_Q4_1)
                                    sa[r] = ss[mi];
                            }
                        }
#pragma unroll
                        for (int r = 0; r < 4; r++) {
                            acc[r] = fmaf((float)dot[t][r], dw * da[r], acc[r]);
                            if constexpr (QT == TQ_Q4_1)
                                acc[r] = fmaf(mw, da[r] * sa[r], acc[r]);   // the min
                        }
                    }
                }
            } else {
                const int tp = min(2 * j + half, pn - 1);     // this half's tile, pass-local
                const bool valid = 2 * j + half < pn;
                TileRegs<QT> w;
                lds_tile<QT>(w, my + half * TS, l);
                ActRegs<QT, MM> x;
                lds_act<QT, MM>(x, qs, ds, ss, tp, l);
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
                    // a missing second tile was staged as zeros: scale 0, adds 0;
                    // the weights' power-of-two factor is applied to the sums
                    // at the end (exact)
                    const float dw = f16_bits_to_f32(w.sc);
#pragma unroll
                    for (int m = 0; m < MM; m++)
                        acc[m] = fmaf((float)s[m], dw * x.d[m], acc[m]);
                    if constexpr (QT == TQ_Q4_1) {
                        // the min: m_w * da * sum(q), da * sum exact in fp32
                        const float mw = f16_bits_to_f32(w.mn);
#pragma unroll
                        for (int m = 0; m < MM; m++)
                            acc[m] = fmaf(mw, x.d[m] * x.s[m], acc[m]);
                    }
                }
            }
        };
        // A ring of D unit buffers: buffer r holds the wave's units r, r + D,
        // ...; once a buffer's unit is copied to LDS the buffer is refilled
        // with the unit D further on, before that unit is computed, so D
        // units stay in flight during the compute.  Loads are never under a
        // branch (past-the-end units are zero-size), which lets the compiler
        // wait for exactly the oldest buffer.
        for (int it = 0; it < count; it += D) {
#pragma unroll
            for (int r = 0; r < D; r++) {
                const int j = wave + (it + r) * NW;
                const bool live = it + r < count;
                if (live)
                    store_unit<QT>(u[r], my, lane);
                load_stage(u[r], it + r + D);
                if (live)
                    process(j);
            }
        }
    }
    if constexpr (DOTS)
        return;

    if constexpr (MMA) {
#pragma unroll
        for (int r = 0; r < 4; r++) {
            if (4 * half + r < MM)
                red[wave][min(4 * half + r, MM - 1)][l] = acc[r] * weight_unscale<QT>();
        }
    } else {
#pragma unroll
        for (int m = 0; m < MM; m++)
            red[hs][m][l] = acc[m] * weight_unscale<QT>();
    }
    __syncthreads();
    const int i = threadIdx.x;
    const int m = i >> 5, r = i & 31;
    float part = 0.0f;
    if (i < MM * 32) {
#pragma unroll
        for (int c = 0; c < NSLOT; c++)
            part += red[c][m][r];
    }
    const int64_t n = 32 * ct + r;
    if (S == 1) {
        if (i < MM * 32 && n < N)
            y[m * ldy + n] = part;
        return;
    }
    // Cross-workgroup reduction over the S = 2^L workgroups of the stripe, as
    // a pairwise tree: at level lv, workgroups ks and ks ^ 2^lv pair up.  Each
    // output exchanges (marker | value bits) into its pair's 64-bit slot with
    // a relaxed agent-scope atomic (coherent across the XCD L2s without a
    // cache write-back).  The first to arrive leaves its value there; the
    // second finds it, adds (fp32 addition is commutative, so the sum has the
    // same bits whoever arrives second), clears the slot and goes on to the
    // next level.  The result is ((p0 + p1) + (p2 + p3)) + ... in every run,
    // and the workspace is zero again when the call ends.
    if (i >= MM * 32)
        return;
    float v = part;
    uint64_t *slots = ws_slots;
    for (int lv = 0; (1 << lv) < S; lv++) {
        const int pairs = S >> (lv + 1);
        uint64_t *slot = slots + ((ct * pairs + (ks >> (lv + 1))) * MM + m) * 32 + r;
        const uint64_t mine = (uint64_t(1) << 32) | __float_as_uint(v);
        const uint64_t old =
            __hip_atomic_exchange(slot, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (old == 0)
            return;                               // first of the pair: done
        v = v + __uint_as_float((uint32_t)old);
        __hip_atomic_store(slot, uint64_t(0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        slots += (size_t)nct * pairs * MM * 32;
    }
    if (n < N)
        y[m * ldy + n] = v;
}

#ifndef TQ_GEMV_NW
#define TQ_GEMV_NW 8
#endif
#ifndef TQ_GEMV_TARGET_WG
#define TQ_GEMV_TARGET_WG 256
#endif
constexpr int NW = TQ_GEMV_NW;                   // waves per workgroup
constexpr int64_t TARGET_WG = TQ_GEMV_TARGET_WG; // workgroups wanted for a full chip

template <int QT, int MM, int XT, bool DOTS>
hipError_t launch_k(const void *tiles, int64_t K, int64_t N, const Act &act, const Lut &lut,
                    float *y, int64_t ldy, int32_t *isum, const Split &sp, hipStream_t s)
{
    const int nkt = (int)(K / 32);
    const int64_t nct = (N + 31) / 32;
    if (!grid_fits(nct * sp.S, NW * 64))
        return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)(nct * sp.S));
    k_qgemv<QT, MM, NW, XT, DOTS><<<grid, NW * 64, 0, s>>>((const uint8_t *)tiles, nkt, N, act, K,
                                                           lut, y, ldy, isum, sp.chunk, sp.S,
                                                           sp.slots);
    return hipGetLastError();
}

template <int QT, int MM>
hipError_t launch_m(const void *tiles, int64_t K, int64_t N, const Act &act, const Lut &lut,
                    float *y, int64_t ldy, int32_t *isum, const Split &sp, hipStream_t s)
{
    if (isum)
        return launch_k<QT, MM, -1, true>(tiles, K, N, act, lut, y, ldy, isum, sp, s);
    switch (act.xt) {
    case -1: return launch_k<QT, MM, -1, false>(tiles, K, N, act, lut, y, ldy, isum, sp, s);
    case TQ_F32: return launch_k<QT, MM, TQ_F32, false>(tiles, K, N, act, lut, y, ldy, isum, sp, s);
    case TQ_BF16: return launch_k<QT, MM, TQ_BF16, false>(tiles, K, N, act, lut, y, ldy, isum, sp, s);
    case TQ_F16: return launch_k<QT, MM, TQ_F16, false>(tiles, K, N, act, lut, y, ldy, isum, sp, s);
    }
    return hipErrorInvalidValue;
}

template <int QT>
hipError_t launch_t(const void *tiles, int64_t K, int64_t N, const Act &act, int64_t M,
                    const Lut &lut, float *y, int64_t ldy, int32_t *isum, const Split &sp,
                    hipStream_t s)
{
    switch (M) {
    case 1: return launch_m<QT, 1>(tiles, K, N, act, lut, y, ldy, isum, sp, s);
    case 2: return launch_m<QT, 2>(tiles, K, N, act, lut, y, ldy, isum, sp, s);
    case 3: return launch_m<QT, 3>(tiles, K, N, act, lut, y, ldy, isum, sp, s);
    case 4: return launch_m<QT, 4>(tiles, K, N, act, lut, y, ldy, isum, sp, s);
    case 5: return launch_m<QT, 5>(tiles, K, N, act, lut, y, ldy, isum, sp, s);
    case 6: return launch_m<QT, 6>(tiles, K, N, act, lut, y, ldy, isum, sp, s);
    case 7: return launch_m<QT, 7>(tiles, K, N, act, lut, y, ldy, isum, sp, s);
    case 8: return launch_m<QT, 8>(tiles, K, N, act, lut, y, ldy, isum, sp, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

// K-split geometry: S = 1, 2, 4 or 8 workgroups per stripe, enough for about
// TARGET_WG workgroups in all, chunks of an even number of k-tiles (whole
// units).  Workgroups whose chunk starts past K contribute zero.
Split gemv_split(int64_t K, int64_t N)
{
    Split sp{};
    const int64_t nkt = K / 32, nct = (N + 31) / 32;
    sp.S = 1;
    if (nkt >= 1 && nct >= 1)
        while (sp.S < 8 && nct * sp.S < TARGET_WG && 2 * sp.S <= (nkt + 1) / 2)
            sp.S *= 2;
    int64_t chunk = (nkt + sp.S - 1) / sp.S;
    chunk += chunk & 1;
    sp.chunk = (int)std::max<int64_t>(chunk, 1);
    return sp;
}

// Workspace: the tree's 64-bit slots, (S - 1) * M * 32 per stripe.
size_t gemv_workspace_bytes(int64_t K, int64_t N, int64_t M)
{
    const Split sp = gemv_split(K, N);
    if (sp.S <= 1)
        return 0;
    return (size_t)((N + 31) / 32) * (sp.S - 1) * M * 32 * 8;
}

hipError_t launch_qgemv(int type, const void *tiles, int64_t K, int64_t N, const Act &act,
                        int64_t M, const Lut &lut, float *y, int64_t ldy, int32_t *isum,
                        void *ws, size_t ws_bytes, hipStream_t s)
{
    Split sp = gemv_split(K, N);
    if (!isum && sp.S > 1) {
        if (!ws || ws_bytes < gemv_workspace_bytes(K, N, M)) {
            // no room for the split: one workgroup per stripe
            sp.S = 1;
            sp.chunk = (int)(K / 32);
        } else {
            sp.slots = (uint64_t *)ws;
        }
    }
    switch (type) {
    case TQ_Q4_0: return launch_t<TQ_Q4_0>(tiles, K, N, act, M, lut, y, ldy, isum, sp, s);
    case TQ_Q8_0: return launch_t<TQ_Q8_0>(tiles, K, N, act, M, lut, y, ldy, isum, sp, s);
    case TQ_IQ4_NL: return launch_t<TQ_IQ4_NL>(tiles, K, N, act, M, lut, y, ldy, isum, sp, s);
    case TQ_MXFP4: return launch_t<TQ_MXFP4>(tiles, K, N, act, M, lut, y, ldy, isum, sp, s);
    case TQ_Q4_1: return launch_t<TQ_Q4_1>(tiles, K, N, act, M, lut, y, ldy, isum, sp, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace tq
