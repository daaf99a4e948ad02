// Prefill matrix-matrix product over 32x32 tiles with int8 MFMA.
//
// A workgroup of 16 waves in two groups of 8 owns a BM x BN = 128 x 64
// output block (128 activation rows x two 32-row weight stripes); wave
// (wm, wn) of each group owns one 32 x 32 sub-block, and the two groups
// split each step's k-blocks (group 0 takes one, group 1 three) and add
// their sums through LDS at the end.  The K loop advances KB = 4 k-blocks
// per step, which group 0 stages:
//   - activations: 128 rows x 4 x 32 int8, natural K order, and their fp16
//     block scales go to LDS as loaded;
//   - weights: each of the group's 8 waves takes one of the step's 8 tiles (2
//     stripes x 4 blocks).  4-bit tiles: the wave gets it as dwords of 4
//     rows of a column pair ("Block-32 Quantized Formats") -- read from the
//     tile directly, or (IQ4_NL) loaded as contiguous chunks and read back
//     from a per-wave LDS slice -- transposes bytes in registers with
//     v_perm_b32, decodes them to int8 (code - 8 or a table lookup) and
//     writes them to LDS in [row][K] order.  Q8_0 tiles go to LDS as loaded
//     and the MFMA operand is gathered from them with 16-bit transposing
//     reads.  The fp16 row scales go to LDS beside them.
// LDS is double-buffered and the global loads run two steps ahead of the
// MFMAs (two register stages), with one barrier per step.  Q4_0 weights are
// staged as 16 * (code - 8) (two bit operations per 4 weights); the 16 is
// taken out of the fp32 result at the end, exactly, as is MXFP4's 2 (its
// weights staged as the integers 2 * E2M1, its E8M0 row bytes as the fp16
// powers of two they stand for).
//
// Per k-block each wave runs one v_mfma_i32_32x32x32_i8, whose K depth equals
// the block size, so its int32 result is exactly the per-block integer dot.
// The scale products dw[n] * da[m] (fp16 x fp16, exact in fp32) for the whole
// 32 x 32 sub-block come from one rank-1 v_mfma_f32_32x32x8_f16, whose
// operands are read from LDS ready-made (each scale stored as an 8-byte
// [d, 0, 0, 0] fp16 vector next to an all-zero copy for the lanes holding
// k = 4..7), so the vector ALU only converts each dot and adds it into the
// fp32 accumulator (2 operations per output per block).  Load offsets are
// computed once per thread; a step adds only the k offset.
#include <type_traits>

#include "tq_internal.h"

namespace tq {
namespace {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));

// THREADS = a group of 8 waves that owns the 8 32 x 32 output sub-blocks;
// KSW groups of them split each step's KB k-blocks.
#ifndef TQ_GEMM_KSPLIT
#define TQ_GEMM_KSPLIT 2
#endif
constexpr int BM = 128, BN = 64, KB = 4, THREADS = 512;
constexpr int KSW = TQ_GEMM_KSPLIT;                    // wave groups
constexpr int WG_THREADS = THREADS * KSW;
static_assert(KSW == 1 || KSW == 2, "one or two wave groups");
// k-blocks of each step taken by wave group 0, which also stages the step's
// data; the other group takes the rest.  Giving the staging group fewer
// blocks evens out the groups' vector work between two barriers.  Q4_1's
// min term works on pairs of blocks, so there each group takes two, as in
// the block-dot output (no rescale to even out).
#ifndef TQ_GEMM_KB0
#define TQ_GEMM_KB0 1
#endif
template <int QT, bool DOTS>
constexpr int kb_group0()
{
    return KSW == 1 ? KB : ((QT == TQ_Q4_1 || DOTS) ? KB / 2 : TQ_GEMM_KB0);
}
static_assert(TQ_GEMM_KB0 >= 0 && TQ_GEMM_KB0 <= KB, "group 0 takes 0 .. KB k-blocks");
#ifndef TQ_GEMM_MIN_BLOCKS
#define TQ_GEMM_MIN_BLOCKS 1      // workgroups per CU the register budget is sized for
#endif
// A staged row holds the step's KB * 32 = 128 bytes of one activation or
// weight row (k-block kb at bytes 32 kb ..), padded to 144 so that the 16
// lanes of a b128 read of 16 consecutive rows hit 16 different bank groups.
constexpr int LDS_ROW = 144;

// Q8_0 and IQ4_NL tiles are loaded as contiguous chunks in lane order (16
// or 8 bytes per lane, every request whole cache lines).  IQ4_NL chunks go
// through a per-wave LDS slice and are read back in the transposing order
// the decode takes; Q8_0 tiles stay in the B buffer as loaded (see q8_tr).
// The other types load the lane's dwords straight from the tile (4 per
// 64-byte column pair row, half of each line per request), which measured
// as fast or faster for them.
template <int QT>
constexpr bool raw_tiles()
{
    return QT == TQ_Q8_0 || QT == TQ_IQ4_NL;
}
// Q8_0 tiles in the B buffer as loaded (the tile's byte layout, one 1 KB
// tile per stripe and k-block), the MFMA operand read with two
// ds_read_b64_tr_b16: the tile's halfwords are (column pair, row) pairs of
// int8, so a 16-bit transposing read gathers one row's column pairs, in K
// order, with no byte permutes in the staging wave.
template <int QT, int FT>
constexpr bool q8_tr()
{
    return QT == TQ_Q8_0 && FT < 0;
}

struct LdsMain {
    uint8_t A[2][BM * LDS_ROW];
    uint8_t B[2][BN * LDS_ROW];
    // rank-1 MFMA operands: [0][row] = the row's KB fp16 scales of the step,
    // [1][row] = 0 (read by the lanes that hold k = 4..7)
    uint64_t da[2][2][BM];
    uint64_t dw[2][2][BN];
};
// Q4_1's min term, sum_b m_w[n][b] * da[m][b] * asum[m][b], is a product
// over the k-blocks: the step's block sums of each activation row and fp16
// row mins of each weight row feed fp32 MFMAs that accumulate it.
struct LdsMin {
    float asum[2][BM][KB];
    uint64_t mw[2][BN];
};
// Each staging wave's IQ4_NL tile quants as loaded.
struct LdsRaw {
    uint32_t raw[BN / 32 * KB][Fmt<TQ_IQ4_NL>::scale_off / 4];
};
template <int QT>
struct Lds : LdsMain {};
template <>
struct Lds<TQ_Q4_1> : LdsMain, LdsMin {};
template <>
struct Lds<TQ_IQ4_NL> : LdsMain, LdsRaw {};
static_assert(BN / 32 * KB * 1024 <= BN * LDS_ROW, "Q8_0 tiles of a step fit a B buffer");

// Buffer ranges of one workgroup: its activation rows, their scales, and its
// two weight stripes.  Loads past them return zero.
struct Ranges {
    __amdgpu_buffer_rsrc_t q, d, w;
};

// Per-thread byte offsets of the loads at k-tile 0; a step at k-tile kt0 adds
// kt0 * 32 (activations), kt0 * 2 (their scales) or kt0 * tile bytes
// (weights).  Thread roles: activations are 128 rows x 4 blocks x 2 halves =
// 1024 chunks of 16 bytes (chunk ch: row ch/8, block (ch/2)%4, half ch%2),
// two per thread, plus one block scale per thread (row t/4, block t%4).
// Weights: wave w takes the tile of stripe w/4, block w%4; lane 32*hh + l
// reads, for tile lane l, half hh of that lane's column pairs.
// FT: -1 = weights as tiles; else weights as flat GGML blocks of type FT
// (row n's blocks contiguous; FT = TQ_Q4_K runs with QT = TQ_Q4_1).  Flat
// thread roles: weight row tid / 8 (of the 64), k-block (tid / 2) % 4, half
// tid % 2 of the block's quant bytes (4-bit: 8 bytes = elements 8h .. 8h + 7
// and 16 + 8h ..; Q8_0 and Q4_K: 16 elements from 16h).
template <int QT, int FT>
struct Offs {
    static constexpr int NWD = (QT == TQ_Q8_0 || FT == TQ_Q4_K) ? 4 : 2;
    int a[2], da, w[NWD], dw, wt;
    int kba, kbw;                 // k-block of this thread's activation / weight scale
    int hw, rowsb;                // flat: half, and (Q4_K) the row's first super-block
};

template <int QT, int FT>
__device__ __forceinline__ Offs<QT, FT> make_offs(int64_t nkt, int64_t K, int tid)
{
    constexpr int TS = Fmt<QT>::tile;
    Offs<QT, FT> o;
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int ch = tid + THREADS * i;
        const int row = ch >> 3, kb = (ch >> 1) & 3, h = ch & 1;
        o.a[i] = (int)(row * K) + kb * 32 + 16 * h;
    }
    o.kba = tid & 3;
    o.da = (int)((tid >> 2) * nkt + o.kba) * 2;
    if constexpr (FT >= 0) {
        constexpr int BB = Fmt<FT>::block;
        const int rr = tid >> 3, kb = (tid >> 1) & 3, h = tid & 1;
        o.kbw = kb;
        o.hw = h;
        if constexpr (FT == TQ_Q4_K) {
            o.rowsb = (int)(rr * (nkt / 8)) * BB;
            o.w[0] = o.dw = 0;                    // per step: super-block of kt0 + kb
        } else {
            const int blk = (int)(rr * nkt + kb) * BB;
            constexpr int QOFF = FT == TQ_MXFP4 ? 1 : (FT == TQ_Q4_1 ? 4 : 2);
            o.w[0] = blk + QOFF + (FT == TQ_Q8_0 ? 16 : 8) * h;
            o.dw = blk;
        }
        return o;
    }
    const int wave = tid >> 6, lane = tid & 63;
    const int tt = wave >> 2, l = lane & 31, hh = lane >> 5;
    o.kbw = wave & 3;
    const int tile = (int)(tt * nkt + o.kbw) * TS;
    // o.w: the lane's quant dwords, relative to the tile (Q8_0 tiles are
    // loaded and staged whole)
    o.wt = tile;
    if constexpr (QT == TQ_Q8_0) {
#pragma unroll
        for (int i = 0; i < 4; i++)
            o.w[i] = 0;
    } else {
        const int g = l >> 2, c = l & 3;
#pragma unroll
        for (int i = 0; i < 2; i++)
            o.w[i] = ((4 * c + 2 * hh + i) * 8 + g) * 4;
    }
    o.dw = tile + Fmt<QT>::scale_off + (QT == TQ_MXFP4 ? l : (QT == TQ_Q4_1 ? 4 * l : 2 * l));
    return o;
}

template <int QT, int FT>
struct StageRegs {
    uint4 a[2];               // activations: 2 x 16 bytes
    uint16_t da;              // one activation block scale
    uint32_t w[Offs<QT, FT>::NWD]; // weight dwords (tiles, 4-bit: rows 4g..4g+3 at column
                              // pairs 4c+2hh, 4c+2hh+1; Q8_0: the lane's 16 bytes of
                              // the tile in order; flat: the thread's quant bytes in order)
    uint16_t dw;              // weight row scale (MXFP4: its E8M0 byte)
    uint16_t mw;              // Q4_1: weight row min
    uint4 hdr;                // flat Q4_K: the super-block's d, dmin and scale bytes
    int sub;                  // flat Q4_K: sub-block (0..7) of this step's block
    bool da_ok, dw_ok;        // the scales' k-blocks lie inside K
};

// Every load is a raw buffer load issued by every thread, the step's k
// offset (uniform) in the scalar offset and the thread's own offset in the
// vector one, so that a step adds no vector work.  Offsets past a
// range read as zero (rows >= M, stripes past N).  A block kt >= kend (the
// end of this workgroup's k-range) in the last step reads finite bytes of
// the next k-range, row or stripe, or zero, and its two scales are forced to
// zero, so it adds exactly 0; so there are no branches around loads and the
// compiler can wait for exactly the older stage.
template <int QT, bool DOTS, int FT>
__device__ __forceinline__ void load_step(StageRegs<QT, FT> &s, const Ranges &rg,
                                          const Offs<QT, FT> &o, int kend, int kt0)
{
    constexpr int TS = Fmt<QT>::tile;
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const v4i v = __builtin_amdgcn_raw_buffer_load_b128(rg.q, o.a[i], kt0 * 32, 0);
        s.a[i] = make_uint4(v.x, v.y, v.z, v.w);
    }
    if constexpr (DOTS) {
        s.da = 0;
        s.dw = 0;
        s.da_ok = s.dw_ok = false;
    } else {
        // zeroed for blocks past K at store time (a select here would wait
        // for the load)
        s.da = __builtin_amdgcn_raw_buffer_load_b16(rg.d, o.da, kt0 * 2, 0);
        s.da_ok = kt0 + o.kba < kend;
        s.dw_ok = kt0 + o.kbw < kend;
    }
    if constexpr (FT >= 0) {
        // flat blocks: this thread's quant bytes and the block's scales
        constexpr int BB = Fmt<FT>::block;
        if constexpr (FT == TQ_Q4_K) {
            const int kk = kt0 + o.kbw;
            s.sub = kk & 7;
            const int sbo = o.rowsb + (kk >> 3) * BB;
            const v4i v = __builtin_amdgcn_raw_buffer_load_b128(
                rg.w, sbo + 16 + 32 * ((kk & 7) >> 1) + 16 * o.hw, 0, BUF_NT);
            s.w[0] = v.x, s.w[1] = v.y, s.w[2] = v.z, s.w[3] = v.w;
            if constexpr (!DOTS) {
                const v4i h = __builtin_amdgcn_raw_buffer_load_b128(rg.w, sbo, 0, 0);
                s.hdr = make_uint4(h.x, h.y, h.z, h.w);
            }
        } else if constexpr (FT == TQ_MXFP4) {
            // 17-byte blocks start at any byte: byte loads
            uint32_t b[8];
#pragma unroll
            for (int i = 0; i < 8; i++)
                b[i] = __builtin_amdgcn_raw_buffer_load_b8(rg.w, o.w[0] + kt0 * BB + i, 0, 0);
            s.w[0] = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
            s.w[1] = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
            if constexpr (!DOTS)
                s.dw = __builtin_amdgcn_raw_buffer_load_b8(rg.w, o.dw + kt0 * BB, 0, 0);
        } else if constexpr (FT == TQ_Q8_0) {
            const v4i v = __builtin_amdgcn_raw_buffer_load_b128(rg.w, o.w[0] + kt0 * BB, 0, BUF_NT);
            s.w[0] = v.x, s.w[1] = v.y, s.w[2] = v.z, s.w[3] = v.w;
            if constexpr (!DOTS)
                s.dw = __builtin_amdgcn_raw_buffer_load_b16(rg.w, o.dw + kt0 * BB, 0, 0);
        } else {
            const auto v = __builtin_amdgcn_raw_buffer_load_b64(rg.w, o.w[0] + kt0 * BB, 0, BUF_NT);
            s.w[0] = (uint32_t)v[0], s.w[1] = (uint32_t)v[1];
            if constexpr (!DOTS) {
                s.dw = __builtin_amdgcn_raw_buffer_load_b16(rg.w, o.dw + kt0 * BB, 0, 0);
                if constexpr (FT == TQ_Q4_1)
                    s.mw = __builtin_amdgcn_raw_buffer_load_b16(rg.w, o.dw + 2 + kt0 * BB, 0, 0);
            }
        }
        return;
    }
    if constexpr (!DOTS) {
        if constexpr (QT == TQ_MXFP4)
            s.dw = __builtin_amdgcn_raw_buffer_load_b8(rg.w, o.dw, kt0 * TS, 0);
        else
            s.dw = __builtin_amdgcn_raw_buffer_load_b16(rg.w, o.dw, kt0 * TS, 0);
        if constexpr (QT == TQ_Q4_1)
            s.mw = __builtin_amdgcn_raw_buffer_load_b16(rg.w, o.dw + 2, kt0 * TS, 0);
    }
    if constexpr (raw_tiles<QT>()) {
        // the tile's quant bytes as contiguous chunks in lane order
        const int lane = threadIdx.x & 63;
        if constexpr (QT == TQ_Q8_0) {
            const v4i v =
                __builtin_amdgcn_raw_buffer_load_b128(rg.w, o.wt + 16 * lane, kt0 * TS, BUF_NT);
            s.w[0] = v.x, s.w[1] = v.y, s.w[2] = v.z, s.w[3] = v.w;
        } else {
            const auto v =
                __builtin_amdgcn_raw_buffer_load_b64(rg.w, o.wt + 8 * lane, kt0 * TS, BUF_NT);
            s.w[0] = (uint32_t)v[0], s.w[1] = (uint32_t)v[1];
        }
    } else {
#pragma unroll
        for (int i = 0; i < Offs<QT, FT>::NWD; i++)
            s.w[i] = __builtin_amdgcn_raw_buffer_load_b32(rg.w, o.wt + o.w[i], kt0 * TS, BUF_NT);
    }
}

// 8 quant bytes of a flat 4-bit block half (elements 8h .. 8h + 7 in the
// low nibbles, 16 + 8h .. in the high ones) as int8 weights: lo / hi dwords
// for K 8h + 4i .. and 16 + 8h + 4i .., i = 0, 1.
template <int QT>
__device__ __forceinline__ void decode_flat4(uint32_t v, const Lut &lut, uint32_t &lo,
                                             uint32_t &hi)
{
    if constexpr (QT == TQ_Q4_0) {
        const uint32_t t = v ^ 0x88888888u;
        lo = (t << 4) & 0xF0F0F0F0u;
        hi = t & 0xF0F0F0F0u;
    } else if constexpr (QT == TQ_Q4_1) {
        lo = v & 0x0F0F0F0Fu;
        hi = (v >> 4) & 0x0F0F0F0Fu;
    } else {
        lut16x2(v, lut, lo, hi);
    }
}

template <int QT, bool DOTS, int FT>
__device__ __forceinline__ void store_step(const StageRegs<QT, FT> &s0, Lds<QT> &L, int buf,
                                           const Lut &lut, int tid, const Offs<QT, FT> &o)
{
    // IQ4_NL tiles: the loaded chunks go to the wave's LDS slice, and the
    // lane's dwords are read back from it in the transposing order (a wave's
    // LDS operations take effect in program order)
    StageRegs<QT, FT> s = s0;
    if constexpr (FT < 0 && QT == TQ_IQ4_NL) {
        const int lane = tid & 63;
        uint32_t *raw = L.raw[tid >> 6];
        *(uint2 *)(raw + 2 * lane) = make_uint2(s0.w[0], s0.w[1]);
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int i = 0; i < Offs<QT, FT>::NWD; i++)
            s.w[i] = raw[o.w[i] / 4];
    }
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int ch = tid + THREADS * i;
        const int row = ch >> 3, kb = (ch >> 1) & 3, h = ch & 1;
        *(uint4 *)(L.A[buf] + row * LDS_ROW + 32 * kb + 16 * h) = s.a[i];
        if constexpr (QT == TQ_Q4_1 && !DOTS) {
            // block sum: this chunk's 16 int8 plus the other half's, held by
            // the neighbouring thread (ch ^ 1); both threads store the same
            // value (a branch here would split the loop body).  Blocks past
            // K get sums of whatever was read there, but their scales are 0.
            const uint4 a = s.a[i];
            int p = byte_sum(a.x, byte_sum(a.y, byte_sum(a.z, byte_sum(a.w, 0))));
            p += __builtin_amdgcn_update_dpp(0, p, 0xB1, 0xF, 0xF, true);
            L.asum[buf][row][kb] = (float)p;
        }
    }
    ((uint16_t *)&L.da[buf][0][tid >> 2])[tid & 3] = s.da_ok ? s.da : (uint16_t)0;
    if constexpr (FT >= 0) {
        // flat: weight row rr's block kb in [row][K] order (both halves of a
        // block store its scales: the same bits, no branch)
        const int rr = tid >> 3, kb = (tid >> 1) & 3, h = tid & 1;
        uint8_t *B = L.B[buf] + rr * LDS_ROW + 32 * kb;
        uint16_t dwb = s.dw, mwb = s.mw;
        if constexpr (FT == TQ_Q8_0) {
            *(uint4 *)(B + 16 * h) = make_uint4(s.w[0], s.w[1], s.w[2], s.w[3]);
        } else if constexpr (FT == TQ_Q4_K) {
            // sub-block `sub` = nibble sub % 2 of its chunk's bytes
            uint32_t e[4];
#pragma unroll
            for (int i = 0; i < 4; i++)
                e[i] = (s.sub & 1) ? ((s.w[i] >> 4) & 0x0F0F0F0Fu) : (s.w[i] & 0x0F0F0F0Fu);
            *(uint4 *)(B + 16 * h) = make_uint4(e[0], e[1], e[2], e[3]);
            if constexpr (!DOTS) {
                const uint32_t s3[3] = {s.hdr.y, s.hdr.z, s.hdr.w};
                uint32_t sc, mn;
                q4k_scale_min(s3, s.sub, sc, mn);
                dwb = f16_of_product(f16_bits_to_f32((uint16_t)s.hdr.x), (float)sc);
                mwb = f16_of_product(-f16_bits_to_f32((uint16_t)(s.hdr.x >> 16)), (float)mn);
            }
        } else {
            uint32_t lo0, hi0, lo1, hi1;
            decode_flat4<QT>(s.w[0], lut, lo0, hi0);
            decode_flat4<QT>(s.w[1], lut, lo1, hi1);
            *(uint2 *)(B + 8 * h) = make_uint2(lo0, lo1);
            *(uint2 *)(B + 16 + 8 * h) = make_uint2(hi0, hi1);
            if constexpr (FT == TQ_MXFP4)
                dwb = e8m0_f16_bits(s.dw);
        }
        ((uint16_t *)&L.dw[buf][0][rr])[kb] = s.dw_ok ? dwb : (uint16_t)0;
        if constexpr (QT == TQ_Q4_1)
            ((uint16_t *)&L.mw[buf][rr])[kb] = s.dw_ok ? mwb : (uint16_t)0;
        return;
    }
    const int wave = tid >> 6, lane = tid & 63;
    const int tt = wave >> 2, kb = wave & 3, l = lane & 31, hh = lane >> 5;
    uint8_t *B = L.B[buf] + (32 * tt) * LDS_ROW + 32 * kb;
    if constexpr (q8_tr<QT, FT>()) {
        // the tile as loaded: tile (stripe tt, k-block kb) at 1 KB (tt KB + kb)
        *(v4i *)(L.B[buf] + (tt * KB + kb) * 1024 + 16 * lane) =
            v4i{(int)s.w[0], (int)s.w[1], (int)s.w[2], (int)s.w[3]};
    } else {
        // rows 4g+j: byte j of the two column-pair dwords holds K = 2cp (low
        // nibble) and 2cp+1 (high nibble) for cp = 4c+2hh, 4c+2hh+1, i.e. the
        // 4 consecutive K = 8c+4hh .. 8c+4hh+3
        const int g = l >> 2, c = l & 3;
        const uint32_t p01 = __builtin_amdgcn_perm(s.w[1], s.w[0], 0x05010400u);  // rows 0, 1
        const uint32_t p23 = __builtin_amdgcn_perm(s.w[1], s.w[0], 0x07030602u);  // rows 2, 3
#pragma unroll
        for (int r = 0; r < 2; r++) {
            const uint32_t pr = r ? p23 : p01;
            uint32_t lo, hi;          // per byte: even-K / odd-K weight
            if constexpr (QT == TQ_Q4_0) {
                const uint32_t t = pr ^ 0x88888888u;      // nibble c -> c - 8 (4-bit two's complement)
                lo = (t << 4) & 0xF0F0F0F0u;              // 16 * (even-column code - 8)
                hi = t & 0xF0F0F0F0u;                     // 16 * (odd-column code - 8)
            } else if constexpr (QT == TQ_Q4_1) {
                lo = pr & 0x0F0F0F0Fu;                    // the codes themselves
                hi = (pr >> 4) & 0x0F0F0F0Fu;
            } else {
                lut16x2(pr, lut, lo, hi);
            }
            const uint32_t r0 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);  // row 2r:   K +0..+3
            const uint32_t r1 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);  // row 2r+1: K +0..+3
            *(uint32_t *)(B + (4 * g + 2 * r) * LDS_ROW + 8 * c + 4 * hh) = r0;
            *(uint32_t *)(B + (4 * g + 2 * r + 1) * LDS_ROW + 8 * c + 4 * hh) = r1;
        }
    }
    // both halves of the wave hold the same row scale: the duplicate store
    // writes the same bits and keeps the step free of branches
    const uint16_t dwb = (QT == TQ_MXFP4) ? e8m0_f16_bits(s.dw) : s.dw;
    ((uint16_t *)&L.dw[buf][0][32 * tt + l])[kb] = s.dw_ok ? dwb : (uint16_t)0;
    if constexpr (QT == TQ_Q4_1)
        ((uint16_t *)&L.mw[buf][32 * tt + l])[kb] = s.dw_ok ? s.mw : (uint16_t)0;
}

template <int QT, bool DOTS, int FT>
__global__ __launch_bounds__(WG_THREADS, TQ_GEMM_MIN_BLOCKS) void k_qgemm(const uint8_t *__restrict__ tiles,
                                                   int64_t nkt, int64_t N,
                                                   const int8_t *__restrict__ q,
                                                   const uint16_t *__restrict__ d, int64_t M,
                                                   int64_t K, Lut lut, float *__restrict__ y,
                                                   int64_t ldy, int32_t *__restrict__ isum,
                                                   int64_t kchunk, int64_t ysplit)
{
    __shared__ __attribute__((aligned(16))) Lds<QT> L;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = (tid >> 6) & 7;
    const int grp = tid / THREADS;       // wave group (0 stages the data)
    const int wm = wave & 3, wn = wave >> 2;
    const int li = lane & 31, lk = lane >> 5;
    const int64_t nct = (N + 31) / 32;
    const int64_t ct0 = (int64_t)blockIdx.x * (BN / 32);
    const int64_t m0 = (int64_t)blockIdx.y * BM;
    // k-range of this workgroup: k-tiles [kbeg, kend) (blockIdx.z-th of the
    // split; the whole of K without one); a split writes its own partial
    // plane of y, ysplit elements further per range
    const int64_t kbeg = (int64_t)blockIdx.z * kchunk;
    const int64_t kend = min<int64_t>(kbeg + kchunk, nkt);
    const int64_t nsteps = (kend - kbeg + KB - 1) / KB;
    y += (int64_t)blockIdx.z * ysplit;
    constexpr int TS = Fmt<QT>::tile;
    Ranges rg;
    rg.q = make_rsrc(q + m0 * K, min<int64_t>(M - m0, BM) * K);
    rg.d = make_rsrc(DOTS ? (const void *)q : (const void *)(d + m0 * nkt),
                     DOTS ? 0 : min<int64_t>(M - m0, BM) * nkt * 2);
    if constexpr (FT >= 0) {
        // flat: the workgroup's 64 weight rows, each nkt / (block elements / 32) blocks
        const int64_t rb = (FT == TQ_Q4_K ? nkt / 8 : nkt) * Fmt<FT>::block;
        rg.w = make_rsrc(tiles + 32 * ct0 * rb, min<int64_t>(N - 32 * ct0, BN) * rb);
    } else {
        rg.w = make_rsrc(tiles + ct0 * nkt * TS, min<int64_t>(nct - ct0, BN / 32) * nkt * TS);
    }

    const Offs<QT, FT> o = make_offs<QT, FT>(nkt, K, tid);
    // the all-zero halves of the scale operands are never written again
    for (int i = tid; i < 2 * BM; i += WG_THREADS)
        L.da[i / BM][1][i % BM] = 0;
    for (int i = tid; i < 2 * BN; i += WG_THREADS)
        L.dw[i / BN][1][i % BN] = 0;

    // fp32 sums of this wave's 32 x 32 sub-block (Q4_1: the min term's
    // MFMAs accumulate into it too, which needs no final rescale)
    v16f acc = {};
    static_assert(QT != TQ_Q4_1 || weight_unscale<QT>() == 1.0f, "min term shares acc");

    // One k-block: the int8 MFMA (exact block dots) and, for y, the rank-1
    // fp16 MFMA giving sc[m][n] = da[m] * dw[n] (exact in fp32).  Its A
    // operand holds the step's KB activation scales of row m (k = 0..3) and
    // serves every k-block of the step; its B operand keeps only k-block kb's
    // weight scale (k = kb), so the k-sum is the one product.
    // Q8_0 operand through ds_read_b64_tr_b16: lane j of each 16-lane group
    // G gets halfword j % 4 of the 8-byte runs that lanes 4 i + j / 4 of the
    // group point at (i = 0..3).  Lane 4 i + a points at column pair c0 + i,
    // rows 4 s .. 4 s + 3 (s = 4 (G % 2) + a), so lane j holds column pairs
    // c0 .. c0 + 3 of row 16 (G % 2) + j = li: K 2 c0 .. 2 c0 + 7, in order;
    // c0 = 16 lk / 2 for the first read, 4 more for the second.
    const int trq = lane & 15, trg = (lane >> 4) & 1;
    const int tr_off = ((8 * lk + (trq >> 2)) * 32 + 4 * (4 * trg + (trq & 3))) * 2;
    auto mfmas = [&](int buf, int kb, const v4h &ua, uint64_t wv, v16i &dot, v16f &sc) {
        const v4i a = *(const v4i *)(L.A[buf] + (32 * wm + li) * LDS_ROW + 32 * kb + 16 * lk);
        v4i b;
        if constexpr (q8_tr<QT, FT>()) {
            typedef short v4s __attribute__((ext_vector_type(4)));
            const uint8_t *t = L.B[buf] + (wn * KB + kb) * 1024 + tr_off;
            const v4s r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4s *)(t));
            const v4s r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4s *)(t + 256));
            const v2i x0 = __builtin_bit_cast(v2i, r0), x1 = __builtin_bit_cast(v2i, r1);
            b = v4i{x0.x, x0.y, x1.x, x1.y};
        } else {
            b = *(const v4i *)(L.B[buf] + (32 * wn + li) * LDS_ROW + 32 * kb + 16 * lk);
        }
        const v16i z = {};
        dot = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, z, 0, 0, 0);
        if constexpr (!DOTS) {
            const v4h ub = __builtin_bit_cast(v4h, wv & (uint64_t(0xFFFF) << (16 * kb)));
            const v16f zf = {};
            sc = __builtin_amdgcn_mfma_f32_32x32x8f16(ua, ub, zf, 0, 0, 0);
        }
    };
    // Output layout of both MFMAs: lane holds column li, rows
    // 8*(r/4) + 4*lk + (r%4).
    auto epilogue = [&](int64_t kt, const v16i &dot, const v16f &sc) {
        if constexpr (DOTS) {
            const int64_t n = 32 * (ct0 + wn) + li;
            if (kt >= kbeg && kt < kend && n < N) {
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int64_t m = m0 + 32 * wm + 8 * (r >> 2) + 4 * lk + (r & 3);
                    if (m < M)
                        isum[(m * N + n) * nkt + kt] = (QT == TQ_Q4_0) ? (dot[r] >> 4) : dot[r];
                }
            }
        } else {
#pragma unroll
            for (int r = 0; r < 16; r++)
                acc[r] = fmaf((float)dot[r], sc[r], acc[r]);
        }
    };
    // Per step a wave takes its group's k-blocks, each MFMA pair followed
    // by its vector epilogue; the other waves of the SIMD (4 per SIMD) fill
    // the MFMA latency.  (Keeping two blocks' results live, to hide it within
    // the wave, does not fit the 128 registers a wave has at 4 per SIMD.)
    auto compute = [&](int buf, int64_t step, auto group0) {
        // this group's k-blocks J0 .. J1 - 1 of the step
        constexpr int J0 = decltype(group0)::value ? 0 : kb_group0<QT, DOTS>();
        constexpr int J1 = decltype(group0)::value ? kb_group0<QT, DOTS>() : KB;
        if constexpr (J1 == J0)
            return;
        const v4h ua = __builtin_bit_cast(v4h, L.da[buf][lk][32 * wm + li]);
        const uint64_t wv = L.dw[buf][lk][32 * wn + li];
#pragma unroll
        for (int j = J0; j < J1; j++) {
            v16i dot;
            v16f sc;
            mfmas(buf, j, ua, wv, dot, sc);
            epilogue(step * KB + j, dot, sc);
        }
        if constexpr (!DOTS) {
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (QT == TQ_Q4_1) {
                // min term of the group's k-blocks, two per fp32 MFMA: lane
                // (li, lk) holds k = lk, i.e. block J0 + 2j + lk, with A = da
                // * asum of activation row li (exact in fp32) and B = the
                // min of weight row li
                const int ra = 32 * wm + li;
                const uint64_t dav = L.da[buf][0][ra];
                const uint64_t mwv = L.mw[buf][32 * wn + li];
                static_assert((J1 - J0) % 2 == 0, "min term: pairs of k-blocks");
#pragma unroll
                for (int j = 0; j < (J1 - J0) / 2; j++) {
                    const int kb = J0 + 2 * j + lk;
                    const float a = f16_bits_to_f32((uint16_t)(dav >> (16 * kb))) *
                                    L.asum[buf][ra][kb];
                    const float b = f16_bits_to_f32((uint16_t)(mwv >> (16 * kb)));
                    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
                }
            }
        }
    };

    // Two register stages: step s+1's data is in flight while step s+2 is
    // issued.  Only wave group 0 stages; the groups run the same loop with the
    // same barriers, each as one basic block (two steps, no exit in between),
    // so the compiler tracks the two stages without conservative waits.  An
    // odd step count gets one trailing step whose k-blocks all lie past K: its
    // scales are zero, so it adds exactly 0, and its loads (like every
    // prefetch past the end) are range-checked by the buffer descriptors.
    const int64_t nsteps2 = (nsteps + 1) & ~int64_t(1);
    auto run = [&](auto stage) {
        constexpr bool ST = decltype(stage)::value;
        StageRegs<QT, FT> r0, r1;
        if constexpr (ST) {
            load_step<QT, DOTS, FT>(r0, rg, o, (int)kend, (int)kbeg);
            load_step<QT, DOTS, FT>(r1, rg, o, (int)kend, (int)kbeg + KB);
            store_step<QT, DOTS, FT>(r0, L, 0, lut, tid, o);
        }
        __syncthreads();
        for (int64_t step = 0; step < nsteps2; step += 2) {
            // even step: buffer 0 is computed, r1 holds step+1, r0 is free
            if constexpr (ST)
                load_step<QT, DOTS, FT>(r0, rg, o, (int)kend, (int)(kbeg + (step + 2) * KB));
            compute(0, kbeg / KB + step, stage);
            if constexpr (ST)
                store_step<QT, DOTS, FT>(r1, L, 1, lut, tid, o);
            __syncthreads();
            // odd step: buffer 1 is computed, r0 holds step+2, r1 is free
            if constexpr (ST)
                load_step<QT, DOTS, FT>(r1, rg, o, (int)kend, (int)(kbeg + (step + 3) * KB));
            compute(1, kbeg / KB + step + 1, stage);
            if constexpr (ST)
                store_step<QT, DOTS, FT>(r0, L, 0, lut, tid, o);
            __syncthreads();
        }
    };
    if (grp == 0)
        run(std::true_type{});
    else
        run(std::false_type{});
    if constexpr (DOTS)
        return;
    float v[16];
#pragma unroll
    for (int r = 0; r < 16; r++)
        v[r] = acc[r] * weight_unscale<QT>();
    if constexpr (KSW > 1) {
        // the groups' partial sums meet in LDS (the A buffers, done with)
        static_assert(KSW == 2 && 16 * THREADS * 4 <= (int)sizeof(L.A), "reduction space");
        float *red = (float *)L.A[0];
        if (grp == 1) {
#pragma unroll
            for (int r = 0; r < 16; r++)
                red[r * THREADS + (tid - THREADS)] = v[r];
        }
        __syncthreads();
        if (grp == 1)
            return;
#pragma unroll
        for (int r = 0; r < 16; r++)
            v[r] += red[r * THREADS + tid];
    }
    const int64_t n = 32 * (ct0 + wn) + li;
    if (n < N) {
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const int64_t m = m0 + 32 * wm + 8 * (r >> 2) + 4 * lk + (r & 3);
            if (m < M)
                y[m * ldy + n] = v[r];
        }
    }
}

// S > 1: the K dimension split into S ranges of kchunk k-tiles (a multiple
// of KB), range z written as partial plane z of y (ysplit elements apart,
// row stride ldy); S = 1: the whole of K into y.
template <int QT, int FT>
hipError_t launch_t(const void *w, int64_t K, int64_t N, const int8_t *q, const uint16_t *d,
                    int64_t M, const Lut &lut, float *y, int64_t ldy, int32_t *isum,
                    hipStream_t s, int S = 1, int64_t kchunk = 0, int64_t ysplit = 0)
{
    const int64_t nkt = K / 32;
    const int64_t nct = (N + 31) / 32;
    if (S <= 1)
        kchunk = nkt;
    // x = weight blocks, y = activation blocks, z = k-ranges.  The dispatcher
    // deals consecutive workgroup ids round-robin to the 8 XCDs, so when the
    // x extent is a multiple of 8 all activation blocks of one weight block
    // run on one XCD and each weight tile is fetched into a single L2.
    if (!grid_fits((nct + BN / 32 - 1) / (BN / 32), WG_THREADS) ||
        !grid_fits((M + BM - 1) / BM, 1) || S < 1 || S > 64)
        return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)((nct + BN / 32 - 1) / (BN / 32)), (unsigned)((M + BM - 1) / BM),
              (unsigned)S);
    if (isum)
        k_qgemm<QT, true, FT><<<grid, WG_THREADS, 0, s>>>((const uint8_t *)w, nkt, N, q, d, M, K,
                                                       lut, y, ldy, isum, kchunk, ysplit);
    else
        k_qgemm<QT, false, FT><<<grid, WG_THREADS, 0, s>>>((const uint8_t *)w, nkt, N, q, d, M, K,
                                                        lut, y, ldy, isum, kchunk, ysplit);
    return hipGetLastError();
}

// y[m * ldy + n] = sum over z < S of part[z * M * N + m * N + n], added in
// the order z = 0, 1, ..., so the result does not depend on scheduling.
// A thread takes 4 consecutive outputs of a row (N % 4 == 0: 16-byte plane
// loads; ldy % 4 == 0 and y 16-byte aligned too: 16-byte stores).
template <bool VEC>
__global__ void k_sum_planes(const float *__restrict__ part, int64_t M, int64_t N, int S,
                             float *__restrict__ y, int64_t ldy, bool vec_store)
{
    const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    const int64_t plane = M * N;
    if (i >= plane)
        return;
    if constexpr (VEC) {
        float4 v = *(const float4 *)(part + i);
        for (int z = 1; z < S; z++) {
            const float4 w = *(const float4 *)(part + (int64_t)z * plane + i);
            v.x += w.x, v.y += w.y, v.z += w.z, v.w += w.w;
        }
        const int64_t m = i / N, n = i - m * N;
        float *o = y + m * ldy + n;
        if (vec_store) {
            *(float4 *)o = v;
        } else {
            o[0] = v.x, o[1] = v.y, o[2] = v.z, o[3] = v.w;
        }
    } else {
        for (int e = 0; e < 4 && i + e < plane; e++) {
            float v = part[i + e];
            for (int z = 1; z < S; z++)
                v += part[(int64_t)z * plane + i + e];
            const int64_t m = (i + e) / N, n = (i + e) - m * N;
            y[m * ldy + n] = v;
        }
    }
}

}  // namespace

hipError_t launch_qgemm(int type, const void *tiles, int64_t K, int64_t N, const int8_t *q,
                        const uint16_t *d, int64_t M, const Lut &lut, float *y, int64_t ldy,
                        int32_t *isum, hipStream_t s)
{
    switch (type) {
    case TQ_Q4_0: return launch_t<TQ_Q4_0, -1>(tiles, K, N, q, d, M, lut, y, ldy, isum, s);
    case TQ_Q8_0: return launch_t<TQ_Q8_0, -1>(tiles, K, N, q, d, M, lut, y, ldy, isum, s);
    case TQ_IQ4_NL: return launch_t<TQ_IQ4_NL, -1>(tiles, K, N, q, d, M, lut, y, ldy, isum, s);
    case TQ_MXFP4: return launch_t<TQ_MXFP4, -1>(tiles, K, N, q, d, M, lut, y, ldy, isum, s);
    case TQ_Q4_1: return launch_t<TQ_Q4_1, -1>(tiles, K, N, q, d, M, lut, y, ldy, isum, s);
    }
    return hipErrorInvalidValue;
}

// The K split of the GEMM for small output grids: S partial planes of M x N
// fp32 in `part`, then their sum into y.
hipError_t launch_qgemm_split(int type, const void *tiles, int64_t K, int64_t N, const int8_t *q,
                              const uint16_t *d, int64_t M, const Lut &lut, float *y, int64_t ldy,
                              int S, float *part, hipStream_t s)
{
    const int64_t nkt = K / 32;
    int64_t kchunk = (nkt + S - 1) / S;
    kchunk = (kchunk + KB - 1) / KB * KB;
    const int64_t plane = M * N;
    hipError_t e;
    switch (type) {
    case TQ_Q4_0: e = launch_t<TQ_Q4_0, -1>(tiles, K, N, q, d, M, lut, part, N, nullptr, s, S, kchunk, plane); break;
    case TQ_Q8_0: e = launch_t<TQ_Q8_0, -1>(tiles, K, N, q, d, M, lut, part, N, nullptr, s, S, kchunk, plane); break;
    case TQ_IQ4_NL: e = launch_t<TQ_IQ4_NL, -1>(tiles, K, N, q, d, M, lut, part, N, nullptr, s, S, kchunk, plane); break;
    case TQ_MXFP4: e = launch_t<TQ_MXFP4, -1>(tiles, K, N, q, d, M, lut, part, N, nullptr, s, S, kchunk, plane); break;
    case TQ_Q4_1: e = launch_t<TQ_Q4_1, -1>(tiles, K, N, q, d, M, lut, part, N, nullptr, s, S, kchunk, plane); break;
    default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess)
        return e;
    return launch_sum_planes(part, M, N, S, y, ldy, s);
}

hipError_t launch_sum_planes(const float *part, int64_t M, int64_t N, int S, float *y,
                             int64_t ldy, hipStream_t s)
{
    const int64_t plane = M * N;
    const int64_t blocks = (plane / 4 + 256) / 256;
    if (!grid_fits(blocks, 256))
        return hipErrorInvalidConfiguration;
    if (N % 4 == 0) {
        const bool vs = ldy % 4 == 0 && ((uintptr_t)y & 15) == 0;
        k_sum_planes<true><<<(unsigned)blocks, 256, 0, s>>>(part, M, N, S, y, ldy, vs);
    } else {
        k_sum_planes<false><<<(unsigned)blocks, 256, 0, s>>>(part, M, N, S, y, ldy, false);
    }
    return hipGetLastError();
}

hipError_t launch_qgemm_flat(int type, const void *flat, int64_t K, int64_t N, const int8_t *q,
                             const uint16_t *d, int64_t M, const Lut &lut, float *y,
                             int64_t ldy, int32_t *isum, hipStream_t s)
{
    switch (type) {
    case TQ_Q4_0: return launch_t<TQ_Q4_0, TQ_Q4_0>(flat, K, N, q, d, M, lut, y, ldy, isum, s);
    case TQ_Q8_0: return launch_t<TQ_Q8_0, TQ_Q8_0>(flat, K, N, q, d, M, lut, y, ldy, isum, s);
    case TQ_IQ4_NL:
        return launch_t<TQ_IQ4_NL, TQ_IQ4_NL>(flat, K, N, q, d, M, lut, y, ldy, isum, s);
    case TQ_MXFP4: return launch_t<TQ_MXFP4, TQ_MXFP4>(flat, K, N, q, d, M, lut, y, ldy, isum, s);
    case TQ_Q4_1: return launch_t<TQ_Q4_1, TQ_Q4_1>(flat, K, N, q, d, M, lut, y, ldy, isum, s);
    case TQ_Q4_K: return launch_t<TQ_Q4_1, TQ_Q4_K>(flat, K, N, q, d, M, lut, y, ldy, isum, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace tq
