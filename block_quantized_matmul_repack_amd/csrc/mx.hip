// MXFP4 tiles x MXFP8 activations on gfx950's block-scaled matrix cores.
//
// The page's MXFP4 tiles ("MXFP4": 32 x 32 E2M1 codes nibble-paired as in
// Q4_0, one E8M0 scale byte per row) already hold what the OCP Microscaling
// formats define: elements sharing a power-of-two scale per 32 along K.
// v_mfma_scale_f32_32x32x64_f8f6f4 takes such operands directly -- FP8 E4M3
// codes on one side, FP4 E2M1 codes on the other, one E8M0 byte per row and
// 32-element block on each -- and applies both scales inside the matrix
// core, so the product needs no per-block vector rescale at all.  The
// activations are quantized to MXFP8 for it (k_quantize_mx).
//
// Operand layouts (gfx950, one 32 x 32 output per wave and 64 K):
//   A (fp8, 32 bytes per lane): lane (row i = l % 32, h = l / 32) holds
//     K 16h .. 16h + 15 of the step's first 32-block, then the same 16
//     positions of the second; its scale byte is row i's for block h.
//   B (fp4, 16 bytes per lane): lane (row j, h) holds all 32 K of block h
//     of row j, low nibble first -- exactly row j's 16 bytes (column pairs
//     0..15) of an MXFP4 tile, which ds_read_b64_tr_b8 gathers from a raw
//     tile copy in LDS in two reads of 8 column pairs.
//   Output: lane (j, h) holds column j, rows 8 (r / 4) + 4 h + (r % 4).
//
// The page's conversion of the E8M0 byte ("MXFP4", Dequantization: the FP16
// power of two with exponent bits clamp(e - 112, 0, 30)) is kept exactly:
// e >= 142 acts as 142 (2^15); e <= 112 means scale 0, which an E8M0 byte
// cannot express, so those rows' codes are staged as zeros.  Blocks past K
// are staged as zeros too.  (Zeroing is done on the way into LDS, never on
// an MFMA's source registers: a scaled MFMA keeps reading its B operand
// late into its execution, and a vector write to those registers right
// after the issue changes its last result rows.)
#include <type_traits>

#include "tq_internal.h"

namespace tq {
namespace {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// MXFP8 activation quantization (OCP Microscaling v1.0 conversion).  Per 32
// elements: e = biased exponent of amax minus 8 (the largest E4M3 exponent),
// at least 0, i.e. X = 2^(floor(log2 amax) - 8); P = E4M3 nearest to x / X,
// ties to even, saturating at 448; the code's sign bit is x's.  One block per
// quad of lanes, 8 consecutive elements per lane.
// ---------------------------------------------------------------------------
constexpr int QTHREADS = 256;
constexpr int QBPW = QTHREADS / 4;

// E4M3 code of a finite v >= 0 (< 512 here): below 2^-6 the subnormal step
// 2^-9 (v * 512 is exact, rint rounds to even); above, the fp32 mantissa
// rounded to 3 bits, nearest-even, with the carry running into the exponent
// (rebias 127 -> 7).  Codes past 0x7E (448) saturate.
__device__ __forceinline__ uint32_t e4m3_code(float v)
{
    uint32_t c;
    if (v < 0.015625f) {
        c = (uint32_t)__builtin_rintf(v * 512.0f);
    } else {
        const uint32_t b = __float_as_uint(v);
        c = ((b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20) - (120u << 3);
    }
    return c < 0x7Eu ? c : 0x7Eu;
}

template <int DT>
__global__ __launch_bounds__(QTHREADS) void k_quantize_mx(const void *__restrict__ x, int64_t M,
                                                          int64_t nb, int64_t ldx,
                                                          uint8_t *__restrict__ q,
                                                          uint8_t *__restrict__ e)
{
    const int64_t blk = (int64_t)blockIdx.x * QBPW + (threadIdx.x >> 2);
    const int c = threadIdx.x & 3;
    if (blk >= M * nb)
        return;                      // uniform across the quad of a block
    const int64_t m = blk / nb, kt = blk - m * nb;
    float v[8];
    load_x8<DT>(v, x, m * ldx + kt * 32 + 8 * c);
    float amax = fabsf(v[0]);
#pragma unroll
    for (int i = 1; i < 8; i++)
        amax = fmaxf(amax, fabsf(v[i]));
    amax = quad_max(amax);
    const int eb = max((int)(__float_as_uint(amax) >> 23) - 8, 0);
    const float inv = __uint_as_float((uint32_t)(254 - eb) << 23);   // 1 / X, exact
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const uint32_t code = e4m3_code(fabsf(v[i]) * inv) | ((__float_as_uint(v[i]) >> 24) & 0x80u);
        w[i >> 2] |= code << (8 * (i & 3));
    }
    *(u32x2u *)(q + m * nb * 32 + kt * 32 + 8 * c) = u32x2u{w[0], w[1]};
    if (c == 0)
        e[m * nb + kt] = (uint8_t)eb;
}

// ---------------------------------------------------------------------------
// Block-scaled GEMM.  A workgroup of 8 waves owns BM x BN = 64 x 128
// outputs (64 activation rows, four 32-row weight stripes: the 8-bit
// activations are the larger operand, so a workgroup spans more weights
// than activations), in two groups of 4 that own the same outputs and split
// each stage's MFMA steps (two waves per SIMD, so one wave's waits for
// loads and LDS overlap the other's work; at the end group 1 hands its sums
// to group 0 through LDS): wave (g, w) takes activation rows 32 (w % 2) ..
// + 31 against stripes 2 (w / 2) and 2 (w / 2) + 1 (two accumulators).  A
// stage covers SKT = 8 k-tiles (256 K, four MFMA steps of 64), staged by all
// 512 threads: the activation rows (256 bytes each, padded to 272 so that
// b128 reads of 16 consecutive rows hit 16 different bank groups), their
// E8M0 bytes, the 32 tiles' quant bytes as stored and their row scales
// converted once.  (Stages of 512 K measured the same.)
//
// Scales sit in LDS as SKT / 4 dwords per row, k-tile 2s + h in byte s % 4
// of dword h + 2 (s / 4): a lane of half h reads its dwords once per stage
// and the MFMA's byte select (a constant) picks the step's scale.  The page's E8M0
// conversion is applied when staging: min(e, 142), with the codes of rows
// whose e <= 112 (and of tiles past K) staged as zeros.  Which rows to zero
// comes from one wave ballot: the lane that loads row r's scale byte of a
// tile votes for it, and the lanes holding that tile's quant chunks read
// their 16 rows' votes; when every row is kept (the common case) the whole
// wave skips the masking.
//
// LDS is double-buffered and the global loads run two stages ahead in
// registers, one barrier per stage.  The buffer descriptors advance by one
// stage each time (scalar work), so per-thread load offsets never change.
// The stage loop advances two stages per iteration as one basic block, so
// the compiler keeps exact wait counts for the loads; an odd stage count is
// padded with a stage whose k-tiles all lie past K (zeroed, it adds exactly
// 0; its loads are range-checked or land in zeroed rows).
// ---------------------------------------------------------------------------
#ifndef TQ_MX_SKT
#define TQ_MX_SKT 8
#endif
constexpr int BM = 64, BN = 128, SKT = TQ_MX_SKT;
constexpr int KSW = 2;                  // wave groups splitting a stage's steps
constexpr int THREADS = 256 * KSW;
constexpr int SPG = SKT / 2 / KSW;      // MFMA steps (64 K) per group and stage
constexpr int A_ROW = 32 * SKT + 16;
constexpr int TB = 544;                 // MXFP4 tile bytes: 512 quant + 32 E8M0
constexpr int NSTR = BN / 32;           // weight stripes per workgroup
constexpr int NT = NSTR * SKT;          // tiles per stage
constexpr int NA = BM * SKT * 2 / THREADS;     // 16-byte activation chunks per thread
constexpr int NS = BM * SKT / THREADS;         // activation scale bytes per thread
constexpr int NB = NT * 32 / THREADS;          // 16-byte tile chunks per thread
static_assert(NA * THREADS == BM * SKT * 2 && NS * THREADS == BM * SKT &&
              NB * THREADS == NT * 32 && SPG * KSW * 2 == SKT && SKT % 8 == 0, "stage split");
constexpr int SDW = SKT / 4;            // scale dwords per row
constexpr int CPR = 2 * SKT;            // 16-byte chunks per staged activation row

struct LdsMx {
    uint8_t A[2][BM * A_ROW];
    uint8_t B[2][NT * 512];             // tile (stripe c, k-tile j) at (c * SKT + j) * 512
    uint32_t sa[2][BM][SDW];            // activation row: k-tile 2s + h in byte s % 4 of
                                        // dword h + 2 (s / 4)
    uint32_t sb[2][BN][SDW];            // weight row, converted, same arrangement
};

// f(integral_constant<int, I>) for I = I0 .. N - 1: a loop whose index is a
// constant expression (the MFMA's scale byte selects must be constants).
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (I < N) {
        f(std::integral_constant<int, I>());
        static_for<I + 1, N>(f);
    }
}

// Byte of k-tile j in a row's scale dwords.
__device__ __forceinline__ int scale_byte(int j)
{
    const int s = j >> 1;
    return 4 * ((j & 1) + 2 * (s >> 2)) + (s & 3);
}

struct RangesMx {
    __amdgpu_buffer_rsrc_t q, e, w;
};

struct StageMx {
    v4i a[NA];
    v4i b[NB];
    uint32_t sa[NS];
    uint32_t sb[NB];
};

// Per-thread load offsets, relative to the stage's descriptors (thread tid
// of 512):
//   activation chunk ch = tid + 512 i (i < NA): row ch / CPR, 16 bytes at
//     16 (ch % CPR);
//   activation scale byte g = tid + 512 i (i < NS) of the stage's 64 x SKT:
//     row g / SKT, k-tile g % SKT (byte loads, each range-checked on its
//     own; consecutive lanes read one row's bytes, so a wave's load touches
//     a few cache lines, not 64);
//   tile chunk ch = tid + 512 i (i < NB): tile t = ch / 32 (stripe t / SKT,
//     k-tile t % SKT), 16 quant bytes at 16 (ch % 32) -- column pair (ch % 32)
//     / 2, rows 16 (ch % 2) .. + 15 -- and that tile's scale of row ch % 32
//     (so the 32 lanes of a tile hold all its row scales).
struct OffsMx {
    int a[NA], sa[NS], b[NB], sb[NB];
};

__device__ __forceinline__ OffsMx make_offs_mx(int tid, int K, int nkt)
{
    OffsMx o;
#pragma unroll
    for (int i = 0; i < NA; i++) {
        const int ch = tid + THREADS * i;
        o.a[i] = (ch / CPR) * K + 16 * (ch % CPR);
    }
#pragma unroll
    for (int i = 0; i < NS; i++) {
        const int g = tid + THREADS * i;
        o.sa[i] = (g / SKT) * nkt + g % SKT;
    }
#pragma unroll
    for (int i = 0; i < NB; i++) {
        const int ch = tid + THREADS * i;
        const int t = ch >> 5;
        const int tile = ((t / SKT) * nkt + t % SKT) * TB;
        o.b[i] = tile + 16 * (ch & 31);
        o.sb[i] = tile + 512 + (ch & 31);
    }
    return o;
}

// The descriptors of the stage at k-tile kt0: bases advanced, sizes shrunk
// by the same amount (a past-the-end size is clamped to 0: every load of the
// stage then returns 0), so each check is the original one.
__device__ __forceinline__ RangesMx stage_ranges(const uint8_t *q, const uint8_t *e,
                                                 const uint8_t *w, int64_t qb, int64_t eb,
                                                 int64_t wb, int64_t kt0)
{
    RangesMx r;
    r.q = make_rsrc(q + kt0 * 32, qb - kt0 * 32);
    r.e = make_rsrc(e + kt0, eb - kt0);
    r.w = make_rsrc(w + kt0 * TB, wb - kt0 * TB);
    return r;
}

__device__ __forceinline__ void load_stage(StageMx &s, const RangesMx &rg, const OffsMx &o)
{
#pragma unroll
    for (int i = 0; i < NA; i++)
        s.a[i] = __builtin_amdgcn_raw_buffer_load_b128(rg.q, o.a[i], 0, 0);
#pragma unroll
    for (int i = 0; i < NS; i++)
        s.sa[i] = __builtin_amdgcn_raw_buffer_load_b8(rg.e, o.sa[i], 0, 0);
#pragma unroll
    for (int i = 0; i < NB; i++) {
        s.b[i] = __builtin_amdgcn_raw_buffer_load_b128(rg.w, o.b[i], 0, BUF_NT);
        s.sb[i] = __builtin_amdgcn_raw_buffer_load_b8(rg.w, o.sb[i], 0, 0);
    }
}

// Four keep bits (bit i: byte i) as a byte mask: 0xFF in byte i where bit i
// is set (the product spreads bit i to bit 8i with no carries).
__device__ __forceinline__ uint32_t spread4(uint32_t n)
{
    return ((n * 0x00204081u) & 0x01010101u) * 0xFFu;
}

// kt0: the stage's first k-tile; tiles at kend and past are staged as zeros.
__device__ __forceinline__ void store_stage(const StageMx &s, LdsMx &L, int buf, int tid,
                                            int kt0, int kend)
{
#pragma unroll
    for (int i = 0; i < NA; i++) {
        const int ch = tid + THREADS * i;
        *(v4i *)(L.A[buf] + (ch / CPR) * A_ROW + 16 * (ch % CPR)) = s.a[i];
    }
    // byte stores: no arithmetic on the loaded values, which the compiler
    // could hoist above the stage's MFMAs (and with it a wait for the loads)
#pragma unroll
    for (int i = 0; i < NS; i++) {
        const int g = tid + THREADS * i;
        ((uint8_t *)L.sa[buf])[(g / SKT) * SKT + scale_byte(g % SKT)] = (uint8_t)s.sa[i];
    }
#pragma unroll
    for (int i = 0; i < NB; i++) {
        const int ch = tid + THREADS * i;
        const int t = ch >> 5, c = t / SKT, j = t % SKT;
        // codes of rows with e <= 112 (scale 0 on the page) and of tiles past
        // K are staged as zeros: this lane votes for row ch % 32 of its tile,
        // then takes the votes of its chunk's 16 rows
        v4i b = s.b[i];
        const uint32_t e = s.sb[i] & 0xFFu;
        const uint64_t keep = __builtin_amdgcn_ballot_w64(e > 112u && kt0 + j < kend);
        if (keep != ~uint64_t(0)) {
            const uint32_t k = (uint32_t)(keep >> (32 * ((tid >> 5) & 1) + 16 * (ch & 1)));
            b.x &= spread4(k & 0xFu);
            b.y &= spread4((k >> 4) & 0xFu);
            b.z &= spread4((k >> 8) & 0xFu);
            b.w &= spread4((k >> 12) & 0xFu);
        }
        *(v4i *)(L.B[buf] + t * 512 + 16 * (ch & 31)) = b;
        // the page's scale: 2^15 for e >= 142 (rows with e <= 112 are zero)
        ((uint8_t *)L.sb[buf])[(32 * c + (ch & 31)) * SKT + scale_byte(j)] = (uint8_t)min(e, 142u);
    }
}

__global__ __launch_bounds__(THREADS) void k_qgemm_mx(const uint8_t *__restrict__ tiles,
                                                      int64_t nkt, int64_t N,
                                                      const uint8_t *__restrict__ q,
                                                      const uint8_t *__restrict__ e, int64_t M,
                                                      int64_t K, float *__restrict__ y,
                                                      int64_t ldy, int64_t kchunk,
                                                      int64_t ysplit)
{
    __shared__ __attribute__((aligned(16))) LdsMx L;

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = (tid >> 6) & 3, grp = tid >> 8;
    const int wm = w & 1, wn = w >> 1;          // activation fragment, stripe pair
    const int li = lane & 31, lk = lane >> 5;
    const int64_t nct = (N + 31) / 32;
    const int64_t ct0 = (int64_t)blockIdx.x * NSTR;
    const int64_t m0 = (int64_t)blockIdx.y * BM;
    const int64_t rows = min<int64_t>(M - m0, BM);
    // k-range of this workgroup: k-tiles [kbeg, kend), the blockIdx.z-th of
    // the split (a multiple of SKT long), the whole of K without one; a
    // split writes its own partial plane of y, ysplit elements further per
    // range.  Tiles past kend are staged as zeros, so a range's last stage
    // adds nothing of the next range.
    const int64_t kbeg = (int64_t)blockIdx.z * kchunk;
    const int64_t kend = min<int64_t>(kbeg + kchunk, nkt);
    y += (int64_t)blockIdx.z * ysplit;

    const uint8_t *qw = q + m0 * K, *ew = e + m0 * nkt, *tw = tiles + ct0 * nkt * TB;
    const int64_t qb = rows * K, eb = rows * nkt;
    const int64_t wb = min<int64_t>(nct - ct0, NSTR) * nkt * TB;
    const OffsMx o = make_offs_mx(tid, (int)K, (int)nkt);

    // B operand: lane 2i + p of 16-lane group G points at column pair 8r + i,
    // rows 16 (G % 2) + 8p .. + 7 of tile (G / 2 = lk); the transposing read
    // hands lane l row l % 32's column pairs 8r .. 8r + 7
    const int G = lane >> 4, s16 = lane & 15;
    const int boff = (s16 >> 1) * 32 + 16 * (G & 1) + 8 * (s16 & 1);

    v16f acc[2] = {};
    // One stage, group GR's steps s = GR * SPG + i: the operand reads are
    // issued first, then the MFMAs.
    auto compute = [&](auto gr, int buf) {
        constexpr int GR = decltype(gr)::value;
        uint32_t sav[SDW / 2], sbv[2][SDW / 2];
#pragma unroll
        for (int d = 0; d < SDW / 2; d++) {
            sav[d] = L.sa[buf][32 * wm + li][lk + 2 * d];
            sbv[0][d] = L.sb[buf][64 * wn + li][lk + 2 * d];
            sbv[1][d] = L.sb[buf][64 * wn + 32 + li][lk + 2 * d];
        }
        v4i a[SPG][2];
        v2i b[SPG][2][2];
#pragma unroll
        for (int i = 0; i < SPG; i++) {
            constexpr int s0 = GR * SPG;
            const int s = s0 + i;
            const uint8_t *ar = L.A[buf] + (32 * wm + li) * A_ROW + 64 * s + 16 * lk;
            a[i][0] = *(const v4i *)ar;
            a[i][1] = *(const v4i *)(ar + 32);
#pragma unroll
            for (int c = 0; c < 2; c++) {
                const uint8_t *bt = L.B[buf] + ((2 * wn + c) * SKT + 2 * s + lk) * 512 + boff;
                b[i][c][0] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (__attribute__((address_space(3))) v2i *)(bt));
                b[i][c][1] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (__attribute__((address_space(3))) v2i *)(bt + 256));
            }
        }
        static_for<0, SPG>([&](auto ic) {
            constexpr int i = decltype(ic)::value, s = GR * SPG + i;
            const v8i av = {a[i][0].x, a[i][0].y, a[i][0].z, a[i][0].w,
                            a[i][1].x, a[i][1].y, a[i][1].z, a[i][1].w};
#pragma unroll
            for (int c = 0; c < 2; c++) {
                const v2i b0 = b[i][c][0], b1 = b[i][c][1];
                const v8i bv = {b0.x, b0.y, b1.x, b1.y, 0, 0, 0, 0};
                // byte select = step: the scale of k-tile 2s + lk
                acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    av, bv, acc[c], 0, 4, s & 3, (int)sav[s >> 2], s & 3, (int)sbv[c][s >> 2]);
            }
        });
    };

    const int nst = (int)((kend - kbeg + SKT - 1) / SKT);
    const int nst2 = (nst + 1) & ~1;
    // Each group runs its own copy of the stage loop (the same barriers).
    // Group 0 computes a stage and then stores the next one into LDS, group
    // 1 stores first and computes after, so that the two waves sharing a
    // SIMD are not both waiting for LDS operands or both staging at once.
    // Storing before computing is safe: the buffer written was last read in
    // the previous stage, which every wave finished before the barrier.  The
    // scheduling barriers keep each phase in place: hoisting a stage's LDS
    // stores above its MFMAs would wait for its loads a stage early.
    auto run = [&](auto gr) {
        constexpr int GR = decltype(gr)::value;
        StageMx r0, r1;
        load_stage(r0, stage_ranges(qw, ew, tw, qb, eb, wb, kbeg), o);
        load_stage(r1, stage_ranges(qw, ew, tw, qb, eb, wb, kbeg + SKT), o);
        store_stage(r0, L, 0, tid, (int)kbeg, (int)kend);
        __syncthreads();
        // compute buffer cb, store staged registers sr (stage kt0) into the other
        auto stage = [&](int cb, const StageMx &sr, int kt0) {
            if constexpr (GR == 0) {
                compute(gr, cb);
                __builtin_amdgcn_sched_barrier(0);
                store_stage(sr, L, cb ^ 1, tid, kt0, (int)kend);
            } else {
                store_stage(sr, L, cb ^ 1, tid, kt0, (int)kend);
                __builtin_amdgcn_sched_barrier(0);
                compute(gr, cb);
            }
        };
        for (int st = 0; st < nst2; st += 2) {
            // even stage: buffer 0 is computed, r1 holds stage st + 1, r0 is free
            load_stage(r0, stage_ranges(qw, ew, tw, qb, eb, wb, kbeg + (int64_t)(st + 2) * SKT), o);
            __builtin_amdgcn_sched_barrier(0);
            stage(0, r1, (int)kbeg + (st + 1) * SKT);
            __syncthreads();
            // odd stage: buffer 1 is computed, r0 holds stage st + 2, r1 is free
            load_stage(r1, stage_ranges(qw, ew, tw, qb, eb, wb, kbeg + (int64_t)(st + 3) * SKT), o);
            __builtin_amdgcn_sched_barrier(0);
            stage(1, r0, (int)kbeg + (st + 2) * SKT);
            __syncthreads();
        }
    };
    if (grp == 0)
        run(std::integral_constant<int, 0>());
    else
        run(std::integral_constant<int, 1>());

    // group 1's sums to group 0 (through the activation buffers, free now)
    float *red = (float *)L.A;
    static_assert(4 * 2 * 16 * 64 * sizeof(float) <= sizeof(L.A), "reduction fits");
    if (grp == 1) {
#pragma unroll
        for (int c = 0; c < 2; c++)
#pragma unroll
            for (int r = 0; r < 16; r++)
                red[((w * 2 + c) * 16 + r) * 64 + lane] = acc[c][r];
    }
    __syncthreads();
    if (grp == 1)
        return;
#pragma unroll
    for (int c = 0; c < 2; c++) {
        const int64_t n = 32 * (ct0 + 2 * wn + c) + li;
#pragma unroll
        for (int r = 0; r < 16; r++)
            acc[c][r] += red[((w * 2 + c) * 16 + r) * 64 + lane];
        if (n < N) {
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int64_t m = m0 + 32 * wm + 8 * (r >> 2) + 4 * lk + (r & 3);
                if (m < M)
                    y[m * ldy + n] = acc[c][r];
            }
        }
    }
}

}  // namespace

hipError_t launch_quantize_mx(int dtype, const void *x, int64_t M, int64_t K, int64_t ldx,
                              uint8_t *q, uint8_t *e, hipStream_t s)
{
    const int64_t nb = K / 32;
    if (!grid_fits((M * nb + QBPW - 1) / QBPW, QTHREADS))
        return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)((M * nb + QBPW - 1) / QBPW));
    switch (dtype) {
    case TQ_F32: k_quantize_mx<TQ_F32><<<grid, QTHREADS, 0, s>>>(x, M, nb, ldx, q, e); break;
    case TQ_BF16: k_quantize_mx<TQ_BF16><<<grid, QTHREADS, 0, s>>>(x, M, nb, ldx, q, e); break;
    case TQ_F16: k_quantize_mx<TQ_F16><<<grid, QTHREADS, 0, s>>>(x, M, nb, ldx, q, e); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_qgemm_mx(const void *tiles, int64_t K, int64_t N, const uint8_t *q,
                           const uint8_t *e, int64_t M, float *y, int64_t ldy, int S, float *part,
                           hipStream_t s)
{
    const int64_t nkt = K / 32, nct = (N + 31) / 32;
    if (!grid_fits((nct + NSTR - 1) / NSTR, THREADS) || !grid_fits((M + BM - 1) / BM, 1) ||
        S < 1 || S > 64)
        return hipErrorInvalidConfiguration;
    int64_t kchunk = nkt, ysplit = 0;
    float *out = y;
    int64_t ldo = ldy;
    if (S > 1) {
        kchunk = (nkt + S - 1) / S;
        kchunk = (kchunk + SKT - 1) / SKT * SKT;
        ysplit = M * N;
        out = part;
        ldo = N;
    }
    dim3 grid((unsigned)((nct + NSTR - 1) / NSTR), (unsigned)((M + BM - 1) / BM), (unsigned)S);
    k_qgemm_mx<<<grid, THREADS, 0, s>>>((const uint8_t *)tiles, nkt, N, q, e, M, K, out, ldo,
                                        kchunk, ysplit);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess || S <= 1)
        return err;
    return launch_sum_planes(part, M, N, S, y, ldy, s);
}

}  // namespace tq
