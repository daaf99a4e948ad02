// C ABI of the tiledq library: host-side validation, then one launch on the
// caller's stream.  Support is decided from static properties only (type,
// shape, pointer alignment), as the page "Hexagon backend developer details"
// asks of supports_op in "supports_op Independence from Buffer and Repack
// State"; launch geometry is computed here on the host ("Host-Side
// Precomputation via kernel_params").
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <mutex>

#include "tq_internal.h"

namespace {

// Scratch of tq_qgemv_noalloc: the K split's reduction slots live here
// instead of in a caller's workspace.  Every GPU the library runs on holds
// its own copy of the array until the process ends.  On the host the name
// `tq_scratch` is only a stand-in for the symbol: its device address comes
// from hipGetSymbolAddress, once per device, and only that address is
// passed to kernels.
__device__ __align__(256) uint64_t tq_scratch[TQ_NOALLOC_SCRATCH_BYTES / 8];

constexpr int MAX_DEVICES = 64;
std::once_flag scratch_once[MAX_DEVICES];
void *scratch_ptr[MAX_DEVICES];
hipError_t scratch_err[MAX_DEVICES];

__global__ void k_zero_u64(uint64_t *p, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

// The current device's scratch address, looked up (and the array cleared on
// `stream`, in stream order before any use) on the first call on that
// device; nullptr with `err` set if that failed.
void *device_scratch(hipStream_t stream, hipError_t &err)
{
    int dev = -1;
    err = hipGetDevice(&dev);
    if (err != hipSuccess)
        return nullptr;
    if (dev < 0 || dev >= MAX_DEVICES) {
        err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::call_once(scratch_once[dev], [&] {
        void *p = nullptr;
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(tq_scratch));
        if (e == hipSuccess) {
            // a fill kernel, not a memset: a first call made under stream
            // capture records it as an ordinary kernel node
            k_zero_u64<<<64, 256, 0, stream>>>((uint64_t *)p, TQ_NOALLOC_SCRATCH_BYTES / 8);
            e = hipGetLastError();
        }
        scratch_err[dev] = e;
        scratch_ptr[dev] = e == hipSuccess ? p : nullptr;
    });
    err = scratch_err[dev];
    return scratch_ptr[dev];
}

// Shape limits.  With them every grid stays below 2^31 work-items per
// dimension (a dispatch counts them in 32 bits): the decode and GEMM grids
// run 16 and 32 work-items per weight row (N <= 2^27), activation
// quantization 4 per 32-element block (M * K < 2^34).
constexpr int64_t MAX_K = int64_t(1) << 20;
constexpr int64_t MAX_N = int64_t(1) << 27;
constexpr int64_t MAX_M = int64_t(1) << 20;
constexpr int64_t MAX_PROD = int64_t(1) << 40;
constexpr int64_t MAX_MK = int64_t(1) << 34;

bool valid_type(int t)
{
    return t == TQ_Q4_0 || t == TQ_Q8_0 || t == TQ_IQ4_NL || t == TQ_MXFP4 || t == TQ_Q4_1 ||
           t == TQ_Q4_K;
}

// The tile kernels a type runs on: Q4_K tiles are Q4_1 tiles.
int kernel_type(int t) { return t == TQ_Q4_K ? TQ_Q4_1 : t; }

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool valid_kn(int64_t K, int64_t N)
{
    return K >= 32 && K <= MAX_K && K % 32 == 0 && N >= 0 && N <= MAX_N && K * N < MAX_PROD;
}

bool valid_mk(int64_t M, int64_t K) { return M >= 0 && M <= MAX_M && M * K < MAX_MK; }

// K, N valid for `type`: Q4_K also needs whole 256-element super-blocks.
bool valid_tkn(int type, int64_t K, int64_t N)
{
    return valid_kn(K, N) && (type != TQ_Q4_K || K % 256 == 0);
}

int launch_status(hipError_t e) { return e == hipSuccess ? TQ_OK : TQ_E_LAUNCH; }

// Twice the OCP Microscaling FP4 (E2M1) values of codes 0..15 ("MXFP4":
// the nibbles are E2M1 codes): 0, 0.5, 1, 1.5, 2, 3, 4, 6, then the same
// negated.  Doubled they are int8, and the kernels' int8 path stays exact.
constexpr int8_t MXFP4_TWICE_E2M1[16] = {0, 1, 2, 3, 4, 6, 8, 12,
                                         0, -1, -2, -3, -4, -6, -8, -12};

// The table a launch of `type` uses: the caller's for IQ4_NL, the fixed one
// for MXFP4, none for the others.
tq::Lut pack_lut(int type, const int8_t *lut)
{
    if (type == TQ_MXFP4)
        lut = MXFP4_TWICE_E2M1;
    else if (type != TQ_IQ4_NL)
        lut = nullptr;
    tq::Lut t{};
    if (lut)
        for (int i = 0; i < 16; i++)
            t.w[i / 4] |= (uint32_t)(uint8_t)lut[i] << (8 * (i % 4));
    return t;
}

// Alignment a flat block buffer of `type` needs: 2 bytes (fp16 scales), 4
// for the 17-byte MXFP4 and 20-byte Q4_1 blocks (read through aligned
// dwords), 16 for Q4_K's 144-byte super-blocks (read as 16-byte vectors).
uintptr_t flat_align(int type)
{
    return type == TQ_Q4_K ? 16 : ((type == TQ_MXFP4 || type == TQ_Q4_1) ? 4 : 2);
}

// `wa`: the alignment the weight buffer needs (16 for tiles).
int check_matmul(int type, const void *tiles, int64_t K, int64_t N, const int8_t *q,
                 const uint16_t *d, int64_t M, const int8_t *lut, const void *out, int64_t ldy,
                 bool need_d, uintptr_t wa = 16)
{
    if (!valid_type(type))
        return TQ_E_TYPE;
    if (!valid_tkn(type, K, N) || !valid_mk(M, K) || ldy < N)
        return TQ_E_SHAPE;
    if (M == 0 || N == 0)
        return TQ_OK;
    if (!tiles || !q || (need_d && !d) || !out || (type == TQ_IQ4_NL && !lut))
        return TQ_E_NULL;
    if (!aligned(tiles, wa) || !aligned(q, 16) || (need_d && !aligned(d, 2)) ||
        !aligned(out, 4))
        return TQ_E_ALIGN;
    return TQ_OK;
}

}  // namespace

extern "C" {

size_t tq_tile_bytes(int type)
{
    switch (type) {
    case TQ_Q4_0: return tq::Fmt<TQ_Q4_0>::tile;
    case TQ_Q8_0: return tq::Fmt<TQ_Q8_0>::tile;
    case TQ_IQ4_NL: return tq::Fmt<TQ_IQ4_NL>::tile;
    case TQ_MXFP4: return tq::Fmt<TQ_MXFP4>::tile;
    case TQ_Q4_1: return tq::Fmt<TQ_Q4_1>::tile;
    case TQ_Q4_K: return tq::Fmt<TQ_Q4_K>::tile;
    }
    return 0;
}

size_t tq_block_bytes(int type)
{
    switch (type) {
    case TQ_Q4_0: return tq::Fmt<TQ_Q4_0>::block;
    case TQ_Q8_0: return tq::Fmt<TQ_Q8_0>::block;
    case TQ_IQ4_NL: return tq::Fmt<TQ_IQ4_NL>::block;
    case TQ_MXFP4: return tq::Fmt<TQ_MXFP4>::block;
    case TQ_Q4_1: return tq::Fmt<TQ_Q4_1>::block;
    case TQ_Q4_K: return tq::Fmt<TQ_Q4_K>::block;
    }
    return 0;
}

size_t tq_tiled_bytes(int type, int64_t K, int64_t N)
{
    if (!valid_type(type) || !valid_tkn(type, K, N))
        return 0;
    return (size_t)(K / 32) * (size_t)((N + 31) / 32) * tq_tile_bytes(type);
}

size_t tq_flat_bytes(int type, int64_t K, int64_t N)
{
    if (!valid_type(type) || !valid_tkn(type, K, N))
        return 0;
    return (size_t)N * (size_t)(K / (type == TQ_Q4_K ? 256 : 32)) * tq_block_bytes(type);
}

int tq_supported(int type, int64_t K, int64_t N, int64_t M, int path)
{
    if (!valid_type(type) || !valid_tkn(type, K, N) || !valid_mk(M, K))
        return 0;
    if (path == TQ_PATH_GEMV || path == TQ_PATH_GEMV_FLAT)
        return M <= 8;
    if (path == TQ_PATH_GEMM_MX)
        return type == TQ_MXFP4;
    return path == TQ_PATH_GEMM || path == TQ_PATH_GEMM_FLAT;
}

const char *tq_status_string(int status)
{
    switch (status) {
    case TQ_OK: return "TQ_OK";
    case TQ_E_NULL: return "TQ_E_NULL: required pointer is NULL";
    case TQ_E_TYPE: return "TQ_E_TYPE: unknown type, dtype or path";
    case TQ_E_SHAPE: return "TQ_E_SHAPE: shape outside the supported domain";
    case TQ_E_ALIGN: return "TQ_E_ALIGN: pointer misaligned";
    case TQ_E_LAUNCH: return "TQ_E_LAUNCH: kernel launch failed";
    }
    return "unknown tq_status";
}

int tq_repack_tiles(int type, const void *flat, int64_t K, int64_t N, void *tiles,
                    hipStream_t stream)
{
    if (!valid_type(type))
        return TQ_E_TYPE;
    if (!valid_tkn(type, K, N))
        return TQ_E_SHAPE;
    if (N == 0)
        return TQ_OK;
    if (!flat || !tiles)
        return TQ_E_NULL;
    if (!aligned(flat, flat_align(type)) || !aligned(tiles, 16))
        return TQ_E_ALIGN;
    return launch_status(tq::launch_repack(type, flat, K, N, tiles, stream));
}

int tq_quantize_act(int dtype, const void *x, int64_t M, int64_t K, int64_t ldx, int8_t *q,
                    uint16_t *d, hipStream_t stream)
{
    if (dtype != TQ_F32 && dtype != TQ_BF16 && dtype != TQ_F16)
        return TQ_E_TYPE;
    if (K < 32 || K > MAX_K || K % 32 != 0 || !valid_mk(M, K) || ldx < K ||
        M * ldx >= MAX_PROD)
        return TQ_E_SHAPE;
    if (M == 0)
        return TQ_OK;
    if (!x || !q || !d)
        return TQ_E_NULL;
    if (!aligned(x, dtype == TQ_F32 ? 4 : 2) || !aligned(q, 4) || !aligned(d, 2))
        return TQ_E_ALIGN;
    return launch_status(tq::launch_quantize(dtype, x, M, K, ldx, q, d, stream));
}

size_t tq_qgemv_workspace_bytes(int type, int64_t K, int64_t N, int64_t M)
{
    if (!valid_type(type) || !valid_tkn(type, K, N) || N == 0 || M < 1 || M > 8)
        return 0;
    return tq::gemv_workspace_bytes(K, N, M);
}

int tq_qgemv(int type, const void *tiles, int64_t K, int64_t N, const int8_t *q,
             const uint16_t *d, int64_t M, const int8_t *lut, float *y, int64_t ldy,
             void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (valid_type(type) && M > 8)
        return TQ_E_SHAPE;
    int st = check_matmul(type, tiles, K, N, q, d, M, lut, y, ldy, true);
    if (st != TQ_OK || M == 0 || N == 0)
        return st;
    if (workspace && !aligned(workspace, 256))
        return TQ_E_ALIGN;
    const tq::Act act{q, d, nullptr, -1, 0};
    return launch_status(tq::launch_qgemv(kernel_type(type), tiles, K, N, act, M, pack_lut(type, lut), y, ldy,
                                          nullptr, workspace, workspace_bytes, stream));
}

int tq_qgemv_noalloc(int type, const void *tiles, int64_t K, int64_t N, const int8_t *q,
                     const uint16_t *d, int64_t M, const int8_t *lut, float *y, int64_t ldy,
                     hipStream_t stream)
{
    if (valid_type(type) && M > 8)
        return TQ_E_SHAPE;
    int st = check_matmul(type, tiles, K, N, q, d, M, lut, y, ldy, true);
    if (st != TQ_OK || M == 0 || N == 0)
        return st;
    const size_t need = tq::gemv_workspace_bytes(K, N, M);
    if (need > TQ_NOALLOC_SCRATCH_BYTES)
        return TQ_E_SHAPE;
    void *ws = nullptr;
    if (need > 0) {
        hipError_t e;
        ws = device_scratch(stream, e);
        if (!ws)
            return TQ_E_LAUNCH;
    }
    const tq::Act act{q, d, nullptr, -1, 0};
    return launch_status(tq::launch_qgemv(kernel_type(type), tiles, K, N, act, M,
                                          pack_lut(type, lut), y, ldy, nullptr, ws, need,
                                          stream));
}

int tq_qgemv_x(int type, const void *tiles, int64_t K, int64_t N, int dtype, const void *x,
               int64_t ldx, int64_t M, const int8_t *lut, float *y, int64_t ldy,
               void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (dtype != TQ_F32 && dtype != TQ_BF16 && dtype != TQ_F16)
        return TQ_E_TYPE;
    if (valid_type(type) && M > 8)
        return TQ_E_SHAPE;
    if (ldx < K || M * ldx >= MAX_PROD)
        return TQ_E_SHAPE;
    // x stands in for q in the common checks; its own alignment is checked below
    int st = check_matmul(type, tiles, K, N, (const int8_t *)tiles, nullptr, M, lut, y, ldy,
                          false);
    if (st != TQ_OK || M == 0 || N == 0)
        return st;
    if (!x)
        return TQ_E_NULL;
    if (!aligned(x, dtype == TQ_F32 ? 4 : 2) || (workspace && !aligned(workspace, 256)))
        return TQ_E_ALIGN;
    const tq::Act act{nullptr, nullptr, x, dtype, ldx};
    return launch_status(tq::launch_qgemv(kernel_type(type), tiles, K, N, act, M, pack_lut(type, lut), y, ldy,
                                          nullptr, workspace, workspace_bytes, stream));
}

int tq_qgemm(int type, const void *tiles, int64_t K, int64_t N, const int8_t *q,
             const uint16_t *d, int64_t M, const int8_t *lut, float *y, int64_t ldy,
             hipStream_t stream)
{
    int st = check_matmul(type, tiles, K, N, q, d, M, lut, y, ldy, true);
    if (st != TQ_OK || M == 0 || N == 0)
        return st;
    return launch_status(
        tq::launch_qgemm(kernel_type(type), tiles, K, N, q, d, M, pack_lut(type, lut), y, ldy, nullptr, stream));
}

}  // extern "C"

namespace {

// The cost model behind tq_matmul_path, fitted to times measured on MI355X
// (K = 1024 .. 8192, N = 1024 .. 14336, M = 9 .. 256, every tile type):
//   - a decode pass (one qgemv launch of up to 8 rows) takes pass_a + tile
//     bytes / pass_bw;
//   - a GEMM launch takes GEMM_A + steps x step_us x (1 + GEMM_LOAD x
//     w / 256) per round of up to 256 workgroups (128 x 64 outputs each, one
//     per compute unit), with steps = the launch's k-range / 128 and w the
//     workgroups of a round: a step costs more when every compute unit is
//     busy;
//   - a K split into S ranges adds the sum of the S partial planes, SUM_A +
//     SUM_US_PER_MB x their MB.
struct TypeCost {
    double pass_a, pass_bw, step_us;  // us, bytes per us, us per step of 128 k
};
TypeCost type_cost(int type)
{
    switch (type) {
    case TQ_Q4_0: return {4.9, 6.0e6, 0.644};
    case TQ_Q8_0: return {4.5, 6.1e6, 0.624};
    case TQ_IQ4_NL: return {4.8, 4.3e6, 0.725};
    case TQ_MXFP4: return {4.8, 3.7e6, 0.716};
    default: return {4.7, 5.9e6, 0.89};                  // Q4_1, Q4_K
    }
}
constexpr double GEMM_A = 4.6, GEMM_LOAD = 0.27, SUM_A = 2.2, SUM_US_PER_MB = 0.6;

int64_t gemm_blocks(int64_t N, int64_t M) { return ((N + 63) / 64) * ((M + 127) / 128); }

// Estimated time of the GEMM with its K split into S ranges (S = 1: none).
double gemm_cost_us(int type, int64_t K, int64_t N, int64_t M, int S)
{
    const TypeCost c = type_cost(type);
    const int64_t wgs = gemm_blocks(N, M) * S;
    const int64_t rounds = (wgs + 255) / 256;
    const double per_round = (double)std::min<int64_t>(wgs, 256);
    const double steps = std::ceil((double)(K / 32) / S / 4.0);
    double t = (double)rounds * (GEMM_A + steps * c.step_us * (1.0 + GEMM_LOAD * per_round / 256.0));
    if (S > 1)
        t += SUM_A + SUM_US_PER_MB * (double)S * (double)M * (double)N * 4.0 / 1e6;
    return t;
}

// K split of the GEMM: the S in {1, 2, 4, 8} of least estimated time, each
// range at least two steps (8 k-tiles) and the split workgroups fitting one
// round on 256 compute units.
int gemm_split(int type, int64_t K, int64_t N, int64_t M)
{
    const int64_t blocks = gemm_blocks(N, M), nkt = K / 32;
    int best = 1;
    double best_t = gemm_cost_us(type, K, N, M, 1);
    for (int S = 2; S <= 8; S *= 2) {
        if (blocks * S > 256 || nkt / S < 8)
            break;
        const double t = gemm_cost_us(type, K, N, M, S);
        if (t < best_t)
            best = S, best_t = t;
    }
    return best;
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Workspaces of tq_matmul and tq_matmul_x: the decode K split's slots, which
// every call leaves zero, lie in the first SLOT_REGION bytes for every shape
// (the largest split workspace is below it); scratch (activation codes,
// partial planes) starts after it, so that no call writes into another
// shape's slots when calls of different shapes share one workspace.
constexpr size_t SLOT_REGION = TQ_NOALLOC_SCRATCH_BYTES;

// Bytes of tq_matmul's workspace for (type, K, N, M) and the K split S of
// its GEMM (1: none).
size_t matmul_ws_bytes(int type, int64_t K, int64_t N, int64_t M, int &S)
{
    S = 1;
    const size_t slots = tq_qgemv_workspace_bytes(type, K, N, M < 8 ? M : 8);
    if (M <= 8 || tq_matmul_path(type, K, N, M) != TQ_PATH_GEMM_SPLIT)
        return slots;
    S = gemm_split(kernel_type(type), K, N, M);
    return SLOT_REGION + (size_t)S * (size_t)M * (size_t)N * 4;
}

}  // namespace

extern "C" {

int tq_matmul_path(int type, int64_t K, int64_t N, int64_t M)
{
    if (!valid_type(type) || !valid_tkn(type, K, N) || !valid_mk(M, K))
        return -1;
    if (M <= 8)
        return TQ_PATH_GEMV;
    const int kt = kernel_type(type);
    const int S = gemm_split(kt, K, N, M);
    const double gemm = gemm_cost_us(kt, K, N, M, S);
    if (M <= 64) {
        const TypeCost c = type_cost(kt);
        const double pass = c.pass_a + (double)tq_tiled_bytes(type, K, N) / c.pass_bw;
        if ((double)((M + 7) / 8) * pass <= gemm)
            return TQ_PATH_GEMV;
    }
    return S > 1 ? TQ_PATH_GEMM_SPLIT : TQ_PATH_GEMM;
}

size_t tq_matmul_workspace_bytes(int type, int64_t K, int64_t N, int64_t M)
{
    if (!valid_type(type) || !valid_tkn(type, K, N) || !valid_mk(M, K) || N == 0 || M == 0)
        return 0;
    int S;
    return matmul_ws_bytes(type, K, N, M, S);
}

int tq_matmul(int type, const void *tiles, int64_t K, int64_t N, const int8_t *q,
              const uint16_t *d, int64_t M, const int8_t *lut, float *y, int64_t ldy,
              void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (M <= 8)
        return tq_qgemv(type, tiles, K, N, q, d, M, lut, y, ldy, workspace, workspace_bytes,
                        stream);
    int st = check_matmul(type, tiles, K, N, q, d, M, lut, y, ldy, true);
    if (st != TQ_OK || N == 0)
        return st;
    if (workspace && !aligned(workspace, 256))
        return TQ_E_ALIGN;
    const int path = tq_matmul_path(type, K, N, M);
    if (path == TQ_PATH_GEMV) {
        // decode passes of up to 8 rows each, all validated above
        const int64_t nkt = K / 32;
        for (int64_t m0 = 0; m0 < M; m0 += 8) {
            st = tq_qgemv(type, tiles, K, N, q + m0 * K, d + m0 * nkt, std::min<int64_t>(8, M - m0),
                          lut, y + m0 * ldy, ldy, workspace, workspace_bytes, stream);
            if (st != TQ_OK)
                return st;
        }
        return TQ_OK;
    }
    int S = 1;
    const size_t need = matmul_ws_bytes(type, K, N, M, S);
    if (path == TQ_PATH_GEMM_SPLIT && workspace && workspace_bytes >= need) {
        float *part = (float *)((uint8_t *)workspace + SLOT_REGION);
        return launch_status(tq::launch_qgemm_split(kernel_type(type), tiles, K, N, q, d, M,
                                                    pack_lut(type, lut), y, ldy, S, part,
                                                    stream));
    }
    return tq_qgemm(type, tiles, K, N, q, d, M, lut, y, ldy, stream);
}

}  // extern "C"

// tq_matmul_x: the fused decode (tq_qgemv_x) where its activation re-reads
// stay small, else tq_quantize_act into the workspace and tq_matmul.
namespace {
bool matmul_x_fused(int64_t N, int64_t M) { return M <= 8 && M * ((N + 31) / 32) <= 1024; }

// Workspace of tq_matmul_x: the slot region, then q, d and the GEMM's
// partial planes (S of them, 0 without a split).
struct XLayout {
    size_t slots, q, d, rest, total;
    int S;
};
XLayout matmul_x_layout(int type, int64_t K, int64_t N, int64_t M)
{
    XLayout L{};
    L.slots = tq_qgemv_workspace_bytes(type, K, N, M < 8 ? M : 8);
    if (matmul_x_fused(N, M)) {
        L.total = L.slots;
        L.S = 1;
        return L;
    }
    (void)matmul_ws_bytes(type, K, N, M, L.S);
    L.q = SLOT_REGION;
    L.d = align256(L.q + (size_t)M * (size_t)K);
    L.rest = align256(L.d + (size_t)M * (size_t)(K / 32) * 2);
    L.total = L.rest + (L.S > 1 ? (size_t)L.S * (size_t)M * (size_t)N * 4 : 0);
    return L;
}
}  // namespace

extern "C" {

size_t tq_matmul_x_workspace_bytes(int type, int64_t K, int64_t N, int64_t M)
{
    if (!valid_type(type) || !valid_tkn(type, K, N) || !valid_mk(M, K) || N == 0 || M == 0)
        return 0;
    return matmul_x_layout(type, K, N, M).total;
}

int tq_matmul_x(int type, const void *tiles, int64_t K, int64_t N, int dtype, const void *x,
                int64_t ldx, int64_t M, const int8_t *lut, float *y, int64_t ldy,
                void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (dtype != TQ_F32 && dtype != TQ_BF16 && dtype != TQ_F16)
        return TQ_E_TYPE;
    if (ldx < K || M * ldx >= MAX_PROD)
        return TQ_E_SHAPE;
    // x stands in for q in the common checks; its own alignment is checked below
    int st = check_matmul(type, tiles, K, N, (const int8_t *)tiles, nullptr, M, lut, y, ldy,
                          false);
    if (st != TQ_OK || M == 0 || N == 0)
        return st;
    if (!x)
        return TQ_E_NULL;
    if (!aligned(x, dtype == TQ_F32 ? 4 : 2) || (workspace && !aligned(workspace, 256)))
        return TQ_E_ALIGN;
    const XLayout L = matmul_x_layout(type, K, N, M);
    if (matmul_x_fused(N, M))
        return tq_qgemv_x(type, tiles, K, N, dtype, x, ldx, M, lut, y, ldy, workspace,
                          workspace_bytes, stream);
    if (!workspace)
        return TQ_E_NULL;
    if (workspace_bytes < L.rest)
        return TQ_E_SHAPE;
    uint8_t *ws = (uint8_t *)workspace;
    int8_t *q = (int8_t *)(ws + L.q);
    uint16_t *d = (uint16_t *)(ws + L.d);
    st = tq_quantize_act(dtype, x, M, K, ldx, q, d, stream);
    if (st != TQ_OK)
        return st;
    // tq_matmul's workspace: the slots at the front, the planes after q, d:
    // handed over as one buffer whose slot region is the front of ours
    if (M <= 8)
        return tq_qgemv(type, tiles, K, N, q, d, M, lut, y, ldy, workspace, L.slots, stream);
    const int path = tq_matmul_path(type, K, N, M);
    if (path == TQ_PATH_GEMV)
        return tq_matmul(type, tiles, K, N, q, d, M, lut, y, ldy, workspace, L.slots, stream);
    if (path == TQ_PATH_GEMM_SPLIT && workspace_bytes >= L.total)
        return launch_status(tq::launch_qgemm_split(kernel_type(type), tiles, K, N, q, d, M,
                                                    pack_lut(type, lut), y, ldy, L.S,
                                                    (float *)(ws + L.rest), stream));
    return tq_qgemm(type, tiles, K, N, q, d, M, lut, y, ldy, stream);
}

int tq_block_dots(int type, const void *tiles, int64_t K, int64_t N, const int8_t *q,
                  int64_t M, const int8_t *lut, int32_t *isum, int path, hipStream_t stream)
{
    if (path < TQ_PATH_GEMV || path > TQ_PATH_GEMM_FLAT)
        return TQ_E_TYPE;
    const bool flat = path == TQ_PATH_GEMV_FLAT || path == TQ_PATH_GEMM_FLAT;
    const bool gemv = path == TQ_PATH_GEMV || path == TQ_PATH_GEMV_FLAT;
    if (gemv && valid_type(type) && M > 8)
        return TQ_E_SHAPE;
    int st = check_matmul(type, tiles, K, N, q, nullptr, M, lut, isum, N, false,
                          flat ? flat_align(type) : 16);
    if (st != TQ_OK || M == 0 || N == 0)
        return st;
    if ((int64_t)M * N * (K / 32) >= MAX_PROD)
        return TQ_E_SHAPE;
    const tq::Lut t = pack_lut(type, lut);
    const tq::Act act{q, nullptr, nullptr, -1, 0};
    hipError_t e;
    switch (path) {
    case TQ_PATH_GEMV:
        e = tq::launch_qgemv(kernel_type(type), tiles, K, N, act, M, t, nullptr, N, isum, nullptr,
                             0, stream);
        break;
    case TQ_PATH_GEMM:
        e = tq::launch_qgemm(kernel_type(type), tiles, K, N, q, nullptr, M, t, nullptr, N, isum,
                             stream);
        break;
    case TQ_PATH_GEMV_FLAT:
        e = tq::launch_qgemv_flat(type, tiles, K, N, q, nullptr, M, t, nullptr, N, isum, stream);
        break;
    default:
        e = tq::launch_qgemm_flat(type, tiles, K, N, q, nullptr, M, t, nullptr, N, isum, stream);
        break;
    }
    return launch_status(e);
}

int tq_unpack_tiles(int type, const void *tiles, int64_t K, int64_t N, void *flat,
                    hipStream_t stream)
{
    if (!valid_type(type) || type == TQ_Q4_K)
        return TQ_E_TYPE;
    if (!valid_tkn(type, K, N))
        return TQ_E_SHAPE;
    if (N == 0)
        return TQ_OK;
    if (!flat || !tiles)
        return TQ_E_NULL;
    if (!aligned(flat, flat_align(type)) || !aligned(tiles, 16))
        return TQ_E_ALIGN;
    return launch_status(tq::launch_unpack(type, tiles, K, N, flat, stream));
}

int tq_qgemv_flat(int type, const void *flat, int64_t K, int64_t N, const int8_t *q,
                  const uint16_t *d, int64_t M, const int8_t *lut, float *y, int64_t ldy,
                  hipStream_t stream)
{
    if (valid_type(type) && M > 8)
        return TQ_E_SHAPE;
    int st = check_matmul(type, flat, K, N, q, d, M, lut, y, ldy, true, flat_align(type));
    if (st != TQ_OK || M == 0 || N == 0)
        return st;
    return launch_status(tq::launch_qgemv_flat(type, flat, K, N, q, d, M, pack_lut(type, lut),
                                               y, ldy, nullptr, stream));
}

int tq_qgemm_flat(int type, const void *flat, int64_t K, int64_t N, const int8_t *q,
                  const uint16_t *d, int64_t M, const int8_t *lut, float *y, int64_t ldy,
                  hipStream_t stream)
{
    int st = check_matmul(type, flat, K, N, q, d, M, lut, y, ldy, true, flat_align(type));
    if (st != TQ_OK || M == 0 || N == 0)
        return st;
    return launch_status(tq::launch_qgemm_flat(type, flat, K, N, q, d, M, pack_lut(type, lut),
                                               y, ldy, nullptr, stream));
}

int tq_matmul_flat(int type, const void *flat, int64_t K, int64_t N, const int8_t *q,
                   const uint16_t *d, int64_t M, const int8_t *lut, float *y, int64_t ldy,
                   hipStream_t stream)
{
    if (M <= 8)
        return tq_qgemv_flat(type, flat, K, N, q, d, M, lut, y, ldy, stream);
    return tq_qgemm_flat(type, flat, K, N, q, d, M, lut, y, ldy, stream);
}

int tq_quantize_act_mx(int dtype, const void *x, int64_t M, int64_t K, int64_t ldx, uint8_t *q,
                       uint8_t *e, hipStream_t stream)
{
    if (dtype != TQ_F32 && dtype != TQ_BF16 && dtype != TQ_F16)
        return TQ_E_TYPE;
    if (K < 32 || K > MAX_K || K % 32 != 0 || !valid_mk(M, K) || ldx < K ||
        M * ldx >= MAX_PROD)
        return TQ_E_SHAPE;
    if (M == 0)
        return TQ_OK;
    if (!x || !q || !e)
        return TQ_E_NULL;
    if (!aligned(x, dtype == TQ_F32 ? 4 : 2) || !aligned(q, 8))
        return TQ_E_ALIGN;
    return launch_status(tq::launch_quantize_mx(dtype, x, M, K, ldx, q, e, stream));
}

int tq_qgemm_mx(const void *tiles, int64_t K, int64_t N, const uint8_t *q, const uint8_t *e,
                int64_t M, float *y, int64_t ldy, hipStream_t stream)
{
    if (!valid_kn(K, N) || !valid_mk(M, K) || ldy < N)
        return TQ_E_SHAPE;
    if (M == 0 || N == 0)
        return TQ_OK;
    if (!tiles || !q || !e || !y)
        return TQ_E_NULL;
    if (!aligned(tiles, 16) || !aligned(q, 16) || !aligned(y, 4))
        return TQ_E_ALIGN;
    return launch_status(tq::launch_qgemm_mx(tiles, K, N, q, e, M, y, ldy, 1, nullptr, stream));
}

}  // extern "C"

namespace {

// K split of the block-scaled GEMM for output grids too small to fill the
// chip, from a cost model fitted to times measured on MI355X (K = 4096 and
// 8192, N = 4096 and 14336, M = 8 .. 512): a launch of one round (its 64 x
// 128 output blocks times the S ranges, at most one per compute unit) takes
// MX_A + MX_STAGE per 256-K stage of a range, and a split adds the sum of
// the S partial planes (SUM_A + SUM_US_PER_MB per MB read and written).
// S = 1, 2, 4 or 8, each range at least two stages; ties keep the smaller S.
constexpr double MX_A = 7.0, MX_STAGE = 0.77;
int mx_split(int64_t K, int64_t N, int64_t M)
{
    const int64_t blocks = ((N + 127) / 128) * ((M + 63) / 64);
    const int64_t nkt = K / 32;
    int best = 1;
    double best_us = 0.0;
    for (int S = 1; S <= 8; S *= 2) {
        if (S > 1 && (blocks * S > 256 || nkt / S < 16))
            break;
        const double stages = (double)((nkt + 8 * S - 1) / (8 * S));
        double us = MX_A + MX_STAGE * stages;
        if (S > 1)
            us += SUM_A + SUM_US_PER_MB * (double)(S + 1) * (double)M * (double)N * 4e-6;
        if (S == 1 || us < best_us) {
            best = S;
            best_us = us;
        }
    }
    return best;
}

bool mx_args_valid(int64_t K, int64_t N, int64_t M)
{
    return valid_kn(K, N) && valid_mk(M, K);
}

}  // namespace

extern "C" {

size_t tq_matmul_mx_workspace_bytes(int64_t K, int64_t N, int64_t M)
{
    if (!mx_args_valid(K, N, M) || N == 0 || M == 0)
        return 0;
    const int S = mx_split(K, N, M);
    return S > 1 ? SLOT_REGION + (size_t)S * (size_t)M * (size_t)N * 4 : 0;
}

int tq_matmul_mx(const void *tiles, int64_t K, int64_t N, const uint8_t *q, const uint8_t *e,
                 int64_t M, float *y, int64_t ldy, void *workspace, size_t workspace_bytes,
                 hipStream_t stream)
{
    if (!mx_args_valid(K, N, M) || ldy < N)
        return TQ_E_SHAPE;
    if (M == 0 || N == 0)
        return TQ_OK;
    if (!tiles || !q || !e || !y)
        return TQ_E_NULL;
    if (!aligned(tiles, 16) || !aligned(q, 16) || !aligned(y, 4) ||
        (workspace && !aligned(workspace, 256)))
        return TQ_E_ALIGN;
    const int S = mx_split(K, N, M);
    const size_t need = tq_matmul_mx_workspace_bytes(K, N, M);
    if (S > 1 && workspace && workspace_bytes >= need) {
        float *part = (float *)((uint8_t *)workspace + SLOT_REGION);
        return launch_status(tq::launch_qgemm_mx(tiles, K, N, q, e, M, y, ldy, S, part, stream));
    }
    return launch_status(tq::launch_qgemm_mx(tiles, K, N, q, e, M, y, ldy, 1, nullptr, stream));
}

}  // extern "C"
