/*
 * tiledq -- matrix-vector and matrix-matrix multiply over block-32 quantized
 * weights repacked into 32x32 tiles, on AMD Instinct MI355X (gfx950).
 *
 * Formats follow the page "Hexagon backend developer details", section
 * "Tiled Weight Formats":
 *
 *   Grid ("Tile Dimensions and Grid Layout").  A weight matrix of logical
 *   shape [ne0, ne1] = [K, N] (N output rows of K elements each) is cut into
 *   32-row x 32-column tiles: n_k_tiles = K / 32, n_col_tiles = (N + 31) / 32.
 *   The tile of row-tile ct (output rows 32ct..32ct+31) and column-tile kt
 *   (K indices 32kt..32kt+31) sits at byte (ct * n_k_tiles + kt) * tile_size,
 *   so the n_k_tiles tiles of one 32-row stripe are contiguous.
 *
 *   Tiles ("Block-32 Quantized Formats"), quant[row][col] for row, col < 32:
 *     Q4_0   576 B: bytes cp*32 + row (cp = 0..15) hold quant[row][2cp] in the
 *            low nibble and quant[row][2cp+1] in the high nibble; bytes
 *            512 + 2*row hold row's fp16 scale d.  Weight = d * (quant - 8).
 *     Q8_0  1088 B: byte cp*64 + 2*row + h holds int8 quant[row][2cp + h];
 *            bytes 1024 + 2*row hold the fp16 scale d.  Weight = d * quant.
 *     IQ4_NL 576 B: the Q4_0 layout, each nibble an index into a 16-entry
 *            table.  Weight = d * lut[index].
 *     MXFP4  544 B: the Q4_0 nibble layout of OCP FP4 (E2M1) codes; byte
 *            512 + row holds row's E8M0 scale byte e.  Weight =
 *            E2M1(code) * s(e), s(e) the fp16 power of two with exponent
 *            bits clamp(e - 112, 0, 30): 2^(e-127) for 113 <= e <= 142, 0
 *            for e <= 112, 2^15 for e > 142.  The kernels multiply the
 *            integers 2 * E2M1(code) (0, 1, 2, 3, 4, 6, 8, 12 and their
 *            negatives) by s(e) / 2, exactly.
 *     Q4_1   640 B: the Q4_0 nibble layout of codes 0..15; bytes 512 + 4*row
 *            hold row's fp16 scale d, bytes 514 + 4*row its fp16 min m.
 *            Weight = d * quant + m.
 *     Q4_K   640 B: a Q4_1 tile ("K-Quants") whose pair is (d * sc, -dmin * m)
 *            of the 32-k sub-block: fp32 products rounded to fp16
 *            nearest-even.  Computed exactly like Q4_1.
 *   Rows n >= N of the last row-tile are zero (codes 0, scale +0.0).
 *
 *   Flat source ("repacked from flat row-major GGML layouts"): row n holds
 *   K/32 consecutive GGML blocks: Q4_0 / IQ4_NL = fp16 d + 16 bytes (low
 *   nibbles elements 0..15, high nibbles 16..31), 18 B; Q8_0 = fp16 d + 32
 *   int8, 34 B; MXFP4 = E8M0 byte e + 16 bytes in the Q4_0 nibble order,
 *   17 B; Q4_1 = fp16 d + fp16 m + 16 bytes in the Q4_0 nibble order, 20 B.
 *   Q4_K: 256-element super-blocks of 144 B (K % 256 == 0, else
 *   TQ_E_SHAPE): fp16 d, fp16 dmin, 12 bytes of eight 6-bit scales sc and
 *   mins m (sub-block j < 4: low 6 bits of bytes j, j + 4; j >= 4: the low /
 *   high nibble of byte j + 4 plus the top 2 bits of byte j - 4 / j), then
 *   128 nibble bytes: 64-element chunk c at bytes 32c.., its first 32
 *   elements in the low nibbles.
 *
 *   Activations (section "Memory buffers": dynamically quantized activations,
 *   used as Q8_0 activation tiles by the vector dot of "Q2_0 Format"): per
 *   32-element K block, d = amax/127 (fp32), q = round-half-away(x * (1/d)),
 *   d stored as fp16 (nearest-even).  q is int8 row-major [M][K], d is fp16
 *   [M][K/32].  Domain: finite x, each block all zero or with
 *   2^-120 <= amax <= 65504 * 127: 1/d stays finite and the stored fp16 d
 *   stays finite (it may be an fp16 subnormal, or round to zero, for
 *   amax below about 7.75e-3 and 3.8e-6).  Outside it the results are
 *   unspecified.
 *
 *   Product: y[m*ldy + n] = sum_k W[n][k] * A[m][k] for m < M, n < N, with
 *   W the dequantized weights and A[m][k] = d[m][k/32] * q[m][k] (GGML's
 *   dst = src0^T * src1).  Per 32-element block the integer dot
 *   isum = sum_j w_int * q is formed exactly in int32, then scaled by the
 *   fp16 row scale times the fp16 activation scale (exact in fp32) and
 *   summed in fp32 over blocks.  Q4_1's min adds m * da * sum_j q per block
 *   (the activation sum exact in int32, times da exact in fp32).
 *
 * Calling convention (all entry points):
 *   - Data pointers are DEVICE pointers, except `lut`, which is a HOST
 *     pointer to 16 int8 (copied by value into the launch; may be freed on
 *     return).  The caller allocates and owns every buffer; the library
 *     allocates nothing, frees nothing and keeps no pointer after return.
 *   - Each call validates its arguments on the host, then enqueues its
 *     kernel(s) on `stream` (NULL = the default stream) and returns without
 *     synchronizing.  Buffers must stay alive until that work has completed.
 *     Faults inside a kernel surface at the caller's next synchronization.
 *   - Validation errors are returned before anything is enqueued and leave
 *     every output untouched.  M == 0 or N == 0 is TQ_OK with no launch.
 *   - The library is stateless; calls on different streams may run
 *     concurrently.  Outputs of concurrent calls must not overlap.
 *   - Shapes: 32 <= K <= 2^20 with K % 32 == 0 (Q4_K: K % 256 == 0);
 *     0 <= N <= 2^27;
 *     0 <= M <= 2^20; K*N below 2^40 and M*K below 2^34 (so that every
 *     kernel's grid fits the 32-bit work-item count of a dispatch).
 *     Shapes outside these limits return TQ_E_SHAPE.
 */
#ifndef TILEDQ_H
#define TILEDQ_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TQ_Q4_0 = 0, TQ_Q8_0 = 1, TQ_IQ4_NL = 2, TQ_MXFP4 = 3, TQ_Q4_1 = 4, TQ_Q4_K = 5
} tq_type;
typedef enum { TQ_F32 = 0, TQ_BF16 = 1, TQ_F16 = 2 } tq_dtype;
typedef enum {
    TQ_OK = 0,
    TQ_E_NULL = 1,    /* a required pointer is NULL                           */
    TQ_E_TYPE = 2,    /* unknown tq_type / tq_dtype / path                    */
    TQ_E_SHAPE = 3,   /* K, N, M, ldx or ldy outside the documented domain     */
    TQ_E_ALIGN = 4,   /* a pointer lacks the documented alignment             */
    TQ_E_LAUNCH = 5   /* the HIP runtime rejected a launch                    */
} tq_status;

/* Which kernel family tq_block_dots runs, and whether its weights are tiles
 * or flat GGML blocks. */
typedef enum {
    TQ_PATH_GEMV = 0, TQ_PATH_GEMM = 1, TQ_PATH_GEMV_FLAT = 2, TQ_PATH_GEMM_FLAT = 3,
    TQ_PATH_GEMM_MX = 4,   /* tq_qgemm_mx: MXFP4 tiles only */
    TQ_PATH_GEMM_SPLIT = 5 /* tq_matmul: the GEMM with K split over workgroups */
} tq_path;

/* Bytes of one tile ("Block-32 Quantized Formats"): 576, 1088, 576, 544,
 * 640, 640; 0 for an unknown type. */
size_t tq_tile_bytes(int type);

/* Bytes of one flat GGML block: 18, 34, 18, 17, 20 (32 elements each), and
 * 144 for a 256-element Q4_K super-block; 0 for an unknown type.  The pages
 * name the flat source ("Tiled Weight Formats": weights repacked from flat
 * row-major GGML layouts) but do not print it.  The reading taken is GGML's
 * own block of 32 elements: the scale field(s) followed by the quants, so
 * that one tile holds exactly 32 blocks (576 = 32 * 18, 1088 = 32 * 34,
 * 544 = 32 * 17, 640 = 32 * 20, per the tile sizes of "Block-32 Quantized
 * Formats"). */
size_t tq_block_bytes(int type);

/* (K/32) * ((N+31)/32) * tq_tile_bytes(type) ("Tile Dimensions and Grid
 * Layout"); 0 if the shape or type is invalid. */
size_t tq_tiled_bytes(int type, int64_t K, int64_t N);

/* N * (K/32) * tq_block_bytes(type) (Q4_K: N * (K/256) * 144); 0 if the
 * shape or type is invalid.  Row n's blocks are contiguous and rows follow
 * one another: the flat-block reading stated at tq_block_bytes. */
size_t tq_flat_bytes(int type, int64_t K, int64_t N);

/* 1 if (type, K, N, M) is supported by `path` (TQ_PATH_GEMV and
 * TQ_PATH_GEMV_FLAT need M <= 8; Q4_K needs K % 256 == 0; TQ_PATH_GEMM_MX
 * takes TQ_MXFP4 only), judged from these static properties alone; 0
 * otherwise.  No pointer is needed or read: the page's "supports_op
 * Independence from Buffer and Repack State" has support decided from
 * operand types, shapes and operation parameters only, before any buffer
 * exists, and every type supported tiled is supported flat as well. */
int tq_supported(int type, int64_t K, int64_t N, int64_t M, int path);

/* Static, NUL-terminated name of a status code.  The codes follow the
 * status convention of the page's operators: an empty range returns OK
 * ("Multi-Device Partitioning" > "Row-Partitioned Operators": nrows == 0
 * returns the OK status) and any status above OK is an error
 * ("Multi-Device Synchronization" > "Deterministic Monotonic Sequence
 * Numbers": a peer status greater than OK propagates as an error).  Unknown
 * codes give "unknown tq_status". */
const char *tq_status_string(int status);

/* Repack flat GGML blocks into tiles ("Tiled Weight Formats": repacking at
 * model load or at run time).
 *   flat  : device, tq_flat_bytes(type, K, N) bytes, 2-byte aligned
 *           (TQ_MXFP4, TQ_Q4_1: 4-byte aligned; TQ_Q4_K: 16-byte aligned).
 *   tiles : device, tq_tiled_bytes(type, K, N) bytes, 16-byte aligned; fully
 *           written, padding rows included.  Must not overlap `flat`.
 * Bit-exact byte permutation; deterministic. */
int tq_repack_tiles(int type, const void *flat, int64_t K, int64_t N,
                    void *tiles, hipStream_t stream);

/* Dynamic activation quantization ("Memory buffers"), per 32-element block.
 *   x   : device, M rows of K elements at row stride ldx (>= K) elements;
 *         fp32 (4-byte aligned) or bf16 / fp16 (2-byte aligned), per dtype.
 *   q   : device, int8 [M][K] row-major, 4-byte aligned.
 *   d   : device, fp16 bits [M][K/32] row-major, 2-byte aligned.
 * Bit-exact (IEEE fp32 divide, round half away from zero, fp16 nearest-even). */
int tq_quantize_act(int dtype, const void *x, int64_t M, int64_t K, int64_t ldx,
                    int8_t *q, uint16_t *d, hipStream_t stream);

/* Bytes of workspace tq_qgemv can use for (type, K, N, M) to split K across
 * workgroups when N alone gives too few of them (0: no split is useful, or
 * the arguments are invalid). */
size_t tq_qgemv_workspace_bytes(int type, int64_t K, int64_t N, int64_t M);

/* Decode matrix-vector product over tiles (M <= 8 activation rows), reading
 * every weight tile exactly once.  Per tile and activation row, the integer
 * dot of the 32 decoded weights with the 32 int8 activations is formed in
 * int32 (the int8 multiply-accumulate into 32-bit words against Q8_0
 * activation tiles of "Q2_0 Format" > "HVX Vector Dot-Product"), then
 * multiplied by the row scale d ("Block-32 Quantized Formats": each decoded
 * quant is multiplied by the row scale d) and by the activation scale.
 *   tiles : device, tq_tiled_bytes(type, K, N) bytes, 16-byte aligned.
 *   q, d  : device, from tq_quantize_act with the same M and K; q 16-byte
 *           aligned, d 2-byte aligned.
 *   M     : 1..8 (else TQ_E_SHAPE).
 *   lut   : host, 16 int8 table entries for TQ_IQ4_NL (required), ignored
 *           (may be NULL) for the other types (TQ_MXFP4's values are fixed
 *           by E2M1).
 *   y     : device fp32, y[m*ldy + n] written for m < M, n < N only;
 *           ldy >= N; 4-byte aligned.
 *   workspace, workspace_bytes : optional device scratch, 256-byte aligned,
 *           owned by the caller.  It must be zero-filled before its first
 *           use; every call leaves it zero-filled again, so it can be reused
 *           by later calls of any shape without clearing.  Calls that share
 *           a workspace must not run concurrently.  With NULL or fewer than
 *           tq_qgemv_workspace_bytes() bytes the K dimension is not split
 *           (the same terms summed in another order, fewer workgroups).
 * Deterministic: each mode (with a large enough workspace, or without) is
 * bitwise repeatable, its partial sums added in a fixed order; the two
 * modes add the per-block terms in different orders, so their results may
 * differ in the last bits (both within the fp32 bound of the sum). */
int tq_qgemv(int type, const void *tiles, int64_t K, int64_t N,
             const int8_t *q, const uint16_t *d, int64_t M,
             const int8_t *lut, float *y, int64_t ldy,
             void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of the device scratch array behind tq_qgemv_noalloc (1 MiB per
 * GPU).  It covers the K-split workspace of every shape tq_qgemv accepts:
 * tq_qgemv_workspace_bytes() never exceeds it. */
#define TQ_NOALLOC_SCRATCH_BYTES (1u << 20)

/* tq_qgemv for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.
 * Arguments and results as tq_qgemv with a workspace of
 * tq_qgemv_workspace_bytes() bytes: the K split's reduction slots live in a
 * device array of TQ_NOALLOC_SCRATCH_BYTES inside the library (one per GPU,
 * held until the process ends), so y is bit-identical to tq_qgemv given such
 * a workspace.  The call allocates and frees nothing; the caller passes the
 * inputs and the output.  The first call on a device looks up the array's
 * address and clears it with a kernel on `stream`; every call leaves it
 * zero again.  All calls on one GPU share the array: calls that may overlap
 * on one GPU (different streams, or concurrent graph replays) race and give
 * undefined results; serialize them.  A shape whose workspace would exceed
 * the array returns TQ_E_SHAPE (none of the accepted shapes does); a failed
 * address lookup or clear returns TQ_E_LAUNCH. */
int tq_qgemv_noalloc(int type, const void *tiles, int64_t K, int64_t N,
                     const int8_t *q, const uint16_t *d, int64_t M,
                     const int8_t *lut, float *y, int64_t ldy, hipStream_t stream);

/* Decode in one launch: tq_quantize_act fused into tq_qgemv.  Each
 * workgroup quantizes the activation blocks it needs into on-chip memory
 * with the same arithmetic as tq_quantize_act, so y is bit-identical to
 * tq_quantize_act followed by tq_qgemv with the same workspace.
 *   dtype, x, ldx : as tq_quantize_act (device x, row stride ldx >= K).
 *   other arguments as tq_qgemv.
 * Every workgroup reads and quantizes its K range of all M rows, i.e. the
 * activations are read N / 32 times: the fused launch pays off for small
 * products (one launch saved, e.g. M = 1, K = N = 4096; level at M = 4),
 * while for large N or M >= 8 (a vocabulary head, several rows)
 * tq_quantize_act followed by tq_qgemv is faster. */
int tq_qgemv_x(int type, const void *tiles, int64_t K, int64_t N,
               int dtype, const void *x, int64_t ldx, int64_t M,
               const int8_t *lut, float *y, int64_t ldy,
               void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Prefill matrix-matrix product over tiles with int8 matrix-core (MFMA)
 * instructions, any M >= 1.  Arguments as tq_qgemv without the workspace.
 * The same arithmetic as tq_qgemv: exact int32 block dots of decoded weights
 * and int8 activations ("Q2_0 Format" > "HVX Vector Dot-Product": int8
 * multiply-accumulate into 32-bit words against Q8_0 activation tiles),
 * each multiplied by the row scale d ("Block-32 Quantized Formats") and the
 * activation scale, summed in fp32.  The pages' prefill converts weights to
 * FP16 for the matrix unit ("Q2_0 Format" > "HMX Mapping"); here the
 * matrix unit takes the int8 operands, so that tq_qgemv and tq_qgemm form
 * identical block dots.  Deterministic. */
int tq_qgemm(int type, const void *tiles, int64_t K, int64_t N,
             const int8_t *q, const uint16_t *d, int64_t M,
             const int8_t *lut, float *y, int64_t ldy, hipStream_t stream);

/* The path tq_matmul takes for (type, K, N, M), given a workspace of
 * tq_matmul_workspace_bytes(type, K, N, M) bytes (-1: invalid arguments):
 *   TQ_PATH_GEMV       M <= 8: one tq_qgemv launch; 9 <= M <= 64: ceil(M / 8)
 *                      decode passes (rows 0..7, 8..15, ...), each streaming
 *                      all tiles, where estimated no slower than the GEMM;
 *   TQ_PATH_GEMM_SPLIT the GEMM with K split into S ranges (S = 2, 4 or 8) when
 *                      its 128 x 64 output blocks would leave most of the 256
 *                      compute units idle ("Op and Kernel Development
 *                      Guidelines" > "Work Queue and Threading": workers take
 *                      independent chunks): each range writes a partial fp32
 *                      plane into the workspace and a second launch adds the S
 *                      planes in a fixed order;
 *   TQ_PATH_GEMM       the GEMM (tq_qgemm).
 * The estimate uses per-type costs measured on MI355X (a decode pass ~5.5 us
 * plus the tiles at 4.5 (IQ4_NL, MXFP4) to 7.0 (Q8_0) TB/s; a GEMM round of up
 * to 256 output blocks 29 (Q4_0) to 46 (Q4_1, Q4_K) us x K / 4096; a split
 * round ~round / S + 2 us, plus the sum of the planes).  Static properties
 * only. */
int tq_matmul_path(int type, int64_t K, int64_t N, int64_t M);

/* Bytes of workspace tq_matmul uses for (type, K, N, M) (0: none, or invalid
 * arguments).  Layout shared by tq_matmul and tq_matmul_x: the decode K
 * split's slots (tq_qgemv_workspace_bytes for up to 8 rows; for every shape
 * they lie in the first TQ_NOALLOC_SCRATCH_BYTES) must be zero before the
 * first use and are left zero by every call; scratch starts at byte
 * TQ_NOALLOC_SCRATCH_BYTES (on TQ_PATH_GEMM_SPLIT, S * M * N fp32 partial
 * planes) and its contents do not matter.  So one zero-filled workspace, as
 * large as the largest call needs, serves calls of any shapes, in turn. */
size_t tq_matmul_workspace_bytes(int type, int64_t K, int64_t N, int64_t M);

/* The product for any M, on the path tq_matmul_path() names: tq_qgemv (M <= 8,
 * or one pass per 8 rows), the split GEMM, or tq_qgemm.  Arguments as
 * tq_qgemv, except that M >= 0 is unbounded (TQ_E_SHAPE only for the limits
 * of the calling convention) and the workspace (256-byte aligned, layout as
 * tq_matmul_workspace_bytes states) may be smaller than that size: without
 * room for the planes the GEMM runs unsplit, without room for the slots the
 * decode runs unsplit (same results up to the order of the fp32 sums).
 * Calls sharing a workspace must not run concurrently.  Deterministic for a
 * given workspace size. */
int tq_matmul(int type, const void *tiles, int64_t K, int64_t N,
              const int8_t *q, const uint16_t *d, int64_t M,
              const int8_t *lut, float *y, int64_t ldy,
              void *workspace, size_t workspace_bytes, hipStream_t stream);

/* The whole product from fp32 / bf16 / fp16 activations, any M: for M <= 8
 * with M * ceil(N / 32) <= 1024 the fused decode (tq_qgemv_x, which reads
 * its K range of x once per 32-row stripe, cheap while that is small);
 * otherwise tq_quantize_act into the workspace followed by tq_matmul on its
 * path.  y is bit-identical to tq_quantize_act + tq_matmul (or tq_qgemv_x)
 * with the same workspace regions.
 *   dtype, x, ldx : as tq_quantize_act;  other arguments as tq_matmul.
 *   workspace : device, 256-byte aligned, tq_matmul_x_workspace_bytes(type,
 *     K, N, M) bytes, laid out as tq_matmul's: the decode slots (zero before
 *     the first use, left zero), then from TQ_NOALLOC_SCRATCH_BYTES on, as
 *     scratch, q (M * K int8), d (M * K/32 fp16) and the GEMM's planes.  The
 *     unfused path without room for q and d returns TQ_E_SHAPE (NULL
 *     workspace: TQ_E_NULL); without room for the planes the GEMM runs
 *     unsplit. */
size_t tq_matmul_x_workspace_bytes(int type, int64_t K, int64_t N, int64_t M);
int tq_matmul_x(int type, const void *tiles, int64_t K, int64_t N,
                int dtype, const void *x, int64_t ldx, int64_t M,
                const int8_t *lut, float *y, int64_t ldy,
                void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Flat (un-repacked) weights ("supports_op Independence from Buffer and
 * Repack State": every supported type must work tiled and stored flat).
 *
 * tq_unpack_tiles: the inverse of tq_repack_tiles, rows n < N only.
 *   tiles : device, tq_tiled_bytes(type, K, N) bytes, 16-byte aligned.
 *   flat  : device, tq_flat_bytes(type, K, N) bytes, aligned as for
 *           tq_repack_tiles; fully written.  Must not overlap `tiles`.
 *   TQ_Q4_K is rejected (TQ_E_TYPE): its tiles keep d * sc and -dmin * m,
 *   not the super-block's fields.  Bit-exact; deterministic. */
int tq_unpack_tiles(int type, const void *tiles, int64_t K, int64_t N,
                    void *flat, hipStream_t stream);

/* Products over flat GGML blocks, with the same results as over the tiles
 * of the same data (each weight the value its tile holds; Q4_K with the
 * fp16 pairs of its tile).  Arguments as tq_qgemv / tq_qgemm / tq_matmul,
 * with `flat` (device, tq_flat_bytes(type, K, N) bytes, aligned as for
 * tq_repack_tiles) in place of the tiles and no workspace.
 * tq_qgemv_flat: M <= 8 (else TQ_E_SHAPE); tq_qgemm_flat: any M;
 * tq_matmul_flat: dispatched on M as tq_matmul. */
int tq_qgemv_flat(int type, const void *flat, int64_t K, int64_t N,
                  const int8_t *q, const uint16_t *d, int64_t M,
                  const int8_t *lut, float *y, int64_t ldy, hipStream_t stream);
int tq_qgemm_flat(int type, const void *flat, int64_t K, int64_t N,
                  const int8_t *q, const uint16_t *d, int64_t M,
                  const int8_t *lut, float *y, int64_t ldy, hipStream_t stream);
int tq_matmul_flat(int type, const void *flat, int64_t K, int64_t N,
                   const int8_t *q, const uint16_t *d, int64_t M,
                   const int8_t *lut, float *y, int64_t ldy, hipStream_t stream);

/* MXFP4 on block-scaled matrix cores.  The page's MXFP4 tiles ("MXFP4":
 * E2M1 codes with one E8M0 scale per row and 32-element block) multiplied by
 * activations in the matching OCP Microscaling format, MXFP8: FP8 E4M3 codes
 * with one E8M0 scale per 32 elements, so that the matrix core applies both
 * power-of-two scales itself.  This is a second activation format beside the
 * page's Q8_0 one (tq_quantize_act); results differ from tq_qgemm on the
 * same MXFP4 tiles by the activation rounding.
 *
 * tq_quantize_act_mx: per 32-element block of each row (OCP Microscaling
 * v1.0 conversion): e = floor(log2 amax) - 8 + 127, clamped to 0..254 (0 for
 * an all-zero block); q = the E4M3 code nearest to x / 2^(e - 127), ties to
 * even, magnitudes above 448 saturating to 448, sign bit = x's sign bit.
 * Never writes the NaN codes 0x7F / 0xFF.  Bit-exact, deterministic.
 *   x : device, dtype TQ_F32 / TQ_BF16 / TQ_F16, row m at x + m*ldx
 *       elements (ldx >= K), aligned to its element size.
 *   q : device, uint8 [M][K] E4M3 codes, 8-byte aligned.
 *   e : device, uint8 [M][K/32] E8M0 bytes.
 *   K % 32 == 0 (else TQ_E_SHAPE); M == 0 returns TQ_OK with no launch.
 *
 * tq_qgemm_mx: y[m*ldy + n] = sum_k W[n][k] * A[m][k] for m < M, n < N, with
 * W the MXFP4 tile weights (E2M1 value times the FP16 power of two of
 * exponent bits clamp(e - 112, 0, 30), exactly as the page converts the
 * E8M0 byte: rows with e <= 112 weigh 0) and A[m][k] = E4M3(q[m][k]) *
 * 2^(e[m][k/32] - 127).  Any M >= 1; fp32 sums in the matrix core (not
 * bit-reproducible against a sequential fp32 sum: see the tolerance the
 * tests state).
 *   tiles : device, tq_tiled_bytes(TQ_MXFP4, K, N) bytes, 16-byte aligned.
 *   q, e  : device, as written by tq_quantize_act_mx (q 16-byte aligned);
 *           q must hold no NaN code.
 *   y     : device fp32, row stride ldy >= N, 4-byte aligned; only n < N,
 *           m < M written.
 *   Errors as tq_qgemm.  Deterministic. */
int tq_quantize_act_mx(int dtype, const void *x, int64_t M, int64_t K, int64_t ldx,
                       uint8_t *q, uint8_t *e, hipStream_t stream);
int tq_qgemm_mx(const void *tiles, int64_t K, int64_t N, const uint8_t *q,
                const uint8_t *e, int64_t M, float *y, int64_t ldy,
                hipStream_t stream);

/* tq_qgemm_mx with the K dimension split over S = 2, 4 or 8 workgroups per
 * output block when its 64 x 128 output blocks would leave most of the 256
 * compute units idle (small M), as tq_matmul splits the int8 GEMM ("Op and
 * Kernel Development Guidelines" > "Work Queue and Threading": workers take
 * independent chunks): each range writes a partial fp32 plane into the
 * workspace and a second launch adds the S planes in a fixed order.  The
 * split is chosen from (K, N, M) alone, by a cost model fitted to times
 * measured on MI355X (a split only where it is estimated faster).
 * tq_matmul_mx_workspace_bytes: the bytes that split needs (0: no split for
 * this shape, or invalid arguments); the layout is tq_matmul's (planes from
 * byte TQ_NOALLOC_SCRATCH_BYTES on, the first TQ_NOALLOC_SCRATCH_BYTES
 * untouched), so one workspace serves both.
 * tq_matmul_mx: arguments as tq_qgemm_mx plus the workspace (device,
 * 256-byte aligned, caller-owned); with a smaller workspace (or none) the
 * product runs unsplit.  Deterministic for a given workspace size; split
 * and unsplit results differ only in the order of the fp32 sums.  Calls
 * sharing a workspace must not run concurrently. */
size_t tq_matmul_mx_workspace_bytes(int64_t K, int64_t N, int64_t M);
int tq_matmul_mx(const void *tiles, int64_t K, int64_t N, const uint8_t *q,
                 const uint8_t *e, int64_t M, float *y, int64_t ldy,
                 void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Test instrument for the per-block integer dot ("Q2_0 Format" > "HVX
 * Vector Dot-Product": int8 products accumulated in 32-bit words, before the
 * row scale d of "Block-32 Quantized Formats" is applied): run the tq_qgemv
 * (path TQ_PATH_GEMV, M <= 8) or tq_qgemm
 * (TQ_PATH_GEMM) kernel, or their flat forms (TQ_PATH_GEMV_FLAT,
 * TQ_PATH_GEMM_FLAT; `tiles` then holds flat blocks, aligned as for
 * tq_repack_tiles), with the integer block dots as output instead of y:
 * isum[(m*N + n)*(K/32) + kt] (int32, device, 4-byte aligned) =
 * sum_{j<32} w_int[n][32kt+j] * q[m][32kt+j], for m < M, n < N, with w_int
 * = code - 8 (Q4_0), the int8 (Q8_0), lut[code] (IQ4_NL), 2 * E2M1(code)
 * (MXFP4) or the code itself (Q4_1 and Q4_K, whose min is not part of the
 * block dot). */
int tq_block_dots(int type, const void *tiles, int64_t K, int64_t N,
                  const int8_t *q, int64_t M, const int8_t *lut,
                  int32_t *isum, int path, hipStream_t stream);

/* Measurement instrument, outside the product path: the achievable HBM read
 * rate that the decode's weight stream ("Tiled Weight Formats": a stripe's
 * tiles are one contiguous byte range, streamed once per call) is compared
 * with.  Reads `bytes` bytes at `src` once, with 16-byte nontemporal loads
 * in a grid-stride loop over TQ_STREAM_READ_BLOCKS workgroups of 256
 * work-items, and writes to sink[b] the XOR of the 32-bit words workgroup b
 * read, so the XOR of the TQ_STREAM_READ_BLOCKS sink words is the XOR of
 * every 32-bit word of the buffer.
 *   src  : device, 16-byte aligned; bytes a multiple of 16 (else TQ_E_ALIGN,
 *          TQ_E_SHAPE).
 *   sink : device uint32[TQ_STREAM_READ_BLOCKS], 4-byte aligned, caller-owned;
 *          every word is written.
 * bytes == 0: TQ_OK, no launch, sink untouched. */
#define TQ_STREAM_READ_BLOCKS 2048
int tq_stream_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TILEDQ_H */
