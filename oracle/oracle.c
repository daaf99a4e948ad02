/*
 * Plain, slow CPU oracle for tiled block-32 quantized matmul.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path (the
 * HIP library and its Python binding) never calls it and shares no code,
 * header, table or constant with it.
 *
 * Source of every definition: the page "Hexagon backend developer details",
 * section "Tiled Weight Formats" with its subsections "Tile Dimensions and Grid Layout" and
 * "Block-32 Quantized Formats" (Q4_0, Q8_0, IQ4_NL, MXFP4, Q4_1), and section "Memory
 * buffers" (dynamically quantized activations).  Where the page is silent the
 * reading taken is stated at the function.  The MXFP8 activation side of the
 * MXFP4 block-scaled product (or_quantize_act_mx, or_matmul_mx) follows the
 * OCP Microscaling Formats specification v1.0, stated at the functions.
 *
 * Everything is scalar C, one element at a time, in the order the page states
 * it.  Floating-point results are fp64 unless the data format fixes the
 * precision (fp16 scales, fp32 activation quantization).
 *
 * Parity pins: every exported function is pinned by the tests under
 * tests/test_oracle_*.py except or_flat_decode's nibble order (the flat GGML
 * block layout is not printed on the page), which is "parity unpinned" by the
 * page and only self-consistent with the input generator.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_Q4_0 = 0, OR_Q8_0 = 1, OR_IQ4_NL = 2, OR_MXFP4 = 3, OR_Q4_1 = 4, OR_Q4_K = 5 };
enum { OR_F32 = 0, OR_BF16 = 1, OR_F16 = 2 };

/* ---------------------------------------------------------------------------
 * IEEE 754 binary16 / bfloat16 conversions, written from the format
 * definitions (1 sign bit, 5 exponent bits with bias 15, 10 fraction bits;
 * bfloat16 is the upper half of a binary32).
 * ------------------------------------------------------------------------- */

/* binary16 bits -> value, exact (every binary16 value is a binary32 value). */
float or_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);              /* subnormal: f * 2^-24 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);  /* (1 + f/1024) * 2^(e-15) */
    return (float)(sign ? -v : v);
}

/* value -> binary16 bits, round to nearest, ties to even, with subnormals and
 * overflow to infinity. */
uint16_t or_f32_to_f16(float x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs((double)x);
    if (isnan(x))
        return 0x7e00;
    if (a >= 65520.0)                 /* halfway to 2^16 and above: infinity */
        return sign | 0x7c00;
    if (a == 0.0)
        return sign;
    int ex;
    frexp(a, &ex);                    /* a = m * 2^ex, 0.5 <= m < 1 */
    int e = ex - 1;                   /* a in [2^e, 2^(e+1)) */
    if (e < -14)
        e = -14;                      /* subnormal range shares the quantum of 2^-14 */
    double quantum = ldexp(1.0, e - 10);
    double n = a / quantum;           /* exact: a has 24 significant bits */
    double fl = floor(n);
    double r = n - fl;
    if (r > 0.5 || (r == 0.5 && fmod(fl, 2.0) != 0.0))
        fl += 1.0;
    long ni = (long)fl;
    if (ni == 2048) {                 /* rounded up into the next binade */
        ni = 1024;
        e += 1;
    }
    if (e > 15)
        return sign | 0x7c00;
    if (ni < 1024)                    /* subnormal (only possible at e == -14) */
        return sign | (uint16_t)ni;
    return sign | (uint16_t)(((e + 15) << 10) | (ni - 1024));
}

float or_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* ---------------------------------------------------------------------------
 * Sizes.  Tile sizes from "Block-32 Quantized Formats": Q4_0 576 B, Q8_0
 * 1088 B, IQ4_NL 576 B.  Flat block sizes follow the GGML block-32 layouts
 * (2-byte fp16 scale + 16 bytes of nibbles, or + 32 int8 quants).
 * ------------------------------------------------------------------------- */
long or_tile_bytes(int type)
{
    switch (type) {
    case OR_Q4_0: return 576;
    case OR_Q8_0: return 1088;
    case OR_IQ4_NL: return 576;
    case OR_MXFP4: return 544;
    case OR_Q4_1: return 640;
    case OR_Q4_K: return 640;
    }
    return 0;
}

long or_block_bytes(int type)
{
    switch (type) {
    case OR_Q4_0: return 18;
    case OR_Q8_0: return 34;
    case OR_IQ4_NL: return 18;
    case OR_MXFP4: return 17;
    case OR_Q4_1: return 20;
    case OR_Q4_K: return 144;   /* one 256-element super-block */
    }
    return 0;
}

/* Elements of one flat block: 256 for the K-quant Q4_K, 32 for the others. */
long or_block_elems(int type) { return type == OR_Q4_K ? 256 : 32; }

/* Scale values per row and 32-element block in a tile: Q4_1 and Q4_K keep a
 * pair, the others one. */
long or_scale_count(int type) { return (type == OR_Q4_1 || type == OR_Q4_K) ? 2 : 1; }

/* "Tile Dimensions and Grid Layout": n_k_tiles = ne0 / 32, n_col_tiles =
 * (ne1 + 31) / 32, with ne0 = K and ne1 = N. */
long or_tiled_bytes(int type, long K, long N)
{
    return (K / 32) * ((N + 31) / 32) * or_tile_bytes(type);
}

long or_flat_bytes(int type, long K, long N)
{
    return N * (K / or_block_elems(type)) * or_block_bytes(type);
}

/* ---------------------------------------------------------------------------
 * Flat row-major GGML block-32 layout (the repack source).  The page says only
 * that weights are repacked "from flat row-major GGML layouts"; the reading
 * taken is GGML's own block-32 layout: row n holds K/32 consecutive blocks;
 * a Q4_0 / IQ4_NL block is an fp16 scale followed by 16 bytes whose low
 * nibbles are elements 0..15 and high nibbles elements 16..31; a Q8_0 block is
 * an fp16 scale followed by 32 int8 elements; an MXFP4 block is one E8M0
 * scale byte followed by 16 bytes with the Q4_0 nibble order; a Q4_1 block is
 * the fp16 scale d, the fp16 min m, then 16 bytes with the Q4_0 nibble order.
 *
 * codes[n*K + k] receives the raw code of element k of row n: 0..15 for the
 * 4-bit types, the int8 byte (as uint8) for Q8_0.  scales[(n*(K/32) + b)*ns
 * + i], ns = or_scale_count(type), receives scale value i of block b of row
 * n: the fp16 bits (MXFP4: the E8M0 byte; Q4_1: i = 0 is d, i = 1 is m).
 * ------------------------------------------------------------------------- */
static long quant_offset(int type)
{
    return type == OR_MXFP4 ? 1 : (type == OR_Q4_1 ? 4 : 2);
}

static uint16_t block_scale(int type, const uint8_t *blk, int i)
{
    if (type == OR_MXFP4)
        return blk[0];
    return (uint16_t)(blk[2 * i] | (blk[2 * i + 1] << 8));
}

/* ---------------------------------------------------------------------------
 * Q4_K flat super-blocks ("K-Quants": GGML packs 256 elements per super-block;
 * the page splits each into 8 tiles of 32 k whose row pairs are (d * sc,
 * -dmin * m)).  The page does not print the flat super-block; the reading
 * taken is GGML's: fp16 d, fp16 dmin, 12 bytes holding eight 6-bit scales sc
 * and eight 6-bit mins m, then 128 bytes of nibbles in which 64-element
 * chunk c owns bytes 32c..32c+31, element 64c + i (i < 32) in the low nibble
 * of byte 32c + i and element 64c + 32 + i in its high nibble.
 *
 * The 6-bit values of sub-block j: for j < 4, sc = low 6 bits of byte j and
 * m = low 6 bits of byte j + 4; for j >= 4 the low 4 bits come from byte
 * j + 4 (sc in its low nibble, m in its high one) and the top 2 bits from
 * the top 2 bits of byte j - 4 (sc) and byte j (m).
 * ------------------------------------------------------------------------- */
static void q4k_scale_min(const uint8_t *sb, int j, int *sc, int *m)
{
    if (j < 4) {
        *sc = sb[j] & 63;
        *m = sb[j + 4] & 63;
    } else {
        *sc = (sb[j + 4] & 0x0f) | ((sb[j - 4] >> 6) << 4);
        *m = (sb[j + 4] >> 4) | ((sb[j] >> 6) << 4);
    }
}

static const uint8_t *q4k_block(const uint8_t *flat, long K, long n, long k)
{
    return flat + (n * (K / 256) + k / 256) * 144;
}

static uint8_t q4k_code(const uint8_t *flat, long K, long n, long k)
{
    const uint8_t *qs = q4k_block(flat, K, n, k) + 16;
    int e = (int)(k % 256), c = e / 64, i = e % 64;
    uint8_t byte = qs[32 * c + (i % 32)];
    return i < 32 ? (byte & 0x0f) : (byte >> 4);
}

/* The tile pair of 32-element block kt of row n: i = 0 gives d * sc, i = 1
 * gives -(dmin * m), each product formed in fp32 (exact: an fp16 times a
 * 6-bit integer) and rounded to fp16 nearest-even (the tile holds FP16). */
static uint16_t q4k_pair(const uint8_t *flat, long K, long n, long kt, int i)
{
    const uint8_t *blk = q4k_block(flat, K, n, 32 * kt);
    int sc, m;
    q4k_scale_min(blk + 4, (int)(kt % 8), &sc, &m);
    float d = or_f16_to_f32((uint16_t)(blk[0] | (blk[1] << 8)));
    float dmin = or_f16_to_f32((uint16_t)(blk[2] | (blk[3] << 8)));
    return i == 0 ? or_f32_to_f16(d * (float)sc) : or_f32_to_f16(-(dmin * (float)m));
}

void or_flat_decode(int type, const uint8_t *flat, long K, long N,
                    uint8_t *codes, uint16_t *scales)
{
    if (type == OR_Q4_K) {
        long nb = K / 32;
        for (long n = 0; n < N; n++) {
            for (long k = 0; k < K; k++)
                codes[n * K + k] = q4k_code(flat, K, n, k);
            for (long b = 0; b < nb; b++)
                for (int i = 0; i < 2; i++)
                    scales[(n * nb + b) * 2 + i] = q4k_pair(flat, K, n, b, i);
        }
        return;
    }
    long nb = K / 32, bb = or_block_bytes(type), ns = or_scale_count(type);
    for (long n = 0; n < N; n++) {
        for (long b = 0; b < nb; b++) {
            const uint8_t *blk = flat + (n * nb + b) * bb;
            const uint8_t *qs = blk + quant_offset(type);
            for (int i = 0; i < ns; i++)
                scales[(n * nb + b) * ns + i] = block_scale(type, blk, i);
            for (int j = 0; j < 32; j++) {
                uint8_t c;
                if (type == OR_Q8_0)
                    c = qs[j];
                else if (j < 16)
                    c = qs[j] & 0x0f;
                else
                    c = qs[j - 16] >> 4;
                codes[n * K + b * 32 + j] = c;
            }
        }
    }
}

/* ---------------------------------------------------------------------------
 * Repack into tiles ("Tile Dimensions and Grid Layout" and "Block-32
 * Quantized Formats").  The tile of row-tile ct and column-tile kt sits at
 * byte (ct * n_k_tiles + kt) * tile_size.  Inside it, quant[row][col] is the
 * code of output row n = 32*ct + row and K index 32*kt + col.
 *
 *   Q4_0, IQ4_NL: 16 column pairs cp; for each, 32 consecutive bytes, one per
 *     row, holding column 2cp in the low nibble and 2cp+1 in the high nibble.
 *     Bytes 512..575: the 32 row scales (fp16).
 *   Q8_0: 16 column pairs; for each, 64 bytes holding, per row, the int8 of
 *     column 2cp then that of column 2cp+1.  Bytes 1024..1087: row scales.
 *
 * Reading for the ragged last row-tile (the page only gives the (ne1+31)/32
 * rounding): rows n >= N hold zero codes and a +0.0 scale, so they contribute
 * exactly nothing.
 * ------------------------------------------------------------------------- */
static uint8_t code_at(int type, const uint8_t *flat, long K, long n, long k)
{
    if (type == OR_Q4_K)
        return q4k_code(flat, K, n, k);
    long nb = K / 32, bb = or_block_bytes(type);
    const uint8_t *qs = flat + (n * nb + k / 32) * bb + quant_offset(type);
    int j = (int)(k % 32);
    if (type == OR_Q8_0)
        return qs[j];
    return j < 16 ? (qs[j] & 0x0f) : (qs[j - 16] >> 4);
}

static uint16_t scale_at(int type, const uint8_t *flat, long K, long n, long kt, int i)
{
    if (type == OR_Q4_K)
        return q4k_pair(flat, K, n, kt, i);
    long nb = K / 32, bb = or_block_bytes(type);
    return block_scale(type, flat + (n * nb + kt) * bb, i);
}

/* Tile scale bytes: 32 fp16 at 512 (Q4_0, IQ4_NL) or 1024 (Q8_0); MXFP4: 32
 * single E8M0 bytes at 512 ("MXFP4": bytes 512..543); Q4_1: 32 fp16 pairs at
 * 512, d of row r at 512 + 4r and m at 512 + 4r + 2 ("Q4_1": scale[2*row] =
 * d, scale[2*row + 1] = m). */
static long scale_byte(int type, int row, int i)
{
    switch (type) {
    case OR_MXFP4: return 512 + row;
    case OR_Q4_1:
    case OR_Q4_K: return 512 + 4 * row + 2 * i;
    case OR_Q8_0: return 1024 + 2 * row;
    }
    return 512 + 2 * row;
}

static void put_tile_scale(int type, uint8_t *tile, int row, int i, uint16_t s)
{
    long o = scale_byte(type, row, i);
    tile[o] = (uint8_t)(s & 0xff);
    if (type != OR_MXFP4)
        tile[o + 1] = (uint8_t)(s >> 8);
}

static uint16_t get_tile_scale(int type, const uint8_t *tile, int row, int i)
{
    long o = scale_byte(type, row, i);
    if (type == OR_MXFP4)
        return tile[o];
    return (uint16_t)(tile[o] | (tile[o + 1] << 8));
}

void or_repack(int type, const uint8_t *flat, long K, long N, uint8_t *tiles)
{
    long n_k_tiles = K / 32;
    long n_col_tiles = (N + 31) / 32;
    long ts = or_tile_bytes(type);
    for (long ct = 0; ct < n_col_tiles; ct++) {
        for (long kt = 0; kt < n_k_tiles; kt++) {
            uint8_t *tile = tiles + (ct * n_k_tiles + kt) * ts;
            for (int row = 0; row < 32; row++) {
                long n = 32 * ct + row;
                int valid = n < N;
                for (int cp = 0; cp < 16; cp++) {
                    uint8_t c0 = valid ? code_at(type, flat, K, n, 32 * kt + 2 * cp) : 0;
                    uint8_t c1 = valid ? code_at(type, flat, K, n, 32 * kt + 2 * cp + 1) : 0;
                    if (type == OR_Q8_0) {
                        tile[cp * 64 + 2 * row + 0] = c0;
                        tile[cp * 64 + 2 * row + 1] = c1;
                    } else {
                        tile[cp * 32 + row] = (uint8_t)((c1 << 4) | c0);
                    }
                }
                for (int i = 0; i < or_scale_count(type); i++)
                    put_tile_scale(type, tile, row, i, valid ? scale_at(type, flat, K, n, kt, i) : 0);
            }
        }
    }
}

/* Inverse of or_repack for rows n < N: codes[n*K + k], scales[(n*(K/32) +
 * kt)*ns + i] as or_flat_decode. */
void or_unpack(int type, const uint8_t *tiles, long K, long N,
               uint8_t *codes, uint16_t *scales)
{
    long n_k_tiles = K / 32;
    long ts = or_tile_bytes(type);
    for (long n = 0; n < N; n++) {
        long ct = n / 32;
        int row = (int)(n % 32);
        for (long kt = 0; kt < n_k_tiles; kt++) {
            const uint8_t *tile = tiles + (ct * n_k_tiles + kt) * ts;
            for (int col = 0; col < 32; col++) {
                int cp = col / 2;
                uint8_t c;
                if (type == OR_Q8_0)
                    c = tile[cp * 64 + 2 * row + (col & 1)];
                else
                    c = (col & 1) ? (tile[cp * 32 + row] >> 4) : (tile[cp * 32 + row] & 0x0f);
                codes[n * K + kt * 32 + col] = c;
            }
            for (int i = 0; i < or_scale_count(type); i++)
                scales[(n * n_k_tiles + kt) * or_scale_count(type) + i] =
                    get_tile_scale(type, tile, row, i);
        }
    }
}

/* ---------------------------------------------------------------------------
 * Integer weight value of a code.  Q8_0: the int8 itself.  Q4_0: the page
 * gives only "4-bit quants" and a row scale; the reading taken is GGML's
 * zero point of 8, value = d * (code - 8), consistent with the page's own
 * half-range offsets for Q2_0 ("codes 0..3 representing signed values -1..2")
 * and Q3_K ("low2 - 4").  IQ4_NL: the code indexes a 16-entry non-linear
 * table (the page names it but does not print it); here the table is an
 * int8[16] supplied by the caller.  MXFP4 ("MXFP4": 4-bit OCP Microscaling
 * FP4, E2M1): the code is sign (bit 3), exponent (bits 2..1, bias 1) and
 * mantissa (bit 0); its value is +-0.5*m for exponent 0 and
 * +-2^(e-1) * (1 + m/2) otherwise.  The integer weight is twice that value
 * (0, 1, 2, 3, 4, 6, 8, 12 with sign), the factor 1/2 going to the scale.
 * Q4_1 ("Q4_1": a scale d and a min m per row): the integer weight is the
 * code itself, 0..15, and the weight value d * code + m (GGML's Q4_1); the
 * block dot is that of the codes, the min enters only the matmul.  Q4_K
 * tiles are Q4_1 tiles ("K-Quants": same layout as the Q4_1 tile) whose pair
 * is (d * sc, -dmin * m), so the same holds with those two values.
 * ------------------------------------------------------------------------- */
static int e2m1_twice(uint8_t code)
{
    int sign = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    int v = (e == 0) ? m : (1 << (e - 1)) * (2 + m);
    return sign ? -v : v;
}

static int weight_value(int type, uint8_t code, const int8_t *lut)
{
    switch (type) {
    case OR_Q4_0: return (int)code - 8;
    case OR_Q8_0: return (int)(int8_t)code;
    case OR_IQ4_NL: return (int)lut[code & 0x0f];
    case OR_MXFP4: return e2m1_twice(code & 0x0f);
    case OR_Q4_1:
    case OR_Q4_K: return (int)code;
    }
    return 0;
}

/* The row scale that multiplies the integer weight.  fp16 types: the fp16
 * value.  MXFP4 ("MXFP4", Dequantization): the E8M0 byte e becomes the FP16
 * power of two with exponent bits clamp(e - 112, 0, 30), i.e. 2^(e-127) for
 * 113 <= e <= 142, 0 for e <= 112 and 2^15 for e >= 142; halved here because
 * the integer weight is twice the FP4 value. */
double or_row_scale(int type, uint16_t s)
{
    if (type != OR_MXFP4)
        return (double)or_f16_to_f32(s);
    int ex = (int)s - 112;
    if (ex < 0)
        ex = 0;
    if (ex > 30)
        ex = 30;
    return 0.5 * (double)or_f16_to_f32((uint16_t)(ex << 10));
}

/* ---------------------------------------------------------------------------
 * Dynamic activation quantization ("Memory buffers": activations are
 * dynamically quantized; "Q2_0 Format › HVX Vector Dot-Product": the dot runs
 * against Q8_0 activation tiles).  Reading: Q8_0 per 32-element K block --
 *   amax = max |x_j|;  d = amax / 127 (fp32);  id = d != 0 ? 1/d : 0 (fp32);
 *   q_j  = round-half-away-from-zero(x_j * id) (fp32 product);
 *   the stored scale is d rounded to fp16 (nearest-even).
 * q is planar row-major q[m*K + k]; d[m*(K/32) + kt].  Inputs are read at row
 * stride ldx elements, as fp32, bf16 or fp16 (each converted exactly).
 * Returns 0, or -1 if some |q| > 127 (cannot happen for finite input).
 * ------------------------------------------------------------------------- */
static float load_act(int dtype, const void *x, long idx)
{
    switch (dtype) {
    case OR_F32: return ((const float *)x)[idx];
    case OR_BF16: return or_bf16_to_f32(((const uint16_t *)x)[idx]);
    case OR_F16: return or_f16_to_f32(((const uint16_t *)x)[idx]);
    }
    return 0.0f;
}

int or_quantize_act(int dtype, const void *x, long M, long K, long ldx,
                    int8_t *q, uint16_t *d)
{
    long nb = K / 32;
    for (long m = 0; m < M; m++) {
        for (long kt = 0; kt < nb; kt++) {
            float amax = 0.0f;
            for (int j = 0; j < 32; j++) {
                float v = fabsf(load_act(dtype, x, m * ldx + kt * 32 + j));
                if (v > amax)
                    amax = v;
            }
            float dv = amax / 127.0f;
            float id = (dv != 0.0f) ? 1.0f / dv : 0.0f;
            for (int j = 0; j < 32; j++) {
                float prod = load_act(dtype, x, m * ldx + kt * 32 + j) * id;
                float r = roundf(prod);
                if (r > 127.0f || r < -127.0f)
                    return -1;
                q[m * K + kt * 32 + j] = (int8_t)r;
            }
            d[m * nb + kt] = or_f32_to_f16(dv);
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Per-block integer dot products: isum[(m*N + n)*(K/32) + kt] =
 *   sum_{j<32} w[n][32kt+j] * q[m][32kt+j], exact in int64, checked to fit
 * int32 (returns -1 otherwise).  Weights are read back out of the tiles.
 * ------------------------------------------------------------------------- */
int or_block_dots(int type, const uint8_t *tiles, long K, long N,
                  const int8_t *q, long M, const int8_t *lut, int32_t *isum)
{
    long nb = K / 32;
    uint8_t *codes = malloc((size_t)(K > 0 ? K : 1));
    for (long n = 0; n < N; n++) {
        /* unpack one row at a time through the tile layout */
        long ct = n / 32;
        int row = (int)(n % 32);
        long ts = or_tile_bytes(type);
        for (long kt = 0; kt < nb; kt++) {
            const uint8_t *tile = tiles + (ct * nb + kt) * ts;
            for (int col = 0; col < 32; col++) {
                int cp = col / 2;
                codes[kt * 32 + col] = (type == OR_Q8_0)
                    ? tile[cp * 64 + 2 * row + (col & 1)]
                    : ((col & 1) ? (tile[cp * 32 + row] >> 4) : (tile[cp * 32 + row] & 0x0f));
            }
        }
        for (long m = 0; m < M; m++) {
            for (long kt = 0; kt < nb; kt++) {
                int64_t s = 0;
                for (int j = 0; j < 32; j++)
                    s += (int64_t)weight_value(type, codes[kt * 32 + j], lut) *
                         (int64_t)q[m * K + kt * 32 + j];
                if (s > INT32_MAX || s < INT32_MIN) {
                    free(codes);
                    return -1;
                }
                isum[(m * N + n) * nb + kt] = (int32_t)s;
            }
        }
    }
    free(codes);
    return 0;
}

/* ---------------------------------------------------------------------------
 * The product itself, from its plain definition:
 *   y[m][n] = sum_k W[n][k] * A[m][k],   W[n][k] = dw[n][kt] * w[n][k],
 *                                        A[m][k] = da[m][kt] * q[m][k],
 * i.e. GGML's dst = src0^T * src1 with ne0 = K and ne1 = N, each row scale
 * applied to its 32-element block ("multiplied by the row scale d").
 * Dequantize-then-dot in fp64, straight from the tiles, for output rows
 * n0 <= n < n1 and every m; y[m*ldy + n].  acond[m*ldy + n] (if not NULL)
 * receives sum_k |W*A|, the scale of the rounding error any fp32 summation of
 * the same terms can make.
 * ------------------------------------------------------------------------- */
void or_matmul(int type, const uint8_t *tiles, long K, long N,
               const int8_t *q, const uint16_t *d, long M, const int8_t *lut,
               long n0, long n1, double *y, double *acond, long ldy)
{
    long nb = K / 32;
    long ts = or_tile_bytes(type);
    if (n1 > N)
        n1 = N;
    double *wrow = malloc((size_t)(K > 0 ? K : 1) * sizeof(double));
    for (long n = n0; n < n1; n++) {
        long ct = n / 32;
        int row = (int)(n % 32);
        for (long kt = 0; kt < nb; kt++) {
            const uint8_t *tile = tiles + (ct * nb + kt) * ts;
            double dw = or_row_scale(type, get_tile_scale(type, tile, row, 0));
            /* Q4_1: w = d * code + m (GGML's Q4_1; "Q4_1" names the pair d,
             * the scale, and m, the min) */
            double mw = (type == OR_Q4_1 || type == OR_Q4_K)
                ? (double)or_f16_to_f32(get_tile_scale(type, tile, row, 1)) : 0.0;
            for (int col = 0; col < 32; col++) {
                int cp = col / 2;
                uint8_t c = (type == OR_Q8_0)
                    ? tile[cp * 64 + 2 * row + (col & 1)]
                    : ((col & 1) ? (tile[cp * 32 + row] >> 4) : (tile[cp * 32 + row] & 0x0f));
                wrow[kt * 32 + col] = dw * (double)weight_value(type, c, lut) + mw;
            }
        }
        for (long m = 0; m < M; m++) {
            double s = 0.0, a = 0.0;
            for (long k = 0; k < K; k++) {
                double act = (double)or_f16_to_f32(d[m * nb + k / 32]) * (double)q[m * K + k];
                double t = wrow[k] * act;
                s += t;
                a += fabs(t);
            }
            y[m * ldy + n] = s;
            if (acond)
                acond[m * ldy + n] = a;
        }
    }
    free(wrow);
}

/* ---------------------------------------------------------------------------
 * The same products over flat GGML blocks ("supports_op Independence from
 * Buffer and Repack State": a supported type must work tiled and flat, the
 * flat form being what test harnesses and non-weight tensors use).  Weights
 * are read from the flat blocks directly (code_at, scale_at), with the
 * values a tile of the same data holds; so the results equal those of
 * or_block_dots / or_matmul on or_repack's tiles.
 * ------------------------------------------------------------------------- */
static double flat_weight(int type, const uint8_t *flat, long K, long n, long k,
                          const int8_t *lut)
{
    long kt = k / 32;
    uint8_t c = code_at(type, flat, K, n, k);
    double dw = or_row_scale(type, scale_at(type, flat, K, n, kt, 0));
    double mw = (type == OR_Q4_1 || type == OR_Q4_K)
        ? (double)or_f16_to_f32(scale_at(type, flat, K, n, kt, 1)) : 0.0;
    return dw * (double)weight_value(type, c, lut) + mw;
}

int or_block_dots_flat(int type, const uint8_t *flat, long K, long N,
                       const int8_t *q, long M, const int8_t *lut, int32_t *isum)
{
    long nb = K / 32;
    for (long n = 0; n < N; n++)
        for (long m = 0; m < M; m++)
            for (long kt = 0; kt < nb; kt++) {
                int64_t s = 0;
                for (int j = 0; j < 32; j++)
                    s += (int64_t)weight_value(type, code_at(type, flat, K, n, 32 * kt + j), lut) *
                         (int64_t)q[m * K + kt * 32 + j];
                if (s > INT32_MAX || s < INT32_MIN)
                    return -1;
                isum[(m * N + n) * nb + kt] = (int32_t)s;
            }
    return 0;
}

void or_matmul_flat(int type, const uint8_t *flat, long K, long N,
                    const int8_t *q, const uint16_t *d, long M, const int8_t *lut,
                    long n0, long n1, double *y, double *acond, long ldy)
{
    long nb = K / 32;
    if (n1 > N)
        n1 = N;
    double *wrow = malloc((size_t)(K > 0 ? K : 1) * sizeof(double));
    for (long n = n0; n < n1; n++) {
        for (long k = 0; k < K; k++)
            wrow[k] = flat_weight(type, flat, K, n, k, lut);
        for (long m = 0; m < M; m++) {
            double s = 0.0, a = 0.0;
            for (long k = 0; k < K; k++) {
                double act = (double)or_f16_to_f32(d[m * nb + k / 32]) * (double)q[m * K + k];
                double t = wrow[k] * act;
                s += t;
                a += fabs(t);
            }
            y[m * ldy + n] = s;
            if (acond)
                acond[m * ldy + n] = a;
        }
    }
    free(wrow);
}


/* ---------------------------------------------------------------------------
 * MXFP8 activations for MXFP4 weights (OCP Microscaling Formats v1.0: a block
 * of 32 elements shares one E8M0 scale X = 2^(e - 127); the elements are
 * FP8 E4M3 codes).  The page's MXFP4 tiles carry exactly such per-32 E8M0
 * scales ("MXFP4"); this is the activation side that pairs with them on
 * matrix hardware that applies per-32 power-of-two scales itself.  Reading
 * (the page quantizes activations to Q8_0 and says nothing of MX
 * activations), following the OCP conversion:
 *   amax = max_j |x_j| (inputs converted exactly to fp32);
 *   X    = 2^(floor(log2 amax) - 8)   (8 = the largest E4M3 exponent),
 *          the biased exponent clamped to 0..254; amax = 0 gives e = 0;
 *   P_j  = the E4M3 value nearest to x_j / X, ties to the even code,
 *          magnitudes above 448 (the largest finite E4M3) saturating to 448;
 *          the code's sign bit is the sign bit of x_j.
 * E4M3 (OCP FP8): sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent
 * field 0 is subnormal (m/8 * 2^-6); codes 0x7F and 0xFF are NaN and never
 * produced.
 * ------------------------------------------------------------------------- */
double or_e4m3_value(uint8_t code)
{
    int e = (code >> 3) & 0x0f, m = code & 7;
    double v = (e == 0) ? ldexp((double)m, -9) : ldexp(8.0 + m, e - 10);
    return (code & 0x80) ? -v : v;
}

/* Nearest non-negative E4M3 code (0..0x7E) to v >= 0, ties to the even
 * code: a walk over the 127 finite values in increasing order. */
static int e4m3_nearest(double v)
{
    int best = 0;
    double bd = fabs(v);
    for (int c = 1; c <= 0x7e; c++) {
        double dist = fabs(v - or_e4m3_value((uint8_t)c));
        if (dist < bd || (dist == bd && (c & 1) == 0 && (best & 1) != 0)) {
            best = c;
            bd = dist;
        }
    }
    return best;
}

void or_quantize_act_mx(int dtype, const void *x, long M, long K, long ldx,
                        uint8_t *q, uint8_t *e)
{
    long nb = K / 32;
    for (long m = 0; m < M; m++) {
        for (long kt = 0; kt < nb; kt++) {
            double amax = 0.0;
            for (int j = 0; j < 32; j++) {
                double v = fabs((double)load_act(dtype, x, m * ldx + kt * 32 + j));
                if (v > amax)
                    amax = v;
            }
            int eb = 0;
            if (amax > 0.0) {
                int ex;
                frexp(amax, &ex);           /* amax = f * 2^ex, 0.5 <= f < 1 */
                eb = (ex - 1) - 8 + 127;    /* floor(log2 amax) - 8, biased */
                if (eb < 0)
                    eb = 0;
                if (eb > 254)
                    eb = 254;
            }
            e[m * nb + kt] = (uint8_t)eb;
            for (int j = 0; j < 32; j++) {
                float xv = load_act(dtype, x, m * ldx + kt * 32 + j);
                double r = ldexp(fabs((double)xv), 127 - eb);   /* |x| / X, exact */
                int c = (r >= 448.0) ? 0x7e : e4m3_nearest(r);
                q[m * K + kt * 32 + j] = (uint8_t)(c | (signbit(xv) ? 0x80 : 0));
            }
        }
    }
}

/* The MXFP4 x MXFP8 product from its plain definition:
 *   y[m][n] = sum_k W[n][k] * A[m][k],
 *   W[n][k] = s(e_w[n][kt]) * E2M1(code)  -- the page's MXFP4 dequantization,
 *             s(e) = the FP16 power of two with exponent bits clamp(e-112, 0, 30);
 *   A[m][k] = 2^(e_a[m][kt] - 127) * E4M3(q[m][k]).
 * fp64, output rows n0 <= n < n1; acond as in or_matmul. */
void or_matmul_mx(const uint8_t *tiles, long K, long N, const uint8_t *q, const uint8_t *e,
                  long M, long n0, long n1, double *y, double *acond, long ldy)
{
    long nb = K / 32;
    long ts = or_tile_bytes(OR_MXFP4);
    if (n1 > N)
        n1 = N;
    double *wrow = malloc((size_t)(K > 0 ? K : 1) * sizeof(double));
    for (long n = n0; n < n1; n++) {
        long ct = n / 32;
        int row = (int)(n % 32);
        for (long kt = 0; kt < nb; kt++) {
            const uint8_t *tile = tiles + (ct * nb + kt) * ts;
            /* or_row_scale halves the power of two for the doubled integer
             * weight; the E2M1 value is half that integer: together s * E2M1 */
            double dw = or_row_scale(OR_MXFP4, get_tile_scale(OR_MXFP4, tile, row, 0));
            for (int col = 0; col < 32; col++) {
                int cp = col / 2;
                uint8_t c = (col & 1) ? (tile[cp * 32 + row] >> 4) : (tile[cp * 32 + row] & 0x0f);
                wrow[kt * 32 + col] = dw * (double)e2m1_twice(c);
            }
        }
        for (long m = 0; m < M; m++) {
            double s = 0.0, a = 0.0;
            for (long k = 0; k < K; k++) {
                double act = ldexp(or_e4m3_value(q[m * K + k]), (int)e[m * nb + k / 32] - 127);
                double t = wrow[k] * act;
                s += t;
                a += fabs(t);
            }
            y[m * ldy + n] = s;
            if (acond)
                acond[m * ldy + n] = a;
        }
    }
    free(wrow);
}
