/*
 * oracle.c -- the plain CPU oracle of the quantized linear layer y = x.W^T.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the bench's
 * cpu_baseline leg do.  It shares no code, header, table or constant with the
 * HIP library: it decodes every byte format itself and carries its own IEEE
 * binary16 conversion.
 *
 * Every routine is the plain definition written out: integer block sums are
 * exact int32 sums, float scaling and accumulation are done in f64, the
 * quantizers use IEEE f32 arithmetic exactly as the definitions read.  Loops
 * run in the order of the definition; output elements are independent and are
 * spread over OpenMP threads only across whole outputs, so a run on P threads
 * is bit-identical to a run on one ("Chapter 06 -- Going fast on CPUs", 6.7:
 * disjoint output ranges computed by the same serial loop give the same bits).
 *
 * Sources (web pages, cited by title and section):
 *  [CPU]   llama.cpp visual guide, lesson 31 "CPU backend", section "How the
 *          quantized dot product works": block_q4_0 = fp16 d + 16 bytes of
 *          nibbles, unpack 16 bytes -> 32 values in [0,15] (low 4 bits, then
 *          the high 4), subtract 8, int8 dot against the Q8_0 block, multiply
 *          by the product of the two blocks' fp16 scales, accumulate.
 *  [FAST]  Fucina course "Chapter 06 -- Going fast on CPUs", 6.1 (GEMM
 *          naming: A m x k, B k x n, C m x n) and 6.4 "The scalar backend is
 *          the specification" (the triple-loop referee; a naive f64 reference
 *          referees the blocked kernel).
 *  [LOOM]  Loom "Plan 9 SIMD Forward", section "BitNet ternary MAD kernel":
 *          ternary weights packed 16 per uint32, code = w + 1, the identity
 *          dot = sum(code*act) - sum(act), per-row int8 activations with
 *          activation_scale = 127 / max|x|, output dot * absmean / act_scale.
 *  [BACK]  Fucina reference "Backends", 9.7 "Quantized matmul dispatch":
 *          the f32 activation rows are quantized to Q8_0 blocks per call;
 *          weights may themselves be quantized to Q8_0 (the Q8_0 x Q8_0
 *          block dot).
 *
 * Readings where the pages are silent (the same list is kept with the
 * design notes): element t < 16 of a Q4_0 block is the low nibble of qs[t],
 * element t >= 16 the high nibble of qs[t-16]; block_q8_0 = {fp16 d, int8
 * qs[32]} (34 bytes); the Q8_0 quantizer is d = amax/127 in f32, q =
 * round-half-away(x/d) with f32 division, clamped to +-127, fp16(d) stored
 * round-to-nearest-even, and a block whose f32 d is 0 gets q = 0; ternary code
 * s of a word sits at bits 2s..2s+1 (LSB first); ternary activations are
 * q = round-half-away(x*s) with s = 127/amax in f32, clamped to +-127, and a
 * row with amax = 0 or with s not finite is all-zero with act_scale = 0.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_ERR_ARG -1
#define ORC_ERR_CODE -2     /* a ternary code equal to 3 */
#define ORC_ERR_IDENTITY -3 /* the ternary identity failed (cannot happen) */

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary16.                                                        */
/* ------------------------------------------------------------------------ */

/* binary16 bits -> exact double value. */
double orc_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24); /* subnormal: f * 2^-24 */
    else if (e == 31)
        v = (f == 0) ? INFINITY : NAN;
    else
        v = ldexp((double)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* Round a non-negative double to an integer, ties to even. */
static double round_half_even(double v)
{
    double r = floor(v);
    double diff = v - r;
    if (diff > 0.5)
        return r + 1.0;
    if (diff < 0.5)
        return r;
    return (fmod(r, 2.0) == 0.0) ? r : r + 1.0;
}

/* float -> binary16 bits, round to nearest even (the IEEE default). */
uint16_t orc_float_to_half(float x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs((double)x);
    if (isnan(x))
        return (uint16_t)(sign | 0x7e00);
    /* 65504 is the largest finite half; 65520 is half-way to 2^16 and the
     * tie goes to the even neighbour, which is the overflow to infinity. */
    if (a >= 65520.0)
        return (uint16_t)(sign | 0x7c00);
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: the value is an integer multiple of 2^-24 */
        double q = round_half_even(a * ldexp(1.0, 24));
        return (uint16_t)(sign | (uint16_t)q); /* q == 1024 is the min normal */
    }
    int E;
    frexp(a, &E);       /* a = m * 2^E, m in [0.5, 1) */
    int e = E - 1;      /* a in [2^e, 2^(e+1)) */
    double mant = round_half_even(a * ldexp(1.0, 10 - e)); /* in [1024, 2048] */
    if (mant == 2048.0) {
        mant = 1024.0;
        e += 1;
    }
    if (e + 15 >= 31)
        return (uint16_t)(sign | 0x7c00);
    return (uint16_t)(sign | ((uint16_t)(e + 15) << 10) | (uint16_t)(mant - 1024.0));
}

void orc_half_to_double_array(const uint16_t *h, double *out, int64_t count)
{
    for (int64_t i = 0; i < count; i++)
        out[i] = orc_half_to_double(h[i]);
}

void orc_float_to_half_array(const float *x, uint16_t *out, int64_t count)
{
    for (int64_t i = 0; i < count; i++)
        out[i] = orc_float_to_half(x[i]);
}

static uint16_t load_u16le(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static void store_u16le(uint8_t *p, uint16_t v)
{
    p[0] = (uint8_t)(v & 0xff);
    p[1] = (uint8_t)(v >> 8);
}

/* ------------------------------------------------------------------------ */
/* Q4_0 weight blocks [CPU]: 18 bytes = u16 d (binary16) + u8 qs[16].       */
/* ------------------------------------------------------------------------ */

/* codes[n][k] (each 0..15), d_bits[n][k/32] -> w[n][k/32] blocks. */
int orc_pack_q4_0(const uint8_t *codes, const uint16_t *d_bits, uint8_t *w, int64_t n, int64_t k)
{
    if (k % 32 != 0 || n < 0 || k < 0)
        return ORC_ERR_ARG;
    int64_t nb = k / 32;
    for (int64_t j = 0; j < n; j++)
        for (int64_t b = 0; b < nb; b++) {
            uint8_t *blk = w + (j * nb + b) * 18;
            const uint8_t *c = codes + j * k + b * 32;
            store_u16le(blk, d_bits[j * nb + b]);
            for (int t = 0; t < 16; t++) {
                if (c[t] > 15 || c[t + 16] > 15)
                    return ORC_ERR_ARG;
                blk[2 + t] = (uint8_t)(c[t] | (c[t + 16] << 4));
            }
        }
    return ORC_OK;
}

/* w[n][k/32] blocks -> codes[n][k] (0..15), d_bits[n][k/32]. */
int orc_unpack_q4_0(const uint8_t *w, uint8_t *codes, uint16_t *d_bits, int64_t n, int64_t k)
{
    if (k % 32 != 0 || n < 0 || k < 0)
        return ORC_ERR_ARG;
    int64_t nb = k / 32;
    for (int64_t j = 0; j < n; j++)
        for (int64_t b = 0; b < nb; b++) {
            const uint8_t *blk = w + (j * nb + b) * 18;
            uint8_t *c = codes + j * k + b * 32;
            d_bits[j * nb + b] = load_u16le(blk);
            for (int t = 0; t < 16; t++) {
                c[t] = blk[2 + t] & 0x0f;
                c[t + 16] = blk[2 + t] >> 4;
            }
        }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Q8_0 activation blocks: 34 bytes = u16 d (binary16) + int8 qs[32].       */
/* ------------------------------------------------------------------------ */

/* x[m][k] f32 -> xq[m][k/32] Q8_0 blocks ([BACK] 9.7: per-call activation
 * quantization; the block scale is the block's max |x| over 127). */
int orc_quantize_q8_0(const float *x, uint8_t *xq, int64_t m, int64_t k)
{
    if (k % 32 != 0 || m < 0 || k < 0)
        return ORC_ERR_ARG;
    int64_t nb = k / 32;
    for (int64_t i = 0; i < m; i++)
        for (int64_t b = 0; b < nb; b++) {
            const float *xb = x + i * k + b * 32;
            uint8_t *blk = xq + (i * nb + b) * 34;
            float amax = 0.0f;
            for (int t = 0; t < 32; t++) {
                float a = fabsf(xb[t]);
                if (a > amax)
                    amax = a;
            }
            float d = amax / 127.0f; /* IEEE f32 division */
            store_u16le(blk, orc_float_to_half(d));
            for (int t = 0; t < 32; t++) {
                int q = 0;
                if (d != 0.0f) {
                    float r = roundf(xb[t] / d); /* half away from zero */
                    if (r > 127.0f)
                        r = 127.0f;
                    if (r < -127.0f)
                        r = -127.0f;
                    q = (int)r;
                }
                blk[2 + t] = (uint8_t)(int8_t)q;
            }
        }
    return ORC_OK;
}

/* xq[m][k/32] -> q[m][k] int8 and d_bits[m][k/32]. */
int orc_unpack_q8_0(const uint8_t *xq, int8_t *q, uint16_t *d_bits, int64_t m, int64_t k)
{
    if (k % 32 != 0 || m < 0 || k < 0)
        return ORC_ERR_ARG;
    int64_t nb = k / 32;
    for (int64_t i = 0; i < m; i++)
        for (int64_t b = 0; b < nb; b++) {
            const uint8_t *blk = xq + (i * nb + b) * 34;
            d_bits[i * nb + b] = load_u16le(blk);
            for (int t = 0; t < 32; t++)
                q[i * k + b * 32 + t] = (int8_t)blk[2 + t];
        }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Q4_0 x Q8_0 dot [CPU]: per block b                                       */
/*   sumi_b = sum_t (qw_t - 8) * qx_t            (int32, exact)             */
/*   term_b = f64(dw_b) * f64(dx_b) * sumi_b     (exact in f64)             */
/* y = sum_b term_b in b order (f64), mag = sum_b |term_b|.                  */
/* ------------------------------------------------------------------------ */

/* Elements t = 0..15 are the low nibbles of qs[t], t = 16..31 the high
 * nibbles of qs[t - 16]: the sum runs over t in order, in two loops. */
static int32_t q4_0_q8_0_block_sum(const uint8_t *wblk, const uint8_t *xblk)
{
    int32_t s = 0;
    for (int t = 0; t < 16; t++) {
        int qw = wblk[2 + t] & 0x0f;
        s += (qw - 8) * (int8_t)xblk[2 + t];
    }
    for (int t = 16; t < 32; t++) {
        int qw = wblk[2 + t - 16] >> 4;
        s += (qw - 8) * (int8_t)xblk[2 + t];
    }
    return s;
}

/* Every binary16 bit pattern decoded once by orc_half_to_double, so that a
 * large product does not decode the same scale bits again for each output
 * (the values are those of orc_half_to_double; NULL when out of memory). */
static double *half_table(void)
{
    double *t = malloc(sizeof(double) * 65536);
    if (t)
        for (int h = 0; h < 65536; h++)
            t[h] = orc_half_to_double((uint16_t)h);
    return t;
}

static void q4_0_q8_0_one(const uint8_t *wrow, const uint8_t *xrow, int64_t nb, const double *half, double *y,
                          double *mag)
{
    double acc = 0.0, m = 0.0;
    for (int64_t b = 0; b < nb; b++) {
        const uint8_t *wb = wrow + b * 18;
        const uint8_t *xb = xrow + b * 34;
        int32_t sumi = q4_0_q8_0_block_sum(wb, xb);
        double s = half[load_u16le(wb)] * half[load_u16le(xb)];
        double term = s * (double)sumi;
        acc += term;
        m += fabs(term);
    }
    *y = acc;
    *mag = m;
}

/* Y[m][n] = X.W^T with X = xq[m][k/32] (Q8_0) and W = w[n][k/32] (Q4_0). */
int orc_q4_0_q8_0(const uint8_t *w, const uint8_t *xq, int64_t m, int64_t n, int64_t k, double *y, double *mag)
{
    if (k % 32 != 0 || m < 0 || n < 0 || k < 0)
        return ORC_ERR_ARG;
    int64_t nb = k / 32;
    double *half = half_table();
    if (!half)
        return ORC_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; j++)
        for (int64_t i = 0; i < m; i++)
            q4_0_q8_0_one(w + j * nb * 18, xq + i * nb * 34, nb, half, &y[i * n + j], &mag[i * n + j]);
    free(half);
    return ORC_OK;
}

/* The same definition evaluated only at the listed (ii[s], jj[s]) outputs. */
int orc_q4_0_q8_0_sampled(const uint8_t *w, const uint8_t *xq, int64_t m, int64_t n, int64_t k,
                          const int64_t *ii, const int64_t *jj, int64_t count, double *y, double *mag)
{
    if (k % 32 != 0 || m < 0 || n < 0 || k < 0)
        return ORC_ERR_ARG;
    for (int64_t s = 0; s < count; s++)
        if (ii[s] < 0 || ii[s] >= m || jj[s] < 0 || jj[s] >= n)
            return ORC_ERR_ARG;
    int64_t nb = k / 32;
    double *half = half_table();
    if (!half)
        return ORC_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t s = 0; s < count; s++)
        q4_0_q8_0_one(w + jj[s] * nb * 18, xq + ii[s] * nb * 34, nb, half, &y[s], &mag[s]);
    free(half);
    return ORC_OK;
}

/* The integer block sums themselves: sumi[i][j][b] for every output. */
int orc_q4_0_q8_0_block_sums(const uint8_t *w, const uint8_t *xq, int64_t m, int64_t n, int64_t k, int32_t *sumi)
{
    if (k % 32 != 0 || m < 0 || n < 0 || k < 0)
        return ORC_ERR_ARG;
    int64_t nb = k / 32;
    for (int64_t i = 0; i < m; i++)
        for (int64_t j = 0; j < n; j++)
            for (int64_t b = 0; b < nb; b++)
                sumi[(i * n + j) * nb + b] = q4_0_q8_0_block_sum(w + (j * nb + b) * 18, xq + (i * nb + b) * 34);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Q8_0 weights x Q8_0 activations: the weights quantized to Q8_0 blocks    */
/* (the quantized right-hand side of [BACK] 9.7, quantizeMatmulRhsQ8_0; the  */
/* activations quantized per call as above).  Per block b                    */
/*   sumi_b = sum_t qw_t * qx_t                   (int32, exact)             */
/*   term_b = f64(dw_b) * f64(dx_b) * sumi_b      (exact in f64)             */
/* y = sum_b term_b in b order (f64), mag = sum_b |term_b|.                  */
/* ------------------------------------------------------------------------ */

/* q int8[n][k] and d_bits uint16[n][k/32] -> w[n][k/32] block_q8_0. */
int orc_pack_q8_0(const int8_t *q, const uint16_t *d_bits, uint8_t *w, int64_t n, int64_t k)
{
    if (k % 32 != 0 || n < 0 || k < 0)
        return ORC_ERR_ARG;
    int64_t nb = k / 32;
    for (int64_t j = 0; j < n; j++)
        for (int64_t b = 0; b < nb; b++) {
            uint8_t *out = w + (j * nb + b) * 34;
            store_u16le(out, d_bits[j * nb + b]);
            for (int t = 0; t < 32; t++)
                out[2 + t] = (uint8_t)q[j * k + b * 32 + t];
        }
    return ORC_OK;
}

static int32_t q8_0_q8_0_block_sum(const uint8_t *wblk, const uint8_t *xblk)
{
    int32_t s = 0;
    for (int t = 0; t < 32; t++) {
        int qw = (int8_t)wblk[2 + t];
        int qx = (int8_t)xblk[2 + t];
        s += qw * qx;
    }
    return s;
}

static void q8_0_q8_0_one(const uint8_t *wrow, const uint8_t *xrow, int64_t nb, double *y, double *mag)
{
    double sum = 0.0, sum_abs = 0.0;
    for (int64_t b = 0; b < nb; b++) {
        const uint8_t *wblk = wrow + b * 34;
        const uint8_t *xblk = xrow + b * 34;
        int32_t sumi = q8_0_q8_0_block_sum(wblk, xblk);
        double sc = orc_half_to_double(load_u16le(wblk)) * orc_half_to_double(load_u16le(xblk));
        double term = sc * (double)sumi;
        sum += term;
        sum_abs += fabs(term);
    }
    *y = sum;
    *mag = sum_abs;
}

/* Y[m][n] = X.W^T with X = xq[m][k/32] and W = w[n][k/32], both Q8_0. */
int orc_q8_0_q8_0(const uint8_t *w, const uint8_t *xq, int64_t m, int64_t n, int64_t k, double *y, double *mag)
{
    if (k % 32 != 0 || m < 0 || n < 0 || k < 0)
        return ORC_ERR_ARG;
    int64_t nb = k / 32;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; j++)
        for (int64_t i = 0; i < m; i++)
            q8_0_q8_0_one(w + j * nb * 34, xq + i * nb * 34, nb, &y[i * n + j], &mag[i * n + j]);
    return ORC_OK;
}

/* The same definition evaluated only at the listed (ii[s], jj[s]) outputs. */
int orc_q8_0_q8_0_sampled(const uint8_t *w, const uint8_t *xq, int64_t m, int64_t n, int64_t k,
                          const int64_t *ii, const int64_t *jj, int64_t count, double *y, double *mag)
{
    if (k % 32 != 0 || m < 0 || n < 0 || k < 0)
        return ORC_ERR_ARG;
    for (int64_t s = 0; s < count; s++)
        if (ii[s] < 0 || ii[s] >= m || jj[s] < 0 || jj[s] >= n)
            return ORC_ERR_ARG;
    int64_t nb = k / 32;
#pragma omp parallel for schedule(static)
    for (int64_t s = 0; s < count; s++)
        q8_0_q8_0_one(w + jj[s] * nb * 34, xq + ii[s] * nb * 34, nb, &y[s], &mag[s]);
    return ORC_OK;
}

/* The integer block sums themselves: sumi[i][j][b] for every output. */
int orc_q8_0_q8_0_block_sums(const uint8_t *w, const uint8_t *xq, int64_t m, int64_t n, int64_t k, int32_t *sumi)
{
    if (k % 32 != 0 || m < 0 || n < 0 || k < 0)
        return ORC_ERR_ARG;
    int64_t nb = k / 32;
    for (int64_t i = 0; i < m; i++)
        for (int64_t j = 0; j < n; j++)
            for (int64_t b = 0; b < nb; b++)
                sumi[(i * n + j) * nb + b] = q8_0_q8_0_block_sum(w + (j * nb + b) * 34, xq + (i * nb + b) * 34);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* f32 GEMM, plain orientation [FAST] 6.4:                                   */
/*   C[i][j] = sum_p A[i][p] * B[p][j], accumulated in f64 in p order;       */
/*   mag[i][j] = sum_p |A[i][p] * B[p][j]|.                                 */
/* ------------------------------------------------------------------------ */

/* bt is B transposed (bt[j][p] = B[p][j]), so that one output streams two
 * contiguous rows; the products and their order are those of the definition. */
static void sgemm_one(const float *a, const float *bt, int64_t k, int64_t i, int64_t j, double *c, double *mag)
{
    double acc = 0.0, m = 0.0;
    for (int64_t p = 0; p < k; p++) {
        double prod = (double)a[i * k + p] * (double)bt[j * k + p];
        acc += prod;
        m += fabs(prod);
    }
    *c = acc;
    *mag = m;
}

/* A private copy of b[rows][cols] transposed to [cols][rows] (NULL when out
 * of memory or empty). */
static float *transposed(const float *b, int64_t rows, int64_t cols)
{
    float *t = malloc(sizeof(float) * (size_t)(rows * cols > 0 ? rows * cols : 1));
    if (t)
        for (int64_t p = 0; p < rows; p++)
            for (int64_t j = 0; j < cols; j++)
                t[j * rows + p] = b[p * cols + j];
    return t;
}

int orc_sgemm(const float *a, const float *b, int64_t m, int64_t n, int64_t k, double *c, double *mag)
{
    if (m < 0 || n < 0 || k < 0)
        return ORC_ERR_ARG;
    float *bt = transposed(b, k, n);
    if (!bt && n * k > 0)
        return ORC_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; i++)
        for (int64_t j = 0; j < n; j++)
            sgemm_one(a, bt, k, i, j, &c[i * n + j], &mag[i * n + j]);
    free(bt);
    return ORC_OK;
}

int orc_sgemm_sampled(const float *a, const float *b, int64_t m, int64_t n, int64_t k,
                      const int64_t *ii, const int64_t *jj, int64_t count, double *c, double *mag)
{
    if (m < 0 || n < 0 || k < 0)
        return ORC_ERR_ARG;
    for (int64_t s = 0; s < count; s++)
        if (ii[s] < 0 || ii[s] >= m || jj[s] < 0 || jj[s] >= n)
            return ORC_ERR_ARG;
    float *bt = transposed(b, k, n);
    if (!bt && n * k > 0)
        return ORC_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t s = 0; s < count; s++)
        sgemm_one(a, bt, k, ii[s], jj[s], &c[s], &mag[s]);
    free(bt);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Transposed-B orientation, the linear layer's own [FAST] 6.6: W stored     */
/* [n][k], C[i][j] = sum_p A[i][p] * W[j][p] -- one two-stream dot per       */
/* output.  W is f32, bf16 or f16; bf16 and f16 weights are widened exactly   */
/* ([FAST] "reduced precision": bf16 is the top 16 bits of an f32, widened    */
/* by a 16-bit shift; f16 is widened once per load).  Accumulated in f64 in   */
/* p order; mag = sum_p |A[i][p] * W[j][p]|.                                 */
/* ------------------------------------------------------------------------ */

enum { ORC_W_F32 = 0, ORC_W_BF16 = 1, ORC_W_F16 = 2 };

/* half: orc_half_to_double of every binary16 pattern (half_table). */
static double widen_weight(const void *w, int wtype, int64_t idx, const double *half)
{
    if (wtype == ORC_W_F32)
        return (double)((const float *)w)[idx];
    const uint16_t h = ((const uint16_t *)w)[idx];
    if (wtype == ORC_W_BF16) {
        uint32_t bits = (uint32_t)h << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    return half[h];
}

static void gemm_nt_one(const float *a, const void *w, int wtype, int64_t k, int64_t i, int64_t j,
                        const double *half, double *c, double *mag)
{
    double sum = 0.0, sum_abs = 0.0;
    for (int64_t p = 0; p < k; p++) {
        double prod = (double)a[i * k + p] * widen_weight(w, wtype, j * k + p, half);
        sum += prod;
        sum_abs += fabs(prod);
    }
    *c = sum;
    *mag = sum_abs;
}

int orc_gemm_nt(const float *a, const void *w, int wtype, int64_t m, int64_t n, int64_t k, double *c, double *mag)
{
    if (m < 0 || n < 0 || k < 0 || wtype < ORC_W_F32 || wtype > ORC_W_F16)
        return ORC_ERR_ARG;
    double *half = half_table();
    if (!half)
        return ORC_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; j++)
        for (int64_t i = 0; i < m; i++)
            gemm_nt_one(a, w, wtype, k, i, j, half, &c[i * n + j], &mag[i * n + j]);
    free(half);
    return ORC_OK;
}

int orc_gemm_nt_sampled(const float *a, const void *w, int wtype, int64_t m, int64_t n, int64_t k,
                        const int64_t *ii, const int64_t *jj, int64_t count, double *c, double *mag)
{
    if (m < 0 || n < 0 || k < 0 || wtype < ORC_W_F32 || wtype > ORC_W_F16)
        return ORC_ERR_ARG;
    for (int64_t s = 0; s < count; s++)
        if (ii[s] < 0 || ii[s] >= m || jj[s] < 0 || jj[s] >= n)
            return ORC_ERR_ARG;
    double *half = half_table();
    if (!half)
        return ORC_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t s = 0; s < count; s++)
        gemm_nt_one(a, w, wtype, k, ii[s], jj[s], half, &c[s], &mag[s]);
    free(half);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* BitNet ternary [LOOM].                                                    */
/* ------------------------------------------------------------------------ */

/* codes[n][k] (each 0..2) -> words[n][k/16], code s of a word at bits 2s. */
int orc_pack_ternary(const uint8_t *codes, uint32_t *words, int64_t n, int64_t k)
{
    if (k % 16 != 0 || n < 0 || k < 0)
        return ORC_ERR_ARG;
    int64_t nw = k / 16;
    for (int64_t j = 0; j < n; j++)
        for (int64_t wi = 0; wi < nw; wi++) {
            uint32_t word = 0;
            for (int s = 0; s < 16; s++) {
                uint8_t c = codes[j * k + wi * 16 + s];
                if (c > 2)
                    return ORC_ERR_CODE;
                word |= (uint32_t)c << (2 * s);
            }
            words[j * nw + wi] = word;
        }
    return ORC_OK;
}

int orc_unpack_ternary(const uint32_t *words, uint8_t *codes, int64_t n, int64_t k)
{
    if (k % 16 != 0 || n < 0 || k < 0)
        return ORC_ERR_ARG;
    int64_t nw = k / 16;
    for (int64_t j = 0; j < n; j++)
        for (int64_t wi = 0; wi < nw; wi++)
            for (int s = 0; s < 16; s++)
                codes[j * k + wi * 16 + s] = (uint8_t)((words[j * nw + wi] >> (2 * s)) & 3u);
    return ORC_OK;
}

/* Per-row int8 activations: act_scale = 127 / max|x| (f32), q = round-half-
 * away(x * act_scale) clamped to +-127, act_sum = sum q.  A row whose amax is
 * 0, or whose scale overflows, is all-zero with act_scale = 0. */
int orc_quantize_i8_rows(const float *x, int8_t *q, float *act_scale, int32_t *act_sum, int64_t m, int64_t k)
{
    if (m < 0 || k < 0)
        return ORC_ERR_ARG;
    for (int64_t i = 0; i < m; i++) {
        const float *xr = x + i * k;
        float amax = 0.0f;
        for (int64_t t = 0; t < k; t++) {
            float a = fabsf(xr[t]);
            if (a > amax)
                amax = a;
        }
        float s = (amax == 0.0f) ? 0.0f : 127.0f / amax; /* IEEE f32 division */
        if (!isfinite(s))
            s = 0.0f;
        int32_t sum = 0;
        for (int64_t t = 0; t < k; t++) {
            int v = 0;
            if (s != 0.0f) {
                float r = roundf(xr[t] * s); /* f32 product, half away from zero */
                if (r > 127.0f)
                    r = 127.0f;
                if (r < -127.0f)
                    r = -127.0f;
                v = (int)r;
            }
            q[i * k + t] = (int8_t)v;
            sum += v;
        }
        act_scale[i] = s;
        act_sum[i] = sum;
    }
    return ORC_OK;
}

/* One ternary output: dot = sum_t code_t * q_t - act_sum (the identity),
 * checked against sum_t (code_t - 1) * q_t; y = dot * w_scale / act_scale. */
static int ternary_one(const uint32_t *wrow, int64_t k, const int8_t *qrow, float s, int32_t asum,
                       float w_scale, double *y, double *mag, int32_t *dot_out)
{
    int32_t dot_c = 0, dot_direct = 0, abs_terms = 0;
    for (int64_t t = 0; t < k; t++) {
        int c = (int)((wrow[t / 16] >> (2 * (t % 16))) & 3u);
        if (c == 3)
            return ORC_ERR_CODE;
        dot_c += c * qrow[t];
        dot_direct += (c - 1) * qrow[t];
        abs_terms += abs((c - 1) * qrow[t]);
    }
    int32_t dot = dot_c - asum;
    if (dot != dot_direct)
        return ORC_ERR_IDENTITY;
    if (dot_out)
        *dot_out = dot;
    if (s == 0.0f) {
        *y = 0.0;
        *mag = 0.0;
    } else {
        *y = (double)dot * (double)w_scale / (double)s;
        *mag = (double)abs_terms * fabs((double)w_scale) / (double)s;
    }
    return ORC_OK;
}

int orc_ternary(const uint32_t *w, float w_scale, const int8_t *q, const float *act_scale, const int32_t *act_sum,
                int64_t m, int64_t n, int64_t k, double *y, double *mag, int32_t *dots)
{
    if (k % 16 != 0 || m < 0 || n < 0 || k < 0)
        return ORC_ERR_ARG;
    int64_t nw = k / 16;
    int status = ORC_OK;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; j++)
        for (int64_t i = 0; i < m; i++) {
            int rc = ternary_one(w + j * nw, k, q + i * k, act_scale[i], act_sum[i], w_scale,
                                 &y[i * n + j], &mag[i * n + j], dots ? &dots[i * n + j] : NULL);
            if (rc != ORC_OK) {
#pragma omp critical
                status = rc;
            }
        }
    return status;
}

int orc_ternary_sampled(const uint32_t *w, float w_scale, const int8_t *q, const float *act_scale,
                        const int32_t *act_sum, int64_t m, int64_t n, int64_t k, const int64_t *ii,
                        const int64_t *jj, int64_t count, double *y, double *mag)
{
    if (k % 16 != 0 || m < 0 || n < 0 || k < 0)
        return ORC_ERR_ARG;
    for (int64_t s = 0; s < count; s++)
        if (ii[s] < 0 || ii[s] >= m || jj[s] < 0 || jj[s] >= n)
            return ORC_ERR_ARG;
    int64_t nw = k / 16;
    int status = ORC_OK;
#pragma omp parallel for schedule(static)
    for (int64_t s = 0; s < count; s++) {
        int rc = ternary_one(w + jj[s] * nw, k, q + ii[s] * k, act_scale[ii[s]], act_sum[ii[s]], w_scale,
                             &y[s], &mag[s], NULL);
        if (rc != ORC_OK) {
#pragma omp critical
            status = rc;
        }
    }
    return status;
}

/* Threads of the next parallel loops (the bench runs the oracle on the
 * physical cores only); results do not depend on it. */
void orc_set_num_threads(int count)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    if (count > 0)
        omp_set_num_threads(count);
#else
    (void)count;
#endif
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
