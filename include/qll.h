/*
 * qll.h -- C ABI of libqll.so, the quantized linear layer y = x.W^T for one
 * AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages, cited by title and section):
 *  [CPU]   llama.cpp visual guide, lesson 31 "CPU backend", section "How the
 *          quantized dot product works" (block_q4_0, the Q4_0 x Q8_0 dot).
 *  [FAST]  Fucina course "Chapter 06 -- Going fast on CPUs": 6.1 "Where the
 *          time goes" (GEMM naming, decode is bandwidth-bound, prefill is
 *          compute-bound), 6.3 "The kernel contract: small, unchecked,
 *          allocation-free", 6.4 "The scalar backend is the specification".
 *  [BACK]  Fucina reference "Backends": 9.2 (the kernel contract: validate
 *          once above, kernels below are unchecked), 9.7 "Quantized matmul
 *          dispatch" (per-call Q8_0 activation quantization; pre-quantized
 *          LHS entries), 9.9 "GPU offload" (an entry reports that it did not
 *          run instead of failing silently).
 *  [LOOM]  Loom "Plan 9 SIMD Forward", section "BitNet ternary MAD kernel".
 *
 * Conventions shared by every entry point
 *  - Data pointers are DEVICE pointers owned by the caller.  The library never
 *    allocates, frees or retains them.  Base addresses must be 16-byte aligned
 *    (every PyTorch/hipMalloc allocation is).  Tensors are dense, row-major.
 *  - `stream` is a hipStream_t passed as `void *` (NULL = the default stream),
 *    so that this header needs no HIP include.  Every call checks
 *    its arguments on the host in O(1), enqueues its kernel(s) on `stream` and
 *    returns without synchronising.  On error nothing is enqueued.  Faults
 *    during execution surface at the caller's next synchronisation.
 *  - Return value: QLL_OK (0) or a negative QLL_ERR_* code; qll_status_string
 *    names it.  Argument checks run before any HIP call, so an invalid call
 *    never touches the device.
 *  - Calls are reentrant; the library keeps no mutable global state besides
 *    a once-per-device architecture check.  Output buffers must not overlap
 *    inputs.
 *  - Not checked (undefined): NaN/Inf inputs, Q4_0 codes > 15 or ternary
 *    codes > 2 handed to the pack entries (the low bits are used), ternary
 *    code 3 inside packed words, act_sum inconsistent with xq.
 *
 * Byte formats (little-endian, packed)
 *  - block_q4_0 (18 B): u16 d (IEEE binary16 bits), u8 qs[16].  Element t < 16
 *    is the low nibble of qs[t], element t >= 16 the high nibble of qs[t-16];
 *    weight = d * (code - 8)  [CPU].
 *  - block_q8_0 (34 B): u16 d (binary16), int8 qs[32]; value ~ d * qs.
 *  - Q4_0 weights W: [n][k/32] blocks, row j = output feature j.
 *    Q8_0 activations X: [m][k/32] blocks.
 *  - Ternary weights: uint32 [n][k/16]; code s of a word (s = 0..15, weight
 *    index 16*word + s) sits at bits 2s..2s+1; code = weight + 1 in {0,1,2}
 *    [LOOM].
 */
#ifndef QLL_H
#define QLL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    QLL_OK = 0,
    QLL_ERR_NULL = -1,      /* a required pointer is NULL */
    QLL_ERR_SHAPE = -2,     /* a size is < 1, not a multiple of the block, or too large */
    QLL_ERR_ALIGN = -3,     /* a base address is not 16-byte aligned */
    QLL_ERR_WORKSPACE = -4, /* ws is NULL or smaller than qll_workspace_bytes() */
    QLL_ERR_LAUNCH = -5,    /* the HIP launch itself failed */
    QLL_ERR_DEVICE = -6,    /* no usable device, or the current device is not gfx950 */
    QLL_ERR_SCRATCH = -7    /* qll_q4_0_q8_0_gemm_noalloc: the shape needs more than its static scratch */
};

/* Operations that may need a caller-owned device workspace. */
enum {
    QLL_OP_SGEMM = 1,
    QLL_OP_Q4_0_Q8_0_GEMM = 2,
    QLL_OP_TERNARY_GEMM = 3,
    QLL_OP_Q4_0_REPACKED_GEMM = 4,
    QLL_OP_Q8_0_REPACKED_GEMM = 5,
    QLL_OP_GEMM_NT_BF16 = 6, /* qll_gemm_nt with QLL_DTYPE_BF16 weights */
    QLL_OP_GEMM_NT_F16 = 7,  /* qll_gemm_nt with QLL_DTYPE_F16 weights on the bf16 matrix core */
    QLL_OP_GEMM_NT_F32 = 8,  /* qll_gemm_nt with QLL_DTYPE_F32 weights on the bf16 matrix core */
    QLL_OP_SGEMM_BF16 = 9,   /* qll_sgemm at m > 1 on the bf16 matrix core */
    QLL_OP_Q4_0_GEMV_F32 = 10 /* qll_q4_0_q8_0_gemv_f32's optional workspace */
};

/* Bytes of device workspace `op` needs at this shape (0 if none); SIZE_MAX if
 * the shape is invalid. */
size_t qll_workspace_bytes(int op, int64_t m, int64_t n, int64_t k);

/* Element types of the weights of qll_gemm_nt. */
enum { QLL_DTYPE_F32 = 0, QLL_DTYPE_BF16 = 1, QLL_DTYPE_F16 = 2 };

/* Static string naming a status code. */
const char *qll_status_string(int status);

/* ---------------------------------------------------------------- packing */

/* Encode Q4_0 weights on the device: codes uint8[n][k] (0..15, weight index
 * t of row j at codes[j*k + t]) and scales uint16[n][k/32] (binary16 bits)
 * -> w block_q4_0[n][k/32] in the layout above [CPU].  k % 32 == 0. */
int qll_pack_q4_0(const uint8_t *codes, const uint16_t *d_bits, void *w, int64_t n, int64_t k, void *stream);

/* Encode ternary codes uint8[n][k] (0..2) into uint32[n][k/16], LSB first
 * [LOOM].  k % 16 == 0. */
int qll_pack_ternary(const uint8_t *codes, uint32_t *w, int64_t n, int64_t k, void *stream);

/* ------------------------------------------------- Q4_0 x Q8_0 (decode, prefill) */

/* Quantize f32 activations x[m][k] to Q8_0 blocks xq[m][k/32] ([BACK] 9.7:
 * the activation rows are quantized per call).  Per 32-block: amax = max|x|,
 * d = amax/127 (IEEE f32 division), q = round-half-away(x/d) (IEEE f32
 * division) clamped to +-127, d stored as binary16 rounded to nearest even;
 * a block whose f32 d is 0 stores q = 0.  Bit-exact with the oracle.
 * k % 32 == 0. */
int qll_quantize_q8_0(const float *x, void *xq, int64_t m, int64_t k, void *stream);

/* Decode GEMV (m = 1): y[j] = sum_b f32(dw[j,b]) * f32(dx[b]) * sumi[j,b],
 * sumi[j,b] = sum_t (qw[j,b,t] - 8) * qx[b,t] exact in int32 [CPU]; the float
 * sum over b is accumulated in f32 in an order of the kernel's choosing
 * (tolerance 1e-4 * sum_b |term_b| against an f64 sum).  w: block_q4_0[n][k/32],
 * xq: block_q8_0[k/32], y: float[n].  k % 32 == 0 and k <= 49152 (else
 * QLL_ERR_SHAPE: the activation row is staged in LDS).  Bandwidth-bound: every
 * weight byte is read once ([FAST] 6.1). */
int qll_q4_0_q8_0_gemv(const void *w, const void *xq, float *y, int64_t n, int64_t k, void *stream);

/* Prefill GEMM: Y[m][n] = X.W^T with the same per-block arithmetic as the
 * GEMV for every (i, j).  xq: block_q8_0[m][k/32], w: block_q4_0[n][k/32],
 * y: float[m][n].  k % 32 == 0, and k < 2^24 when m > 8 (else QLL_ERR_SHAPE:
 * the kernels address 32 activation rows, or a 128-row panel, with 32-bit
 * offsets).  ws/ws_bytes: device workspace of at least
 * qll_workspace_bytes(QLL_OP_Q4_0_Q8_0_GEMM, m, n, k) bytes (nonzero for
 * the 128-row GEMM, m > 64): the call first
 * writes the activations there in the matrix-core operand form (exact f16
 * codes, scale bits, bias terms), then split-k partial sums when it splits
 * k; contents on return are unspecified.  m == 1 runs the GEMV kernel;
 * 2 <= m <= 32 (the small-m band that [BACK] 9.9 gates apart from the
 * general GEMM, one row-dot per weight row in 9.9.2) runs kernels that load
 * every weight once for all m rows -- a GEMV-shaped one, or one that forms
 * 16 x 16 tiles of block sums on the int8 matrix core -- and 33 <= m <= 64
 * runs them on groups of at most 32 activation rows;
 * none of these needs a workspace.  At m == 1 the GEMV's limit k <= 49152
 * applies. */
int qll_q4_0_q8_0_gemm(const void *w, const void *xq, float *y, int64_t m, int64_t n, int64_t k, void *ws,
                       size_t ws_bytes, void *stream);

/* Bytes of the static device scratch of qll_q4_0_q8_0_gemm_noalloc (per device). */
#define QLL_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* qll_q4_0_q8_0_gemm for callers that cannot allocate device memory or pass
 * a workspace (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same kernels, the same results bit for bit,
 * with the workspace taken from a static device array of
 * QLL_NOALLOC_SCRATCH_BYTES (64 MiB) that each device holds from the first
 * call until the process ends.  The call itself allocates nothing.  Shapes
 * whose qll_workspace_bytes(QLL_OP_Q4_0_Q8_0_GEMM, m, n, k) exceeds that
 * size return QLL_ERR_SCRATCH with nothing enqueued (every 8B-class layer at
 * m = 512 fits); the small-m kernels (m <= 64, see above) need no scratch.  All calls on one device share its
 * array and leave their contents there: two calls whose executions overlap
 * on one device (different streams, or graphs replayed concurrently) race
 * and give undefined results, so serialise them.  Other arguments and
 * errors as qll_q4_0_q8_0_gemm. */
int qll_q4_0_q8_0_gemm_noalloc(const void *w, const void *xq, float *y, int64_t m, int64_t n, int64_t k,
                               void *stream);

/* Quantize-fused decode: Y[m][n] = Q8_0(X).W^T for 1 <= m <= 8, from the f32
 * activation rows x: float[m][k] ([BACK] 9.7 quantizes the activation per
 * call), quantized to Q8_0 with exactly the arithmetic of qll_quantize_q8_0
 * and dotted with the per-block arithmetic of qll_q4_0_q8_0_gemm.
 * w: block_q4_0[n][k/32], y: float[m][n], k % 32 == 0; QLL_ERR_SHAPE for m
 * outside [1, 8].
 * ws is optional.  Where qll_workspace_bytes(QLL_OP_Q4_0_GEMV_F32, m, n, k)
 * is nonzero and ws (16-byte aligned, caller-owned, contents not preserved)
 * holds at least that many bytes, the rows are quantized once into ws and
 * the kernel qll_q4_0_q8_0_gemm runs for this shape runs on them: two
 * launches from this one call, as fast as the pair, and the result is that
 * of qll_quantize_q8_0 followed by qll_q4_0_q8_0_gemm bit for bit.
 * Otherwise (ws NULL or smaller, or no workspace needed: m == 1 with a short
 * row and a matrix that one pass of the resident workgroups covers) a single
 * GEMV-shaped launch quantizes the rows inside every workgroup, which is
 * faster only at that size: the same Q8_0 codes and block sums, the float
 * sum over the blocks in that kernel's order (bit for bit the pair's result
 * where qll_q4_0_q8_0_gemm also runs a GEMV-shaped kernel: m == 1, k < 256,
 * m == 2 with n >= 8192, m <= 4 with n >= 32768). */
int qll_q4_0_q8_0_gemv_f32(const void *w, const float *x, float *y, int64_t m, int64_t n, int64_t k, void *ws,
                           size_t ws_bytes, void *stream);

/* ------------------------------------- Q4_0 repacked for the matrix core (prefill) */

/* Bytes of the repacked form of Q4_0 weights W[n][k/32] (SIZE_MAX if the
 * shape is invalid): ceil(n/128) * (k/32) * 3328. */
size_t qll_q4_0_repacked_bytes(int64_t n, int64_t k);

/* Load-time repack of Q4_0 weights into the matrix-core operand form (the
 * packed right-hand side of [BACK] 9.7: rewritten once, reused by every
 * call).  w: block_q4_0[n][k/32]; wp: qll_q4_0_repacked_bytes(n, k) bytes,
 * written in full.  Layout, for 128-row tiles t (rows past n are zero) and
 * blocks b, chunk c = t*(k/32) + b: first the codes, 3072 B per chunk at
 * 3072*c -- the six dwords of row r (r < 128) hold the 6-bit e3m2 codes of
 * w = code - 8 for the block's elements 0..31 (element e at bits 6e), dwords
 * 0..3 at 16*r and dwords 4..5 at 2048 + 8*r; then the scales, the binary16
 * d of row r at byte 2*(128*c + r) of that second region.  Lossless: every
 * w in [-8, 7] is exact in e3m2.  k % 32 == 0. */
int qll_q4_0_repack(const void *w, void *wp, int64_t n, int64_t k, void *stream);

/* Prefill GEMM on repacked weights: Y[m][n] = X.W^T with exactly the
 * per-block arithmetic of qll_q4_0_q8_0_gemm (exact int32 block sums [CPU],
 * f32 scaling; tolerance 1e-4 * sum_b |term_b| against an f64 sum), computed
 * on the matrix core's 6-bit block-scaled path.  wp: the output of
 * qll_q4_0_repack for (n, k); xq: block_q8_0[m][k/32]; y: float[m][n];
 * k % 32 == 0 and k < 2^24 (else QLL_ERR_SHAPE: the kernel addresses the
 * blocks of a row with 32-bit offsets), m >= 1.  ws/ws_bytes: at least
 * qll_workspace_bytes(QLL_OP_Q4_0_REPACKED_GEMM, m, n, k) bytes: the call
 * writes the activations there in operand form (6-bit codes of h and l with
 * q = 16h + l, and d), then split-k partial sums when it splits k; contents on
 * return are unspecified. */
int qll_q4_0_repacked_q8_0_gemm(const void *wp, const void *xq, float *y, int64_t m, int64_t n, int64_t k, void *ws,
                                size_t ws_bytes, void *stream);

/* ------------------------------------------- Q4_0 packed for the decode GEMV */

/* Bytes of the decode-packed form of Q4_0 weights W[n][k/32] (SIZE_MAX if the
 * shape is invalid): n * (16 * (k/32) + 16 * ceil(k/256)) -- 18 bytes per
 * block, as the block_q4_0 array, when k % 256 == 0. */
size_t qll_q4_0_decode_packed_bytes(int64_t n, int64_t k);

/* Load-time repack of Q4_0 weights for the decode GEMV (the packed
 * right-hand side of [BACK] 9.7, with aligned 128-bit loads in place of the
 * 18-byte block stride).  w: block_q4_0[n][k/32]; wp:
 * qll_q4_0_decode_packed_bytes(n, k) bytes, written in full.  Layout, row j
 * at j * (16 * nb + 16 * ceil(nb/8)) with nb = k/32: the nb blocks' 16 nibble
 * bytes (their Q4_0 order) at 16 * b, then their binary16 d at 16 * nb + 2 * b,
 * the scale plane padded with zeros to a multiple of 16 bytes.  k % 32 == 0. */
int qll_q4_0_decode_pack(const void *w, void *wp, int64_t n, int64_t k, void *stream);

/* Decode GEMV on decode-packed weights: y[n] = x.W^T, the arithmetic of
 * qll_q4_0_q8_0_gemv per block (exact int32 block sum, f32 d_w*d_x scaling,
 * tolerance 1e-4 * sum_b |term_b| against an f64 sum; the order of the f32
 * sum differs, so the two are not equal bit for bit).  wp: the output of
 * qll_q4_0_decode_pack for (n, k); xq: block_q8_0[k/32]; y: float[n];
 * k % 32 == 0 and k <= 49152 (the activation row is staged whole in LDS). */
int qll_q4_0_decode_packed_q8_0_gemv(const void *wp, const void *xq, float *y, int64_t n, int64_t k, void *stream);

/* ------------------------------------------------ Q8_0 weights x Q8_0 activations */

/* Weights quantized to Q8_0 blocks too ([BACK] 9.7: a Q8_0-quantized
 * right-hand side against the per-call Q8_0 activation).  Per output and
 * block: sumi = sum_t qw[t] * qx[t] exact in int32, term = f32(dw) * f32(dx)
 * * sumi, summed in f32 (tolerance 1e-4 * sum_b |term_b| against an f64
 * sum).  Weight codes may take the whole int8 range. */

/* Decode GEMV (m = 1): w: block_q8_0[n][k/32], xq: block_q8_0[k/32],
 * y: float[n].  k % 32 == 0 and k <= 49152 (the activation row is staged in
 * LDS).  Bandwidth-bound: every weight byte is read once. */
int qll_q8_0_q8_0_gemv(const void *w, const void *xq, float *y, int64_t n, int64_t k, void *stream);

/* Bytes of the repacked form of Q8_0 weights W[n][k/32] (SIZE_MAX if the
 * shape is invalid): ceil(n/128) * (k/32) * 6400. */
size_t qll_q8_0_repacked_bytes(int64_t n, int64_t k);

/* Load-time repack of Q8_0 weights into the matrix-core operand form
 * ([BACK] 9.7's packed RHS): every code is split exactly as q = 16h + l with
 * l in [-8, 7] and h in [-8, 8] (both e3m2 values).  Layout, for 128-row
 * tiles t (rows past n are zero) and blocks b, chunk c = t*(k/32) + b: the
 * codes first, 6144 B per chunk at 6144*c -- the six dwords of e3m2 codes of
 * h for row r at 16*r (dwords 0..3) and 2048 + 8*r (dwords 4..5), the same
 * for l at 3072 + 16*r and 5120 + 8*r, element e at bits 6e -- then the
 * binary16 d of row r at byte 2*(128*c + r) of the scale region.  Lossless.
 * w: block_q8_0[n][k/32]; wp: qll_q8_0_repacked_bytes(n, k) bytes, written
 * in full.  k % 32 == 0. */
int qll_q8_0_repack(const void *w, void *wp, int64_t n, int64_t k, void *stream);

/* Prefill GEMM on repacked Q8_0 weights: Y[m][n] = X.W^T with the per-block
 * arithmetic above, the exact block sum taken by two 6-bit block-scaled MFMAs
 * (16 h_w and l_w against 16 h_x + l_x).  wp: the output of qll_q8_0_repack;
 * xq: block_q8_0[m][k/32]; y: float[m][n]; k % 32 == 0 and k < 2^24 (else
 * QLL_ERR_SHAPE), m >= 1.  ws/ws_bytes: at least
 * qll_workspace_bytes(QLL_OP_Q8_0_REPACKED_GEMM, m, n, k) bytes
 * (prepared activations, then split-k partials); contents on return are
 * unspecified. */
int qll_q8_0_repacked_q8_0_gemm(const void *wp, const void *xq, float *y, int64_t m, int64_t n, int64_t k, void *ws,
                                size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------- f32 */

/* C[m][n] = A[m][k] . B[k][n], all f32 row-major (the plain orientation of
 * [FAST] 6.4), accumulated in f32 (tolerance 1e-5 * sum_p |a*b| against an
 * f64 sum).  m == 1 runs a split-k GEMV whose partial sums go to ws in a
 * fixed order (results are bit-identical from run to run); ws: at least
 * qll_workspace_bytes(QLL_OP_SGEMM, 1, n, k) bytes.  m > 1 runs on the bf16
 * matrix core when ws holds at least qll_workspace_bytes(QLL_OP_SGEMM_BF16, m,
 * n, k) bytes and k % 16 == 0 (the workspace size selects the algorithm, as
 * in BLAS libraries): A and B (transposed on the way) are each split exactly
 * into three bf16 parts and the part products a_i b_j with i + j <= 4 are
 * accumulated (each one left out is at most 2^-27 of a * b); otherwise (ws
 * NULL or smaller) on the f32 matrix core.  Contents of ws on return
 * unspecified. */
int qll_sgemm(const float *a, const float *b, float *c, int64_t m, int64_t n, int64_t k, void *ws, size_t ws_bytes,
              void *stream);

/* Transposed-B GEMM, the linear layer's own orientation ([FAST] 6.6: W stored
 * [n][k], each output a two-stream dot): Y[m][n] = X[m][k] . W^T, x f32
 * row-major, w of element type w_dtype (QLL_DTYPE_F32, _BF16 or _F16)
 * row-major [n][k], y f32 [m][n].  bf16 and f16 weights are used exactly as
 * stored ([FAST] on reduced precision: bf16 is the top half of an f32; f16 is
 * converted once per load) and never written back as f32; the activations are
 * never rounded; accumulation in f32 (tolerance 1e-5 * sum_p |x * w| against
 * an f64 sum).  m == 1 runs a row-dot GEMV (bandwidth-bound: W is read once).
 * m > 1 runs a matrix-core GEMM: on the f32 matrix core with the weights
 * widened in registers, or, when k % 16 == 0, on the bf16 matrix core with
 * every activation split exactly into three bf16 parts: bf16 weights as
 * stored (each bf16 x bf16 product is exact in f32, so the same products are
 * accumulated), and, when a workspace is passed, f16 weights split exactly
 * into two bf16 parts and f32 weights into three, accumulating the part
 * products x_i w_j with i + j <= 4 (five of six, resp. six of nine; each one
 * left out is at most 2^-27 of x * w).  Any k >= 1.  ws/ws_bytes: bf16
 * weights need at least qll_workspace_bytes(QLL_OP_GEMM_NT_BF16, m, n, k)
 * bytes (the split activations and, when K is split, partial sums; 0 when
 * that path does not run); f16 and f32 weights take the bf16 matrix core when
 * ws holds at least qll_workspace_bytes(QLL_OP_GEMM_NT_F16, resp.
 * QLL_OP_GEMM_NT_F32, m, n, k) bytes (also the weight planes, 2 bytes per
 * weight and plane), and the f32 matrix core otherwise (ws NULL or smaller).
 * Contents on return unspecified.  QLL_ERR_SHAPE for an unknown w_dtype. */
int qll_gemm_nt(const float *x, const void *w, int w_dtype, float *y, int64_t m, int64_t n, int64_t k, void *ws,
                size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------- ternary */

/* Per-row int8 activations [LOOM]: act_scale[i] = 127 / max|x[i,:]| (IEEE
 * f32), xq = round-half-away(x * act_scale) (f32 product) clamped to +-127,
 * act_sum[i] = sum_t xq[i,t].  A row whose amax is 0 or whose scale is not
 * finite gets xq = 0, act_scale = 0, act_sum = 0.  Bit-exact with the oracle.
 * x: float[m][k], xq: int8[m][k], act_scale: float[m], act_sum: int32[m].
 * Any k >= 1. */
int qll_quantize_i8_rows(const float *x, int8_t *xq, float *act_scale, int32_t *act_sum, int64_t m, int64_t k,
                         void *stream);

/* Ternary linear [LOOM]: dot[i,j] = sum_t code[j,t] * xq[i,t] - act_sum[i]
 * (exact int32; equal to sum_t (code - 1) * xq by the ternary identity), then
 * y[i,j] = dot * w_scale / act_scale[i] (0 where act_scale[i] == 0).
 * w: uint32[n][k/16], xq: int8[m][k], y: float[m][n].  k % 16 == 0.
 * The GEMV is the m = 1 case (qll_ternary_gemm with m == 1 runs it): there
 * k <= 65536 (else QLL_ERR_SHAPE: the activation row is staged in LDS). */
int qll_ternary_gemv(const uint32_t *w, float w_scale, const int8_t *xq, const float *act_scale,
                     const int32_t *act_sum, float *y, int64_t n, int64_t k, void *stream);
int qll_ternary_gemm(const uint32_t *w, float w_scale, const int8_t *xq, const float *act_scale,
                     const int32_t *act_sum, float *y, int64_t m, int64_t n, int64_t k, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QLL_H */
