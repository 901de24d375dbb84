// Q4_0 x Q8_0 prefill GEMM, Y[m][n] = X . W^T, with the per-block arithmetic
// of llama.cpp visual guide lesson 31 "CPU backend" ("How the quantized dot
// product works") for every (i, j):
//     P[i,j,b] = sum_t (q_w[j,b,t] - 8) * q_x[i,b,t]     exact integer
//     Y[i,j]  += f32(d_x[i,b]) * f32(d_w[j,b]) * P[i,j,b]
// Prefill reuses each weight m times and is compute-bound (Fucina course
// "Chapter 06", 6.1), so the block sums run on the matrix cores.
//
// Matrix-core route: v_mfma_f32_32x32x16_f16, two K = 16 steps per block, on
// operands that are exact small integers in f16, so every product and every
// partial sum is an exact integer in the f32 accumulator and P is the exact
// block sum.  The per-block scale S = d_x * d_w is the outer product of two
// f16 vectors, and the product of two halves is exact in f32, so the matrix
// core forms it too (v_mfma_f32_32x32x8_f16 with K = 1 used); the vector ALU
// is left with one fma per output per block, acc += S * P, which is what
// bounds the kernel.
//
// Operands.  A weight dword of a Q4_0 block holds codes t..t+3 in its low
// nibbles and t+16..t+19 in its high nibbles.  One v_and_or turns two of its
// nibbles into the halves 1024 + c (low nibble) or 1024 + 16 c (high nibble,
// left in place), so a weight fragment costs five ALU ops and no table.  The
// biases are removed exactly through the MFMA accumulator input instead of
// per element: the activations are prepared once per call (q4gemm_prep_kernel)
// as halves in the same element order -- q_x for low-nibble positions,
// q_x / 16 for high-nibble ones (exact) -- together with
//     C0[i,b] = -(1032 * sum_{t<16} q_x[i,b,t] + 72 * sum_{t>=16} q_x[i,b,t])
// which is the bias term sum_t A_t * (B_t - true B_t).  Starting the block's
// MFMA from C0 yields P exactly: every value on the way is an integer below
// 2^23 in magnitude.
//
// Tiles: 128 x 128 outputs per workgroup, 4 waves of 64 x 64 (2 x 2 MFMA
// tiles of 32 x 32), two blocks per stage, three LDS buffers.  Everything a
// stage reads -- prepared activations, d_x, C0, the weight blocks' code bytes
// and d_w -- goes straight from memory to LDS (global_load_lds, which takes
// the 2-byte aligned addresses of 18-byte weight blocks), two stages ahead.
// Weights stay as nibbles in LDS (a quarter of the bytes of f16) and are
// widened when the fragments are read.  (m <= 32 runs the small-m kernels.)
#include "common.h"

namespace qll {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
#define QLL_LDS __attribute__((address_space(3)))

constexpr int QBM = 128, QBN = 128, QKB = 2, QNBUF = 3;

// A workgroup's four waves in a 2 x 2 grid of 64 x 64 tiles: 2 x 2 MFMA tiles
// of 32 x 32 per wave.
constexpr int QTI = 2, QTJ = 2;
constexpr int QXLoads = QKB * QBM / 16 / 4; // 1 KB activation loads per wave and stage
constexpr int QDma = QXLoads + 1 + 2;       // + d_x or C0, + the weight codes and d_w
__device__ __forceinline__ int q4gemm_wm(int wave) { return (wave >> 1) * 64; }
__device__ __forceinline__ int q4gemm_wn(int wave) { return (wave & 1) * 64; }

constexpr int kQ4GemmThreads = 256;

// Prepared activations: per (row, block) 32 halves = 4 chunks of 16 bytes.
// Chunk c holds the elements paired with weight dword c, in the order the
// weight fragment produces them: codes 4c, 4c+2, 4c+1, 4c+3 (low nibbles),
// then 16+4c, 18+4c, 17+4c, 19+4c (high nibbles, activations divided by 16).
// Rows are padded to a multiple of the row tile and blocks to the end of the last
// split's range, plus two stages, with zeros (zero activations and d_x = 0
// contribute nothing), so the main loop never tests a row or block edge on
// the activation side.
struct Q4GemmPrep {
    u32x4 *x;  // [mp][nbp][4]
    u32x2 *dx; // [nbp][mp]: {binary16 bits of d_x in the low half, 0}
    float *c0; // [nbp][mp]
    int64_t mp, nbp;
};

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Two halves of a dword, h -> h * mul + add (exact for the values used here).
__device__ __forceinline__ uint32_t f16x2_fma(uint32_t h, float mul, float add)
{
    const f16x2 v = __builtin_bit_cast(f16x2, h);
    const f16x2 mm = {(_Float16)mul, (_Float16)mul}, aa = {(_Float16)add, (_Float16)add};
    return __builtin_bit_cast(uint32_t, v * mm + aa);
}

// One thread per (row, block) of the padded prepared arrays; a workgroup
// takes 16 rows x 16 blocks (mp and nbp are multiples of 16), so that both
// the activation chunks (16 blocks of a row are 1 KB) and, through LDS, d_x
// and C0 (16 rows of a block are 64 bytes) are written in contiguous runs.
// The Q8_0 block
// (34 bytes at 34 g, g = row * nb + b) is read as the dword window from
// 34 g - 2 (g & 1): eight dwords plus, for an odd g, a ninth that ends at the
// block's end, for an even g the block's last two bytes as a 16-bit load.
// Codes become halves exactly by the usual exponent trick: the byte q + 128
// placed under the high byte 0x64 is the half 1024 + q + 128.
__global__ __launch_bounds__(256) void q4gemm_prep_kernel(const uint8_t *__restrict__ xq, Q4GemmPrep p, int64_t m,
                                                          int64_t nb)
{
    __shared__ uint32_t sdx[16][17];
    __shared__ float sc0[16][17];
    const int64_t bt = p.nbp / 16;
    const int64_t row0 = (int64_t)(blockIdx.x / bt) * 16, b0 = (int64_t)(blockIdx.x % bt) * 16;
    const int tr = threadIdx.x >> 4, tb = threadIdx.x & 15;
    const int64_t row = row0 + tr, b = b0 + tb;
    u32x4 *dst = p.x + (row * p.nbp + b) * 4;
    uint32_t dxo = 0u;
    float c0o = 0.f;
    if (row >= m || b >= nb) {
#pragma unroll
        for (int c = 0; c < 4; c++)
            dst[c] = u32x4{0u, 0u, 0u, 0u};
    } else {
    const int64_t g = row * nb + b;
    const bool odd = g & 1;
    const uint32_t *w = reinterpret_cast<const uint32_t *>(xq + 34 * g - (odd ? 2 : 0));
    const u32x4 v0 = *reinterpret_cast<const u32x4_a4 *>(w);
    const u32x4 v1 = *reinterpret_cast<const u32x4_a4 *>(w + 4);
    const uint32_t last = odd ? w[8] : (uint32_t)*reinterpret_cast<const uint16_t *>(w + 8);
    const uint32_t win[9] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3], last};
    uint32_t q[8]; // code dwords: codes 4i..4i+3
#pragma unroll
    for (int i = 0; i < 8; i++)
        q[i] = odd ? win[i + 1] : funnel(win[i + 1], win[i], 16);
    const uint32_t d = odd ? (win[0] >> 16) : (win[0] & 0xffffu);
    int lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        lo = sdot4(q[i], 0x01010101u, lo);
        hi = sdot4(q[4 + i], 0x01010101u, hi);
    }
#pragma unroll
    for (int c = 0; c < 4; c++) {
        // codes 4c, 4c+2 | 4c+1, 4c+3 of dword q[c] (low-nibble partners) and
        // of q[4+c] (high-nibble partners, divided by 16)
        const uint32_t ul = q[c] ^ 0x80808080u, uh = q[4 + c] ^ 0x80808080u;
        const uint32_t l02 = __builtin_amdgcn_perm(0x64646464u, ul, 0x04020400u);
        const uint32_t l13 = __builtin_amdgcn_perm(0x64646464u, ul, 0x04030401u);
        const uint32_t h02 = __builtin_amdgcn_perm(0x64646464u, uh, 0x04020400u);
        const uint32_t h13 = __builtin_amdgcn_perm(0x64646464u, uh, 0x04030401u);
        dst[c] = u32x4{f16x2_fma(l02, 1.0f, -1152.0f), f16x2_fma(l13, 1.0f, -1152.0f),
                       f16x2_fma(h02, 0.0625f, -72.0f), f16x2_fma(h13, 0.0625f, -72.0f)};
    }
    dxo = d;
    c0o = -(1032.0f * (float)lo + 72.0f * (float)hi);
    }
    sdx[tb][tr] = dxo;
    sc0[tb][tr] = c0o;
    __syncthreads();
    const int wb = threadIdx.x >> 4, wr = threadIdx.x & 15; // write: block wb, row wr
    p.dx[(b0 + wb) * p.mp + row0 + wr] = u32x2{sdx[wb][wr], 0u};
    p.c0[(b0 + wb) * p.mp + row0 + wr] = sc0[wb][wr];
}

// LDS slot of chunk c of (block kb, row).  Rows are 64 bytes, so without a
// swizzle the 8 (or 16) consecutive rows that one phase of an operand
// ds_read_b128 serves sit on the same banks.  XORing c with
// ((row >> 1) ^ (row >> 3)) & 3 makes any 8 consecutive rows (32 banks of
// 4 bytes) and any 16 consecutive rows (64 banks) distinct.
__device__ __forceinline__ int q4gemm_slot(int kb, int row, int c)
{
    return c ^ (((row >> 1) ^ (row >> 3)) & 3) ^ (kb ? 3 : 0);
}

struct Q4GemmLds {
    u32x4 xs[QKB][QBM][4]; // prepared activations, slots swizzled
    u32x4 wq[QKB][QBN];    // weight code dwords 0..3 of (block, row)
    u32x2 dx[QKB][QBM];    // {binary16 bits of d_x, 0}
    float c0[QKB][QBM];
    uint32_t dw[QKB][QBN]; // binary16 bits of d_w, zero-extended
};

// Every byte a stage needs goes straight from memory to LDS
// (global_load_lds), QDma = 7 wave-wide loads per wave and stage:
//   * the prepared activations (16 KB), four 1 KB loads per wave (lane l of
//     a load writes LDS byte 16 l, so it fetches the chunk that belongs in
//     that slot);
//   * waves 0 and 1: the {d_x, 0} pairs of block kb = wave (1 KB, two rows
//     per lane); waves 2 and 3: C0 of block kb = wave - 2 (512 bytes);
//   * weight rows (wave & 1) * 64 + lane of block kb = wave >> 1: the 16
//     code bytes (block + 2) and d_w (block + 0, a 16-bit load, which the
//     hardware writes to LDS as a zero-extended dword).  Weight blocks are
//     18 bytes, so these addresses are only 2-byte aligned, which the
//     global -> LDS path takes.
// No stage data passes through registers, so the compiler has no loads of
// its own to wait for; the end-of-stage wait (q4gemm_sync) counts these.
struct Q4GemmSrc {
    uint32_t xo[4]; // byte offset of this lane's activation chunk for each 1 KB load, from (m0, block b)
    uint32_t so;    // byte offset of this lane's d_x pair / C0 entries, from (block b, m0)
    uint32_t wo;    // byte offset of this lane's weight block, from (row n0, block b)
};

__device__ __forceinline__ Q4GemmSrc q4gemm_src(const Q4GemmPrep &p, int64_t n0, int64_t n, int nb)
{
    constexpr int XL = QXLoads, RPB = QBM / 16; // 1 KB regions per block
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    Q4GemmSrc c;
#pragma unroll
    for (int j = 0; j < XL; j++) {
        const int region = wave * XL + j; // 1 KB = 16 rows of one block
        const int kb = region / RPB;
        const int row = (region % RPB) * 16 + (lane >> 2);
        c.xo[j] = (uint32_t)((row * p.nbp + kb) * 64 + q4gemm_slot(kb, row, lane & 3) * 16);
    }
    c.so = (uint32_t)(16 * lane);
    const int row = (wave & 1) * 64 + lane;
    const int64_t wrow = (n0 + row < n) ? row : n - 1 - n0; // rows past n: any valid row, output dropped
    c.wo = (uint32_t)(18 * wrow * nb);
    return c;
}

// One wave-wide global -> LDS load: lane l reads `size` bytes at base + off
// (base uniform, in scalar registers) and the wave writes them to LDS at
// lds + 4 l (size 2, zero-extended) or lds + 16 l (size 16).  Inline
// assembly keeps these loads out of the compiler's wait bookkeeping.
__device__ __forceinline__ void q4gemm_dma16(const void *base, uint32_t off, const QLL_LDS void *lds)
{
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base),
                 "s"((uint32_t)(uintptr_t)lds)
                 : "memory", "m0");
}

__device__ __forceinline__ void q4gemm_dma2(const void *base, uint32_t off, const QLL_LDS void *lds)
{
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_ushort %0, %1" ::"v"(off), "s"(base),
                 "s"((uint32_t)(uintptr_t)lds)
                 : "memory", "m0");
}

// Row-tile and column-tile bases of the stage loads, set once per workgroup.
struct Q4GemmBase {
    const uint8_t *x;  // prepared activations of row m0, block 0
    const uint8_t *dx; // {d_x, 0} pairs of block 0, row m0
    const uint8_t *c0; // C0 of block 0, row m0
    const uint8_t *w;  // weight blocks of row n0
    int64_t sblk;      // bytes from one block to the next in dx (c0: half of it)
};

// One wave's loads of stage st (blocks b = b_begin + QKB st + 0, 1).  The
// wave index is a template argument, so that the regions and blocks it
// loads are constants and only the block offsets remain per stage (32-bit
// within a row of prepared activations or of weight blocks, which k < 2^24
// keeps far below 4 GiB; 64-bit across the d_x and C0 arrays).  Weight
// blocks at or past nb load block nb - 1 of the row instead: their
// activations and d_x are zero in the prepared arrays, so they add nothing.
template <int WAVE>
__device__ __forceinline__ void q4gemm_load_wave(const Q4GemmBase &g, const Q4GemmSrc &c, int nb, int b,
                                                 Q4GemmLds &s)
{
    constexpr int XL = QXLoads, RPB = QBM / 16;
    const int lane = threadIdx.x & 63;
    const uint8_t *xb = g.x + (uint32_t)b * 64u;
#pragma unroll
    for (int j = 0; j < XL; j++) {
        constexpr int r0 = WAVE * XL;
        q4gemm_dma16(xb, c.xo[j], (const QLL_LDS void *)&s.xs[(r0 + j) / RPB][((r0 + j) % RPB) * 16][0]);
    }
    // every wave issues exactly one of these (C0: lanes past the data
    // masked), so the per-wave load count stays QDma
    if (WAVE < 2)
        q4gemm_dma16(g.dx + (int64_t)(b + WAVE) * g.sblk, c.so, (const QLL_LDS void *)&s.dx[WAVE][0]);
    else if (lane < QBM / 4)
        q4gemm_dma16(g.c0 + (int64_t)(b + WAVE - 2) * (g.sblk / 2), c.so, (const QLL_LDS void *)&s.c0[WAVE - 2][0]);
    constexpr int kb = WAVE >> 1, rbase = (WAVE & 1) * 64;
    const int bw = (b + kb < nb) ? b + kb : nb - 1;
    const uint8_t *wb = g.w + 18u * (uint32_t)bw;
    q4gemm_dma16(wb + 2, c.wo, (const QLL_LDS void *)&s.wq[kb][rbase]);
    q4gemm_dma2(wb, c.wo, (const QLL_LDS void *)&s.dw[kb][rbase]);
}

// The loads of a stage; `wave` is uniform (a scalar register).
__device__ __forceinline__ void q4gemm_load_stage(const Q4GemmBase &g, const Q4GemmSrc &c, int nb, int b, int wave,
                                                  Q4GemmLds &s)
{
    switch (wave) {
    case 0: q4gemm_load_wave<0>(g, c, nb, b, s); break;
    case 1: q4gemm_load_wave<1>(g, c, nb, b, s); break;
    case 2: q4gemm_load_wave<2>(g, c, nb, b, s); break;
    default: q4gemm_load_wave<3>(g, c, nb, b, s); break;
    }
}

// Weight fragment: dword w of a block (bytes b0..b3) -> eight biased halves,
// 1024 + c for the low nibbles of b0, b2, b1, b3 and 1024 + 16 c for their
// high nibbles in the same order.
// `bias` is 0x64006400 held in a register: with both constants as literals
// the and/or pair cannot be one instruction (no literal operands in VOP3 on
// this architecture), with one of them in a register it is one v_and_or_b32.
__device__ __forceinline__ f16x8 q4gemm_wfrag(uint32_t w, uint32_t bias)
{
    const uint32_t w8 = w >> 8;
    u32x4 h;
    h[0] = (w & 0x000f000fu) | bias;
    h[1] = (w8 & 0x000f000fu) | bias;
    h[2] = (w & 0x00f000f0u) | bias;
    h[3] = (w8 & 0x00f000f0u) | bias;
    return __builtin_bit_cast(f16x8, h);
}

// Byte offsets, from the start of a stage buffer, of everything one lane
// reads in a stage; the reads add only immediates (block, tile, step) to
// them.  Activation slots: q4gemm_slot depends on the row only through bits
// 1..4, which the tile offsets (multiples of 32 rows) leave alone.
struct Q4GemmLaneOff {
    uint32_t x[QKB][2]; // activation chunk of step st, tile row 0
    uint32_t w;         // weight dwords of both steps, tile column 0
    uint32_t dx, dw, c0;
};

__device__ __forceinline__ Q4GemmLaneOff q4gemm_lane_offsets(int wm, int wn, int lane)
{
    using Lds = Q4GemmLds;
    const int lr = lane & 31, lh = lane >> 5;
    Q4GemmLaneOff o;
#pragma unroll
    for (int kb = 0; kb < QKB; kb++)
#pragma unroll
        for (int st = 0; st < 2; st++)
            o.x[kb][st] = (uint32_t)(offsetof(Lds, xs) + (kb * QBM + wm + lr) * 64 +
                                     q4gemm_slot(kb, wm + lr, 2 * lh + st) * 16);
    o.w = (uint32_t)(offsetof(Lds, wq) + (wn + lr) * 16 + lh * 8);
    o.dx = (uint32_t)(offsetof(Lds, dx) + (wm + lr) * 8);
    o.dw = (uint32_t)(offsetof(Lds, dw) + (wn + lr) * 4);
    o.c0 = (uint32_t)(offsetof(Lds, c0) + (wm + 4 * lh) * 4);
    // opaque to the compiler: it would otherwise split off the constant
    // parts again and re-add them per read (read2 pairs take 8-bit offsets)
#pragma unroll
    for (int kb = 0; kb < QKB; kb++)
#pragma unroll
        for (int st = 0; st < 2; st++)
            asm volatile("" : "+v"(o.x[kb][st]));
    asm volatile("" : "+v"(o.w), "+v"(o.dx), "+v"(o.dw), "+v"(o.c0));
    return o;
}

template <typename T>
__device__ __forceinline__ T q4gemm_lds(const QLL_LDS char *base, uint32_t off)
{
    return *reinterpret_cast<const QLL_LDS T *>(base + off);
}

// One stage: for each of its blocks, the block sums of the wave's tile on the
// matrix core -- 2 x 2 tiles of 32 x 32, each two K = 16 steps
// started from C0 -- and the scale tiles, then acc += S * P.  MFMA operand
// lanes: lane l holds row (column) l % 32 of its tile and chunk
// 2 (l / 32) + s of the block in step s (one 8-byte read of a weight row
// gives a lane both of its dwords); A and B use the same chunks, so the two
// steps together cover the block's 32 elements once.
//
// Scale tiles, one K = 8 step: lane l holds k = 4 (l / 32) .. +3.  A row
// lane carries the halves {d_x[r], 0, 0, 0}, a column lane
// {d_w[c], 0, 0, 0}, so the products are zero except at k = 0 and k = 4,
// both d_x[r] d_w[c]: S = 2 d_x d_w exactly (a product of two halves is
// exact in f32, and so is its double).  The factor 2 leaves the kernel as an
// exact halving of the outputs.
__device__ __forceinline__ void q4gemm_compute(const QLL_LDS char *base, const Q4GemmLaneOff &o, uint32_t bias,
                                               f32x16 acc[QTI][QTJ])
{
    constexpr int TI = QTI, TJ = QTJ, NT = TI * TJ;
#pragma unroll
    for (int kb = 0; kb < QKB; kb++) {
        // keeps the two blocks' reads apart (hoisted together they spill)
        __builtin_amdgcn_sched_barrier(0);
        f16x8 a[TI][2], bm[TJ][2];
        f16x4 sa[TI], sb[TJ];
        f32x16 c0[TI];
        static_assert(TI == TJ, "reads interleave row and column tiles");
#pragma unroll
        for (int i = 0; i < TI; i++) {
            const u32x2 wv = q4gemm_lds<u32x2>(base, o.w + kb * QBN * 16 + 512 * i);
            const uint32_t dwb = q4gemm_lds<uint32_t>(base, o.dw + kb * QBN * 4 + 128 * i);
#pragma unroll
            for (int st = 0; st < 2; st++) {
                a[i][st] = __builtin_bit_cast(f16x8, q4gemm_lds<u32x4>(base, o.x[kb][st] + 2048 * i));
                bm[i][st] = q4gemm_wfrag(wv[st], bias);
            }
            sa[i] = __builtin_bit_cast(f16x4, q4gemm_lds<u32x2>(base, o.dx + kb * QBM * 8 + 256 * i));
            sb[i] = __builtin_bit_cast(f16x4, u32x2{dwb, 0u});
            // D layout of a 32 x 32 tile: lane l, register v -> row
            // 8 (v / 4) + 4 (l / 32) + v % 4, column l % 32
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const f32x4 t = q4gemm_lds<f32x4>(base, o.c0 + kb * QBM * 4 + 128 * i + 32 * q);
#pragma unroll
                for (int e = 0; e < 4; e++)
                    c0[i][4 * q + e] = t[e];
            }
        }
        // Software pipeline over the wave's tiles: the matrix core works on
        // tile t while the vector ALU applies tile t-1's scales.  Per tile,
        // in issue order: the first K step and the scale product, half of
        // the previous tile's fmas, the second K step (by then the first has
        // finished), the other half.
        __builtin_amdgcn_sched_barrier(0);
        f32x16 p[2], sc[2];
#pragma unroll
        for (int t = 0; t <= NT; t++) {
            if (t < NT) {
                const int i = t / TJ, j = t % TJ;
                p[t & 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i][0], bm[j][0], c0[i], 0, 0, 0);
                sc[t & 1] = __builtin_amdgcn_mfma_f32_32x32x8f16(sa[i], sb[j], f32x16{}, 0, 0, 0);
                p[t & 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i][1], bm[j][1], p[t & 1], 0, 0, 0);
            }
            if (t > 0) {
                const int u = t - 1, i = u / TJ, j = u % TJ;
#pragma unroll
                for (int v = 0; v < 16; v++)
                    acc[i][j][v] = fmaf(sc[u & 1][v], p[u & 1][v], acc[i][j][v]);
            }
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 3, 0); // tile 0
#pragma unroll
        for (int t = 1; t < NT; t++) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);
    }
}

// Tile order: consecutive workgroup ids go to the 8 XCDs in turn, so tile
// `logical` below is chosen such that each XCD walks a contiguous run of
// (weight tile, all row tiles) -- the row tiles that share a weight tile run
// together on one XCD and meet it in that XCD's L2.
__device__ __forceinline__ void q4gemm_tile(int64_t mt_count, int64_t nt_count, int64_t &m_tile, int64_t &n_tile)
{
    const int64_t total = mt_count * nt_count;
    const int64_t id = blockIdx.x;
    int64_t logical = id;
    if (total % 8 == 0)
        logical = (id % 8) * (total / 8) + id / 8;
    n_tile = logical / mt_count;
    m_tile = logical % mt_count;
}

// Wait until at most N vector-memory loads of this wave are outstanding and
// all its LDS operations are done, then meet the workgroup.  Neither the
// wait nor the barrier is a fence, so compiler barriers keep memory
// operations from moving across them.
template <int N>
__device__ __forceinline__ void q4gemm_sync()
{
    static_assert(N < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | (0x7 << 4)); // vmcnt(N) expcnt(7) lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__global__ __launch_bounds__(kQ4GemmThreads) void q4_0_q8_0_gemm_kernel(const uint8_t *__restrict__ w, Q4GemmPrep prep,
                                                                           float *__restrict__ y, int64_t m,
                                                                           int64_t n, int nb, int per_split)
{
    constexpr int TI = QTI, TJ = QTJ, DMA = QDma;
    __shared__ Q4GemmLds lds[QNBUF];
    int64_t m_tile, n_tile;
    q4gemm_tile(prep.mp / QBM, (n + QBN - 1) / QBN, m_tile, n_tile);
    const int64_t m0 = m_tile * QBM, n0 = n_tile * QBN;
    // split-k: blockIdx.y takes blocks [b_begin, b_begin + per_split) and
    // writes its partial tile to y + blockIdx.y * m * n (the workspace when
    // there are splits); blocks past nb have d_x = 0 in the prepared arrays
    const int b_begin = blockIdx.y * per_split;
    y += (int64_t)blockIdx.y * m * n;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = q4gemm_wm(wave), wn = q4gemm_wn(wave);

    f32x16 acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; i++)
#pragma unroll
        for (int j = 0; j < TJ; j++)
            acc[i][j] = f32x16{};

    const Q4GemmSrc src = q4gemm_src(prep, n0, n, nb);
    const int nstages = per_split / QKB;
    const Q4GemmLaneOff lo = q4gemm_lane_offsets(wm, wn, lane);
    uint32_t bias; // 0x64006400, opaque to the compiler (see q4gemm_wfrag)
    asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(bias));

    // Pipeline, stage st computed from buffer st % 3.  The loads of stage
    // st+2 go out at the start of stage st, into the buffer of stage st-1,
    // which every wave finished reading before the barrier that ended stage
    // st-1; the end-of-stage wait leaves exactly them in flight, so each
    // stage's loads have two stages of compute to land.  Stages past the
    // range load padding and are never computed.
    Q4GemmBase g;
    g.x = reinterpret_cast<const uint8_t *>(prep.x) + m0 * prep.nbp * 64;
    g.dx = reinterpret_cast<const uint8_t *>(prep.dx + m0);
    g.c0 = reinterpret_cast<const uint8_t *>(prep.c0 + m0);
    g.w = w + 18 * n0 * (int64_t)nb;
    g.sblk = prep.mp * 8;
    const int swave = __builtin_amdgcn_readfirstlane(wave);
    q4gemm_load_stage(g, src, nb, b_begin, swave, lds[0]);
    q4gemm_load_stage(g, src, nb, b_begin + QKB, swave, lds[1]);
    q4gemm_sync<DMA>();
    int cur = 0; // buffer of stage st
    for (int st = 0; st < nstages; st++) {
        const int nx2 = cur == 0 ? 2 : cur - 1;
        q4gemm_load_stage(g, src, nb, b_begin + (st + 2) * QKB, swave, lds[nx2]);
        q4gemm_compute((const QLL_LDS char *)&lds[cur], lo, bias, acc);
        q4gemm_sync<DMA>();
        cur = cur == 2 ? 0 : cur + 1;
    }
    // no load may still be writing this workgroup's LDS when it ends
    __builtin_amdgcn_s_waitcnt(0x7 << 4); // vmcnt(0) expcnt(7) lgkmcnt(0)

#pragma unroll
    for (int i = 0; i < TI; i++)
#pragma unroll
        for (int j = 0; j < TJ; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const int64_t row = m0 + wm + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                const int64_t col = n0 + wn + 32 * j + (lane & 31);
                if (row < m && col < n)
                    y[row * n + col] = 0.5f * acc[i][j][v]; // the scale tiles are 2 d_x d_w
            }
}

// y[i] = sum over s of parts[s][i], in split order; four outputs per thread,
// as 16-byte loads and stores when count % 4 == 0 and y is 16-byte aligned
// (VEC): 4096 x 512 outputs of four splits in 6.7 instead of 8.4 us.
template <bool VEC>
__global__ __launch_bounds__(256) void sum_splits_kernel(const float *__restrict__ parts, float *__restrict__ y,
                                                         int64_t count, int splits)
{
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= count)
        return;
    if (VEC) {
        f32x4 v = *reinterpret_cast<const f32x4 *>(parts + i);
        for (int s = 1; s < splits; s++)
            v += *reinterpret_cast<const f32x4 *>(parts + s * count + i);
        *reinterpret_cast<f32x4 *>(y + i) = v;
        return;
    }
    for (int e = 0; e < 4 && i + e < count; e++) {
        float v = parts[i + e];
        for (int s = 1; s < splits; s++)
            v += parts[s * count + i + e];
        y[i + e] = v;
    }
}

hipError_t launch_sum_splits(const float *parts, float *y, int64_t count, int splits, hipStream_t s)
{
    const dim3 grid((unsigned)((count + 1023) / 1024));
    if (count % 4 == 0 && ((uintptr_t)parts & 15u) == 0 && ((uintptr_t)y & 15u) == 0)
        hipLaunchKernelGGL(sum_splits_kernel<true>, grid, dim3(256), 0, s, parts, y, count, splits);
    else
        hipLaunchKernelGGL(sum_splits_kernel<false>, grid, dim3(256), 0, s, parts, y, count, splits);
    return hipGetLastError();
}

// Split k when the output tiles alone leave workgroup slots empty (two
// workgroups fit per CU); each split keeps at least 16 blocks and a multiple
// of 2 QKB of them.  The workspace holds the split partials (if any), then
// the prepared activations, d_x and C0.
struct Q4GemmPlan {
    int splits, per_split;
    int64_t mp, nbp, tiles;
    size_t x_off, dx_off, c0_off, total;
};

static Q4GemmPlan q4gemm_plan(int64_t m, int64_t n, int64_t k)
{
    Q4GemmPlan p;
    const int64_t nb = k / 32;
    p.mp = (m + QBM - 1) / QBM * QBM;
    const int64_t tiles = ((n + QBN - 1) / QBN) * (p.mp / QBM);
    p.tiles = tiles;
    int64_t s = 512 / tiles;
    if (s > nb / 16)
        s = nb / 16;
    if (s > 8)
        s = 8;
    if (s < 2)
        s = 1;
    const int64_t q = 2 * QKB;
    int64_t per = (nb + s - 1) / s;
    per = (per + q - 1) / q * q;
    s = (nb + per - 1) / per;
    p.splits = (int)s;
    p.per_split = (int)per;
    // >= nb: the last split's range plus the two stages the pipeline reads
    // past it, rounded up to the prepass's 16-block tiles
    p.nbp = (per * s + 2 * QKB + 15) / 16 * 16;
    auto up = [](size_t v) { return (v + 255) / 256 * 256; };
    const size_t parts = s > 1 ? up((size_t)s * (size_t)(m * n) * sizeof(float)) : 0;
    p.x_off = parts;
    p.dx_off = p.x_off + up((size_t)(p.mp * p.nbp) * 64);
    p.c0_off = p.dx_off + up((size_t)(p.mp * p.nbp) * 8);
    p.total = p.c0_off + up((size_t)(p.mp * p.nbp) * sizeof(float));
    return p;
}

size_t q4_0_q8_0_gemm_workspace(int64_t m, int64_t n, int64_t k)
{
    return q4gemm_plan(m, n, k).total;
}

hipError_t launch_q4_0_q8_0_gemm(const uint8_t *w, const uint8_t *xq, float *y, int64_t m, int64_t n, int64_t k,
                                 void *ws, hipStream_t s)
{
    const Q4GemmPlan plan = q4gemm_plan(m, n, k);
    uint8_t *base = static_cast<uint8_t *>(ws);
    Q4GemmPrep prep;
    prep.x = reinterpret_cast<u32x4 *>(base + plan.x_off);
    prep.dx = reinterpret_cast<u32x2 *>(base + plan.dx_off);
    prep.c0 = reinterpret_cast<float *>(base + plan.c0_off);
    prep.mp = plan.mp;
    prep.nbp = plan.nbp;
    const int64_t nb = k / 32;
    hipLaunchKernelGGL(q4gemm_prep_kernel, dim3((unsigned)((plan.mp / 16) * (plan.nbp / 16))), dim3(256), 0, s, xq,
                       prep, m, nb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    float *out = plan.splits > 1 ? reinterpret_cast<float *>(base) : y;
    const dim3 grid((unsigned)plan.tiles, (unsigned)plan.splits);
    hipLaunchKernelGGL(q4_0_q8_0_gemm_kernel, grid, dim3(kQ4GemmThreads), 0, s, w, prep, out, m, n, (int)nb,
                       plan.per_split);
    e = hipGetLastError();
    if (e != hipSuccess || plan.splits == 1)
        return e;
    return launch_sum_splits(out, y, m * n, plan.splits, s);
}

} // namespace qll
