// Q4_0 x Q8_0 prefill GEMM, Y[m][n] = X . W^T, with the per-block arithmetic
// of llama.cpp visual guide lesson 31 "CPU backend" ("How the quantized dot
// product works") for every (i, j):
//     P[i,j,b] = sum_t (q_w[j,b,t] - 8) * q_x[i,b,t]     exact integer
//     Y[i,j]  += f32(d_x[i,b]) * f32(d_w[j,b]) * P[i,j,b]
// Prefill reuses each weight m times and is compute-bound (Fucina course
// "Chapter 06", 6.1), so the block sums run on the matrix cores.
//
// Matrix-core route: v_mfma_f32_16x16x32_f16 with K = 32 = one block.  Both
// operands are small integers (q_w - 8 in [-8, 7], q_x in [-127, 127]), exact
// in f16; every product and the 32-term sum (|P| <= 32512 < 2^24) are exact in
// the f32 accumulator, so P is the exact integer block sum.  The MFMA starts
// from a zero accumulator for each block, and the per-block scale is applied
// on the vector ALU: acc += (d_x * d_w) * P (two ops per output per block).
// That epilogue, not the MFMA, bounds this kernel (ceiling near half the f16
// matrix peak); an int8 MFMA would need a third op per output (i32 -> f32).
//
// Tiles: 128 x 128 outputs per workgroup (4 waves of 64 x 64, each 4 x 4 MFMA
// tiles of 16 x 16), two blocks (64 of k) per stage.  Each stage is decoded
// once into LDS as f16 operands in MFMA lane order plus f32 scales, double
// buffered, with the next stage's raw bytes prefetched in registers.
#include "common.h"

namespace qll {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int QBM = 128, QBN = 128, QKB = 2;
constexpr int kQ4GemmThreads = 256;

// Element order inside the 32 halves of one (row, block) in LDS: lane group h
// (lanes 16h..16h+15 of an MFMA operand) holds elements 4h..4h+3 then
// 16+4h..16+4h+3 -- the low and high nibbles of qs dword h of a Q4_0 block,
// and qs dwords h and 4+h of a Q8_0 block.  A and B use the same order, so
// the MFMA's k-sum runs over the block's 32 elements exactly once.

__device__ __forceinline__ uint32_t f16x2_add(uint32_t h, float c)
{
    f16x2 v = __builtin_bit_cast(f16x2, h);
    f16x2 cc = {(_Float16)c, (_Float16)c};
    return __builtin_bit_cast(uint32_t, v + cc);
}

// 4 unsigned bytes u (each < 256) -> 4 halves 1024 + u, two per dword.
__device__ __forceinline__ void bytes_to_f16_biased(uint32_t u, uint32_t &h01, uint32_t &h23)
{
    h01 = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
    h23 = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
}

// qs dword of a Q8_0 block (4 signed codes) -> 4 exact halves.
__device__ __forceinline__ void q8_dword_to_f16(uint32_t d, uint32_t out[2])
{
    uint32_t h01, h23;
    bytes_to_f16_biased(d ^ 0x80808080u, h01, h23); // code + 128
    out[0] = f16x2_add(h01, -1152.0f);
    out[1] = f16x2_add(h23, -1152.0f);
}

// 4 nibble codes (one per byte, 0..15) -> 4 exact halves code - 8.
__device__ __forceinline__ void q4_nibbles_to_f16(uint32_t c, uint32_t out[2])
{
    uint32_t h01, h23;
    bytes_to_f16_biased(c, h01, h23);
    out[0] = f16x2_add(h01, -1032.0f);
    out[1] = f16x2_add(h23, -1032.0f);
}

// LDS slot of 16-byte chunk h of (block kb, row).  Rows are 64 bytes, so
// without a swizzle the 8 (or 16) consecutive rows that one phase of an
// MFMA-operand ds_read_b128 serves sit on the same banks.  XORing h with
// ((row >> 1) ^ (row >> 3)) & 3 makes any 8 consecutive rows (32 banks of
// 4 bytes) and any 16 consecutive rows (64 banks) distinct; XORing with 3 for
// the second block separates the two blocks of a row written by adjacent
// lanes during staging.
__device__ __forceinline__ int q4gemm_slot(int kb, int row, int h)
{
    return h ^ (((row >> 1) ^ (row >> 3)) & 3) ^ (kb ? 3 : 0);
}

struct Q4GemmLds {
    u32x4 xs[QKB][QBM][4]; // 32 halves per (block, row): 4 x 16 bytes, slots swizzled
    u32x4 ws[QKB][QBN][4];
    float dx[QKB][QBM + 8]; // padded: the two blocks' rows land on different banks
    float dw[QKB][QBN + 8];
};

struct Q4GemmRaw {
    uint32_t xd, xq[8]; // one Q8_0 block
    uint32_t wd, wq[4]; // one Q4_0 block
};

// Thread t stages row t/2, block t%2 of the stage, for both X and W.
// Blocks at or past b_end (the end of this split's k range) load as zero.
__device__ __forceinline__ void q4gemm_load(const uint8_t *__restrict__ w, const uint8_t *__restrict__ xq, int64_t m,
                                            int64_t n, int nb, int b_end, int64_t m0, int64_t n0, int b0,
                                            Q4GemmRaw &r)
{
    const int row = threadIdx.x >> 1, kb = threadIdx.x & 1;
    const int b = b0 + kb;
    const int64_t xi = m0 + row, wj = n0 + row;
    if (xi < m && b < b_end) {
        load_q8_0_block(xq, (xi * nb + b) * 34, r.xd, r.xq);
    } else {
        r.xd = 0;
#pragma unroll
        for (int i = 0; i < 8; i++)
            r.xq[i] = 0;
    }
    if (wj < n && b < b_end) {
        const int64_t o = (wj * nb + b) * 18;
        const uint8_t *p = w + (o & ~(int64_t)3);
        if ((o & 3) == 0) {
            u32x4 a = load4_a4(p);
            uint32_t tail = *reinterpret_cast<const uint16_t *>(w + o + 16);
            r.wd = a[0] & 0xffffu;
            r.wq[0] = funnel(a[1], a[0], 16);
            r.wq[1] = funnel(a[2], a[1], 16);
            r.wq[2] = funnel(a[3], a[2], 16);
            r.wq[3] = funnel(tail, a[3], 16);
        } else {
            u32x4 a = load4_a4(p);
            uint32_t tail = *reinterpret_cast<const uint32_t *>(p + 16);
            r.wd = a[0] >> 16;
            r.wq[0] = a[1];
            r.wq[1] = a[2];
            r.wq[2] = a[3];
            r.wq[3] = tail;
        }
    } else {
        r.wd = 0;
        // code 8 everywhere: weight 0 (and d = 0 too)
#pragma unroll
        for (int i = 0; i < 4; i++)
            r.wq[i] = 0x88888888u;
    }
}

__device__ __forceinline__ void q4gemm_store(const Q4GemmRaw &r, Q4GemmLds &s)
{
    const int row = threadIdx.x >> 1, kb = threadIdx.x & 1;
#pragma unroll
    for (int h = 0; h < 4; h++) {
        uint32_t lo[2], hi[2];
        q8_dword_to_f16(r.xq[h], lo);
        q8_dword_to_f16(r.xq[4 + h], hi);
        s.xs[kb][row][q4gemm_slot(kb, row, h)] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        q4_nibbles_to_f16(r.wq[h] & 0x0f0f0f0fu, lo);
        q4_nibbles_to_f16((r.wq[h] >> 4) & 0x0f0f0f0fu, hi);
        s.ws[kb][row][q4gemm_slot(kb, row, h)] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
    s.dx[kb][row] = half_bits_to_float(r.xd);
    s.dw[kb][row] = half_bits_to_float(r.wd);
}

// One stage: for each of its blocks, the 16 block sums of the wave's 64 x 64
// tile on the matrix core (four at a time, one row of subtiles), each scaled
// by d_x * d_w on the vector ALU into the f32 accumulators.
__device__ __forceinline__ void q4gemm_compute(const Q4GemmLds &s, int wm, int wn, int lr, int lh, f32x4 acc[4][4])
{
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
    for (int kb = 0; kb < QKB; kb++) {
        f16x8 a[4], bm[4];
#pragma unroll
        for (int i = 0; i < 4; i++)
            a[i] = __builtin_bit_cast(f16x8, s.xs[kb][wm + 16 * i + lr][q4gemm_slot(kb, wm + 16 * i + lr, lh)]);
#pragma unroll
        for (int j = 0; j < 4; j++)
            bm[j] = __builtin_bit_cast(f16x8, s.ws[kb][wn + 16 * j + lr][q4gemm_slot(kb, wn + 16 * j + lr, lh)]);
        float dwv[4];
#pragma unroll
        for (int j = 0; j < 4; j++)
            dwv[j] = s.dw[kb][wn + 16 * j + lr];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            f32x4 p[4];
#pragma unroll
            for (int j = 0; j < 4; j++)
                p[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], bm[j], zero, 0, 0, 0);
            // D layout of a 16x16 tile: lane l, register v -> row 4*(l/16)+v, column l%16
            const f32x4 dxv = *reinterpret_cast<const f32x4 *>(&s.dx[kb][wm + 16 * i + 4 * lh]);
#pragma unroll
            for (int j = 0; j < 4; j++)
#pragma unroll
                for (int v = 0; v < 4; v++)
                    acc[i][j][v] = fmaf(dxv[v] * dwv[j], p[j][v], acc[i][j][v]);
        }
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

__global__ __launch_bounds__(kQ4GemmThreads) void q4_0_q8_0_gemm_kernel(const uint8_t *__restrict__ w,
                                                                           const uint8_t *__restrict__ xq,
                                                                           float *__restrict__ y, int64_t m,
                                                                           int64_t n, int nb, int splits)
{
    __shared__ Q4GemmLds lds[2];
    int64_t m_tile, n_tile;
    q4gemm_tile((m + QBM - 1) / QBM, (n + QBN - 1) / QBN, m_tile, n_tile);
    const int64_t m0 = m_tile * QBM, n0 = n_tile * QBN;
    // split-k: blockIdx.y takes blocks [b_begin, b_end) and writes its partial
    // tile to y + blockIdx.y * m * n (the workspace when splits > 1)
    const int per = (nb + splits - 1) / splits;
    const int b_begin = blockIdx.y * per;
    const int b_end = (b_begin + per < nb) ? b_begin + per : nb;
    y += (int64_t)blockIdx.y * m * n;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
    const int lr = lane & 15, lh = lane >> 4;

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Pipeline: stage st+1's LDS buffer is filled from registers loaded two
    // stages earlier, so each global load has two stages of compute to land.
    const int nstages = (b_end - b_begin + QKB - 1) / QKB;
    Q4GemmRaw ra, rb;
    q4gemm_load(w, xq, m, n, nb, b_end, m0, n0, b_begin, ra);
    if (nstages > 1)
        q4gemm_load(w, xq, m, n, nb, b_end, m0, n0, b_begin + QKB, rb);
    q4gemm_store(ra, lds[0]);
    __syncthreads();

    for (int st = 0; st < nstages; st += 2) {
        if (st + 2 < nstages)
            q4gemm_load(w, xq, m, n, nb, b_end, m0, n0, b_begin + (st + 2) * QKB, ra);
        q4gemm_compute(lds[0], wm, wn, lr, lh, acc);
        if (st + 1 < nstages)
            q4gemm_store(rb, lds[1]);
        __syncthreads();
        if (st + 1 >= nstages)
            break;
        if (st + 3 < nstages)
            q4gemm_load(w, xq, m, n, nb, b_end, m0, n0, b_begin + (st + 3) * QKB, rb);
        q4gemm_compute(lds[1], wm, wn, lr, lh, acc);
        if (st + 2 < nstages)
            q4gemm_store(ra, lds[0]);
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int v = 0; v < 4; v++) {
                const int64_t row = m0 + wm + 16 * i + 4 * lh + v;
                const int64_t col = n0 + wn + 16 * j + lr;
                if (row < m && col < n)
                    y[row * n + col] = acc[i][j][v];
            }
}

// y[i] = sum over s of parts[s][i], in split order.
__global__ __launch_bounds__(256) void q4gemm_sum_splits_kernel(const float *__restrict__ parts, float *__restrict__ y,
                                                                int64_t count, int splits)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= count)
        return;
    float v = parts[i];
    for (int s = 1; s < splits; s++)
        v += parts[s * count + i];
    y[i] = v;
}

// Split k when the output tiles alone leave workgroup slots empty (two
// workgroups fit per CU); each split keeps at least 16 blocks.
static int q4gemm_splits(int64_t m, int64_t n, int64_t k)
{
    const int64_t tiles = ((n + QBN - 1) / QBN) * ((m + QBM - 1) / QBM);
    int64_t s = 512 / tiles;
    const int64_t max_s = (k / 32) / 16;
    if (s > max_s)
        s = max_s;
    if (s > 8)
        s = 8;
    return s < 2 ? 1 : (int)s;
}

size_t q4_0_q8_0_gemm_workspace(int64_t m, int64_t n, int64_t k)
{
    const int s = q4gemm_splits(m, n, k);
    return s > 1 ? (size_t)s * (size_t)(m * n) * sizeof(float) : 0;
}

hipError_t launch_q4_0_q8_0_gemm(const uint8_t *w, const uint8_t *xq, float *y, int64_t m, int64_t n, int64_t k,
                                 void *ws, hipStream_t s)
{
    const int64_t tiles = ((n + QBN - 1) / QBN) * ((m + QBM - 1) / QBM);
    const int splits = q4gemm_splits(m, n, k);
    float *out = splits > 1 ? static_cast<float *>(ws) : y;
    hipLaunchKernelGGL(q4_0_q8_0_gemm_kernel, dim3((unsigned)tiles, (unsigned)splits), dim3(kQ4GemmThreads), 0, s,
                       w, xq, out, m, n, (int)(k / 32), splits);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1)
        return e;
    const int64_t count = m * n;
    hipLaunchKernelGGL(q4gemm_sum_splits_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, s, out, y,
                       count, splits);
    return hipGetLastError();
}

} // namespace qll
