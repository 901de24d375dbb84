// Q4_0 x Q8_0 prefill GEMM, Y[m][n] = X . W^T, with the per-block arithmetic
// of llama.cpp visual guide lesson 31 "CPU backend" ("How the quantized dot
// product works") for every (i, j):
//     P[i,j,b] = sum_t (q_w[j,b,t] - 8) * q_x[i,b,t]     exact integer
//     Y[i,j]  += f32(d_x[i,b]) * f32(d_w[j,b]) * P[i,j,b]
// Prefill reuses each weight m times and is compute-bound (Fucina course
// "Chapter 06", 6.1), so the block sums run on the matrix cores.
//
// Matrix-core route: v_mfma_f32_32x32x16_f16, two steps per block.  Both
// operands are small integers (q_w - 8 in [-8, 7], q_x in [-127, 127]), exact
// in f16; every product and the 32-term sum (|P| <= 32512 < 2^24) are exact in
// the f32 accumulator, so P is the exact integer block sum.  The MFMA starts
// from a zero accumulator for each block, and the per-block scale is applied
// on the vector ALU: acc += (d_x * d_w) * P (two ops per output per block).
// That epilogue, not the MFMA, bounds this kernel (ceiling near half the f16
// matrix peak); an int8 MFMA would need a third op per output (i32 -> f32).
//
// Tiles: 128 x 128 outputs per workgroup (4 waves of 64 x 64, each 2 x 2 MFMA
// tiles of 32 x 32), two blocks (64 of k) per stage.  Each stage is decoded
// once into LDS as f16 operands in MFMA lane order plus f32 scales, double
// buffered, with the next stage's raw bytes prefetched in registers.
#include "common.h"

namespace qll {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

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

// Where one thread's staging loads come from.  Thread t stages row t/2,
// block t%2 of every stage, for both X and W; a stage advances two blocks, so
// the parity of the flat block index, which fixes the 2-byte offset of a
// block inside its dword window, stays the same over the whole k loop.
struct Q4GemmSrc {
    int64_t xa, wa; // dword index of the stage-0 windows (X: 34-byte, W: 18-byte blocks)
    int xpar, wpar; // parity of the flat block index
    int b0;         // block index of stage 0
    bool xrow, wrow; // the row lies inside the matrix
};

__device__ __forceinline__ Q4GemmSrc q4gemm_src(int64_t m, int64_t n, int nb, int64_t m0, int64_t n0, int b_begin)
{
    const int row = threadIdx.x >> 1, kb = threadIdx.x & 1;
    Q4GemmSrc c;
    c.b0 = b_begin + kb;
    c.xrow = m0 + row < m;
    c.wrow = n0 + row < n;
    const int64_t g = (c.xrow ? m0 + row : 0) * nb + c.b0; // Q8_0 block at byte 34g
    const int64_t h = (c.wrow ? n0 + row : 0) * nb + c.b0; // Q4_0 block at byte 18h
    c.xpar = (int)(g & 1);
    c.wpar = (int)(h & 1);
    c.xa = (17 * g - c.xpar) / 2; // floor(34g / 4)
    c.wa = (9 * h - c.wpar) / 2;  // floor(18h / 4)
    return c;
}

// Raw bytes of one stage for one thread, loaded without being looked at:
// decoding happens in q4gemm_store, so the loads stay in flight through a
// whole stage of compute.
struct Q4GemmRaw {
    uint32_t xw[9], xtail; // Q8_0: nine dwords from the window start, bytes 32..33 of the window
    uint32_t ww[5], wtail; // Q4_0: five dwords from the window start, bytes 16..17 of the window
    int valid_x, valid_w;
};

// Stage st.  A block at or past b_end (the end of this split's k range), or
// in a row past the matrix edge, loads from dword 0 instead and is zeroed
// when decoded.  Every address stays inside its buffer: an odd-parity block
// starts 2 bytes into its window and needs the ninth (fifth) dword, which
// ends exactly at the block's end; an even-parity block takes its last two
// bytes from the 16-bit tail load and re-reads dword 7 (3) in place of the
// ninth (fifth).  All loads are unconditional, so none forces an early wait.
__device__ __forceinline__ void q4gemm_load(const uint8_t *__restrict__ w, const uint8_t *__restrict__ xq,
                                            const Q4GemmSrc &c, int st, int b_end, Q4GemmRaw &r)
{
    const bool in_k = c.b0 + 2 * st < b_end;
    r.valid_x = c.xrow && in_k;
    r.valid_w = c.wrow && in_k;
    {
        const int64_t a = r.valid_x ? c.xa + 17 * (int64_t)st : 0;
        const uint32_t *p = reinterpret_cast<const uint32_t *>(xq) + a;
        const u32x4 v0 = *reinterpret_cast<const u32x4_a4 *>(p);
        const u32x4 v1 = *reinterpret_cast<const u32x4_a4 *>(p + 4);
        r.xw[0] = v0[0]; r.xw[1] = v0[1]; r.xw[2] = v0[2]; r.xw[3] = v0[3];
        r.xw[4] = v1[0]; r.xw[5] = v1[1]; r.xw[6] = v1[2]; r.xw[7] = v1[3];
        r.xw[8] = p[7 + (r.valid_x ? c.xpar : 0)];
        r.xtail = *reinterpret_cast<const uint16_t *>(p + 8);
    }
    {
        const int64_t a = r.valid_w ? c.wa + 9 * (int64_t)st : 0;
        const uint32_t *p = reinterpret_cast<const uint32_t *>(w) + a;
        const u32x4 v0 = *reinterpret_cast<const u32x4_a4 *>(p);
        r.ww[0] = v0[0]; r.ww[1] = v0[1]; r.ww[2] = v0[2]; r.ww[3] = v0[3];
        r.ww[4] = p[3 + (r.valid_w ? c.wpar : 0)];
        r.wtail = *reinterpret_cast<const uint16_t *>(p + 4);
    }
}

__device__ __forceinline__ void q4gemm_store(const Q4GemmRaw &r, const Q4GemmSrc &c, Q4GemmLds &s)
{
    const int row = threadIdx.x >> 1, kb = threadIdx.x & 1;
    const bool xodd = r.valid_x && c.xpar;
    const bool wodd = r.valid_w && c.wpar;
    uint32_t xd, xq[8], wd, wq[4];
    {
        const uint32_t sh = xodd ? 0u : 16u;
        xd = xodd ? (r.xw[0] >> 16) : (r.xw[0] & 0xffffu);
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const uint32_t hi = (i == 7 && !xodd) ? r.xtail : r.xw[i + 1];
            xq[i] = funnel(hi, xodd ? r.xw[i + 1] : r.xw[i], sh);
        }
        if (!r.valid_x) {
            xd = 0;
#pragma unroll
            for (int i = 0; i < 8; i++)
                xq[i] = 0;
        }
    }
    {
        const uint32_t sh = wodd ? 0u : 16u;
        wd = wodd ? (r.ww[0] >> 16) : (r.ww[0] & 0xffffu);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t hi = (i == 3 && !wodd) ? r.wtail : r.ww[i + 1];
            wq[i] = funnel(hi, wodd ? r.ww[i + 1] : r.ww[i], sh);
        }
        if (!r.valid_w) {
            wd = 0;
#pragma unroll
            for (int i = 0; i < 4; i++)
                wq[i] = 0x88888888u; // code 8: weight 0
        }
    }
#pragma unroll
    for (int h = 0; h < 4; h++) {
        uint32_t lo[2], hi[2];
        q8_dword_to_f16(xq[h], lo);
        q8_dword_to_f16(xq[4 + h], hi);
        s.xs[kb][row][q4gemm_slot(kb, row, h)] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        q4_nibbles_to_f16(wq[h] & 0x0f0f0f0fu, lo);
        q4_nibbles_to_f16((wq[h] >> 4) & 0x0f0f0f0fu, hi);
        s.ws[kb][row][q4gemm_slot(kb, row, h)] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
    s.dx[kb][row] = half_bits_to_float(xd);
    s.dw[kb][row] = half_bits_to_float(wd);
}

// One stage: for each of its blocks, the block sums of the wave's 64 x 64
// tile on the matrix core -- 2 x 2 tiles of 32 x 32, each two K = 16 steps --
// then each scaled by d_x * d_w on the vector ALU into the f32 accumulators.
// MFMA operand lanes: lane l holds row (column) l % 32 of its tile and LDS
// chunk 2s + l / 32 of the block in step s; A and B use the same chunks, so
// the two steps together cover the block's 32 elements once.
__device__ __forceinline__ void q4gemm_compute(const Q4GemmLds &s, int wm, int wn, int lane, f32x16 acc[2][2])
{
    const int lr = lane & 31, lh = lane >> 5;
    const f32x16 zero = {};
#pragma unroll 1
    for (int kb = 0; kb < QKB; kb++) {
        f16x8 a[2][2], bm[2][2];
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int st = 0; st < 2; st++) {
                const int ra = wm + 32 * i + lr, rb = wn + 32 * i + lr;
                a[i][st] = __builtin_bit_cast(f16x8, s.xs[kb][ra][q4gemm_slot(kb, ra, 2 * st + lh)]);
                bm[i][st] = __builtin_bit_cast(f16x8, s.ws[kb][rb][q4gemm_slot(kb, rb, 2 * st + lh)]);
            }
        float dwv[2];
#pragma unroll
        for (int j = 0; j < 2; j++)
            dwv[j] = s.dw[kb][wn + 32 * j + lr];
        // all four tiles' block sums first, so the matrix core runs ahead of
        // the epilogue instead of waiting for it
        f32x16 p[2][2];
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int j = 0; j < 2; j++) {
                p[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i][0], bm[j][0], zero, 0, 0, 0);
                p[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i][1], bm[j][1], p[i][j], 0, 0, 0);
            }
#pragma unroll
        for (int i = 0; i < 2; i++) {
            // D layout of a 32 x 32 tile: lane l, register v -> row
            // 8 (v / 4) + 4 (l / 32) + v % 4, column l % 32
            float dxv[16];
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const f32x4 t = *reinterpret_cast<const f32x4 *>(&s.dx[kb][wm + 32 * i + 8 * q + 4 * lh]);
                dxv[4 * q] = t[0];
                dxv[4 * q + 1] = t[1];
                dxv[4 * q + 2] = t[2];
                dxv[4 * q + 3] = t[3];
            }
#pragma unroll
            for (int j = 0; j < 2; j++)
#pragma unroll
                for (int v = 0; v < 16; v++)
                    acc[i][j][v] = fmaf(dxv[v] * dwv[j], p[i][j][v], acc[i][j][v]);
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

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
            acc[i][j] = f32x16{};

    // Pipeline: stage st+1's LDS buffer is filled from registers loaded two
    // stages earlier, so each global load has two stages of compute to land.
    // Stages go in pairs; with an odd count the last pair's second stage is
    // past b_end, decodes to zeros and adds nothing (0 * 0).  No exit in the
    // middle of the pair keeps the two register sets in fixed registers.
    const int nstages = (b_end - b_begin + QKB - 1) / QKB;
    const Q4GemmSrc src = q4gemm_src(m, n, nb, m0, n0, b_begin);
    Q4GemmRaw ra, rb;
    q4gemm_load(w, xq, src, 0, b_end, ra);
    q4gemm_load(w, xq, src, 1, b_end, rb);
    q4gemm_store(ra, src, lds[0]);
    __syncthreads();

    for (int st = 0; st < nstages; st += 2) {
        q4gemm_load(w, xq, src, st + 2, b_end, ra);
        q4gemm_compute(lds[0], wm, wn, lane, acc);
        q4gemm_store(rb, src, lds[1]);
        __syncthreads();
        q4gemm_load(w, xq, src, st + 3, b_end, rb);
        q4gemm_compute(lds[1], wm, wn, lane, acc);
        q4gemm_store(ra, src, lds[0]);
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const int64_t row = m0 + wm + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                const int64_t col = n0 + wn + 32 * j + (lane & 31);
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
