// f32 GEMM in the plain orientation, C[m][n] = A[m][k] . B[k][n] (Fucina
// course "Chapter 06 -- Going fast on CPUs", 6.1 for the naming and 6.4 for
// the definition).
//
//  * m = 1 is a GEMV bound by reading B once (64 MiB at 4096^2).  Each lane
//    owns four adjacent columns (16-byte loads along a row of B), the four
//    waves of a workgroup split a 64-row k-chunk between them (16 rows each,
//    all loads issued before any arithmetic) and combine in LDS, and the
//    k-chunks write partial sums to the caller's workspace; a second kernel
//    adds the chunks in a fixed order, so runs are bit-identical
//    (deterministic reductions rather than float atomics).
//  * m > 1 is compute-bound and runs on the f32 matrix cores
//    (v_mfma_f32_32x32x2_f32; gfx950 has no reduced-precision xf32 path, so
//    products are full f32).  128 x 128 output tiles, k-tiles of 16 staged in
//    double-buffered LDS (A stored k-major so a wave's 32 rows are contiguous,
//    B row-major), four waves of 64 x 64 each.
//  * The same GEMM in the transposed-B orientation (W stored [n][k], the
//    linear layer's own, 6.6 of the same chapter): the W tile is read row-wise
//    like A and stored k-major like A; bf16 and f16 weights are widened to f32
//    exactly as they are loaded (the chapter's reduced-precision policy: f32
//    accumulation, no f32 copy of the weights in memory).
#include "common.h"

namespace qll {

typedef float f32x16 __attribute__((ext_vector_type(16)));

// ------------------------------------------------------------------ GEMV

constexpr int kSgemvThreads = 256;
constexpr int kSgemvRows = 16; // rows of B per wave per chunk, all loads in flight at once

struct SgemvPlan {
    int64_t col_groups; // workgroups along n (64 lanes x vec columns each)
    int64_t kc;         // rows of B per k-chunk: 4 waves x kSgemvRows
    int64_t ks;         // number of k-chunks
    int vec;            // columns per lane
};

static SgemvPlan sgemv_plan(int64_t n, int64_t k)
{
    SgemvPlan p;
    p.vec = (n % 4 == 0) ? 4 : 1;
    const int64_t cols_per_wg = 64 * p.vec;
    p.col_groups = (n + cols_per_wg - 1) / cols_per_wg;
    p.kc = 4 * kSgemvRows;
    p.ks = (k + p.kc - 1) / p.kc;
    return p;
}

size_t sgemv_workspace(int64_t n, int64_t k)
{
    SgemvPlan p = sgemv_plan(n, k);
    return (size_t)(p.ks * n) * sizeof(float);
}

// Workgroup (column group, k-chunk of 64 rows): wave w takes rows
// p0 + w, p0 + w + 4, ... of the chunk, issuing all of its 16 loads before
// the first fma (one memory round trip per wave); the four waves combine in
// LDS in a fixed order and write the chunk's partial sums to ws[chunk][n].
// A chunk cut short by the end of k masks its missing rows' products.
template <int VEC>
__global__ __launch_bounds__(kSgemvThreads) void sgemv_partial_kernel(const float *__restrict__ x,
                                                                      const float *__restrict__ b,
                                                                      float *__restrict__ ws, int64_t n, int64_t k,
                                                                      int64_t kc)
{
    __shared__ float s_part[3][64 * VEC];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t col = ((int64_t)blockIdx.x * 64 + lane) * VEC;
    const int64_t chunk = blockIdx.y;
    const int64_t p0 = chunk * kc;
    const int64_t p1 = (p0 + kc < k) ? p0 + kc : k;
    float acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; e++)
        acc[e] = 0.0f;
    if (col < n) {
        float xv[kSgemvRows];
        float bv[kSgemvRows][VEC];
        const bool full = p1 - p0 == kc;
#pragma unroll
        for (int i = 0; i < kSgemvRows; i++) {
            int64_t pi = p0 + wave + 4 * i;
            if (!full)
                pi = pi < p1 ? pi : p1 - 1; // a valid row; its product is masked below
            xv[i] = x[pi];
            if (VEC == 4) {
                const float4 v = *reinterpret_cast<const float4 *>(b + pi * n + col);
                bv[i][0] = v.x;
                bv[i][1] = v.y;
                bv[i][2] = v.z;
                bv[i][3] = v.w;
            } else {
                bv[i][0] = b[pi * n + col];
            }
        }
        if (full) {
#pragma unroll
            for (int i = 0; i < kSgemvRows; i++)
#pragma unroll
                for (int e = 0; e < VEC; e++)
                    acc[e] = fmaf(xv[i], bv[i][e], acc[e]);
        } else {
#pragma unroll
            for (int i = 0; i < kSgemvRows; i++)
                if (p0 + wave + 4 * i < p1)
#pragma unroll
                    for (int e = 0; e < VEC; e++)
                        acc[e] = fmaf(xv[i], bv[i][e], acc[e]);
        }
    }
    if (wave > 0)
#pragma unroll
        for (int e = 0; e < VEC; e++)
            s_part[wave - 1][lane * VEC + e] = acc[e];
    __syncthreads();
    if (wave == 0 && col < n) {
#pragma unroll
        for (int e = 0; e < VEC; e++) {
            float v = acc[e] + s_part[0][lane * VEC + e];
            v += s_part[1][lane * VEC + e];
            v += s_part[2][lane * VEC + e];
            ws[chunk * n + col + e] = v;
        }
    }
}

// c[j] = sum over chunks of ws[s][j]: wave w adds chunks w, w+4, ... in order,
// then the four waves combine in LDS in a fixed order.  A wave issues the
// loads of up to kFinishBatch of its chunks (clamped to valid rows) before the
// first add, so the partial sums, which come from other XCDs' writes, cost one
// memory round trip per batch rather than one per few chunks.
constexpr int kFinishBatch = 16;

__global__ __launch_bounds__(256) void sgemv_finish_kernel(const float *__restrict__ ws, float *__restrict__ c,
                                                           int64_t n, int64_t ks)
{
    __shared__ float s_part[3][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t j = (int64_t)blockIdx.x * 64 + lane;
    const int64_t jc = j < n ? j : n - 1;
    float v = 0.0f;
    for (int64_t s0 = wave; s0 < ks; s0 += 4 * kFinishBatch) {
        float t[kFinishBatch];
#pragma unroll
        for (int u = 0; u < kFinishBatch; u++) {
            const int64_t sc = s0 + 4 * u < ks ? s0 + 4 * u : ks - 1;
            t[u] = ws[sc * n + jc];
        }
#pragma unroll
        for (int u = 0; u < kFinishBatch; u++)
            if (s0 + 4 * u < ks)
                v += t[u];
    }
    if (wave > 0)
        s_part[wave - 1][lane] = v;
    __syncthreads();
    if (wave == 0 && j < n)
        c[j] = ((v + s_part[0][lane]) + s_part[1][lane]) + s_part[2][lane];
}

hipError_t launch_sgemv(const float *x, const float *b, float *c, int64_t n, int64_t k, float *ws, hipStream_t s)
{
    SgemvPlan p = sgemv_plan(n, k);
    dim3 grid((unsigned)p.col_groups, (unsigned)p.ks);
    if (p.vec == 4)
        hipLaunchKernelGGL(sgemv_partial_kernel<4>, grid, dim3(kSgemvThreads), 0, s, x, b, ws, n, k, p.kc);
    else
        hipLaunchKernelGGL(sgemv_partial_kernel<1>, grid, dim3(kSgemvThreads), 0, s, x, b, ws, n, k, p.kc);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(sgemv_finish_kernel, dim3((unsigned)((n + 63) / 64)), dim3(256), 0, s, ws, c, n, p.ks);
    return hipGetLastError();
}

// ------------------------------------------------------------------ GEMM

constexpr int BM = 128, BN = 128, BK = 16;
constexpr int APAD = 4, BPAD = 4;
constexpr int kSgemmThreads = 256;

struct SgemmTileRegs {
    float a[2][4]; // two float4 of A (rows r, r+64; k 4q..4q+3)
    float b[2][4]; // two float4 of B (k rows kr, kr+8; columns 4c..4c+3)
};

// B operand kinds: the plain orientation B[k][n] f32, or the transposed one
// (W stored [n][k], C = A.W^T) with f32, bf16 or f16 weights widened exactly
// to f32 as they are loaded.
constexpr int kBNN = -1;

template <int BT>
__device__ __forceinline__ float sgemm_w_elem(const void *w, int64_t idx)
{
    if (BT == QLL_W_F32)
        return static_cast<const float *>(w)[idx];
    const uint32_t h = static_cast<const uint16_t *>(w)[idx];
    return BT == QLL_W_BF16 ? __builtin_bit_cast(float, h << 16) : half_bits_to_float(h);
}

// FULL: the tile lies inside the matrices (m and n multiples of 128, k of 16),
// so every load is an unconditional 16-byte (8-byte for 16-bit weights) load.
// The per-element bounds checks of the general path compile to branches and
// selects that cost more vector-ALU time per k-tile than the MFMAs leave free.
template <bool VEC, int BT, bool FULL>
__device__ __forceinline__ void sgemm_load_tile(const float *__restrict__ a, const void *__restrict__ bv, int64_t m,
                                                int64_t n, int64_t k, int64_t m0, int64_t n0, int64_t k0,
                                                SgemmTileRegs &t)
{
    const int tid = threadIdx.x;
    if (FULL) {
#pragma unroll
        for (int it = 0; it < 2; it++) {
            const float4 v = *reinterpret_cast<const float4 *>(a + (m0 + (tid >> 2) + 64 * it) * k + k0 + 4 * (tid & 3));
            t.a[it][0] = v.x; t.a[it][1] = v.y; t.a[it][2] = v.z; t.a[it][3] = v.w;
        }
#pragma unroll
        for (int it = 0; it < 2; it++) {
            if (BT == kBNN) {
                const float4 v = *reinterpret_cast<const float4 *>(static_cast<const float *>(bv) +
                                                                   (k0 + (tid >> 5) + 8 * it) * n + n0 + 4 * (tid & 31));
                t.b[it][0] = v.x; t.b[it][1] = v.y; t.b[it][2] = v.z; t.b[it][3] = v.w;
            } else if (BT == QLL_W_F32) {
                const float4 v = *reinterpret_cast<const float4 *>(static_cast<const float *>(bv) +
                                                                   (n0 + (tid >> 2) + 64 * it) * k + k0 + 4 * (tid & 3));
                t.b[it][0] = v.x; t.b[it][1] = v.y; t.b[it][2] = v.z; t.b[it][3] = v.w;
            } else {
                const uint2 v = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(bv) +
                                                                 (n0 + (tid >> 2) + 64 * it) * k + k0 + 4 * (tid & 3));
                const uint32_t h[4] = {v.x & 0xffffu, v.x >> 16, v.y & 0xffffu, v.y >> 16};
#pragma unroll
                for (int e = 0; e < 4; e++)
                    t.b[it][e] = BT == QLL_W_BF16 ? __builtin_bit_cast(float, h[e] << 16) : half_bits_to_float(h[e]);
            }
        }
        return;
    }
    // A: 128 rows x 16 k = 512 float4, two per thread
#pragma unroll
    for (int it = 0; it < 2; it++) {
        const int64_t row = m0 + (tid >> 2) + 64 * it;
        const int64_t kk = k0 + 4 * (tid & 3);
        if (VEC && row < m && kk + 3 < k) {
            float4 v = *reinterpret_cast<const float4 *>(a + row * k + kk);
            t.a[it][0] = v.x; t.a[it][1] = v.y; t.a[it][2] = v.z; t.a[it][3] = v.w;
        } else {
#pragma unroll
            for (int e = 0; e < 4; e++)
                t.a[it][e] = (row < m && kk + e < k) ? a[row * k + kk + e] : 0.0f;
        }
    }
    if (BT == kBNN) {
        // B: 16 rows x 128 columns = 512 float4, two per thread
        const float *b = static_cast<const float *>(bv);
#pragma unroll
        for (int it = 0; it < 2; it++) {
            const int64_t kr = k0 + (tid >> 5) + 8 * it;
            const int64_t col = n0 + 4 * (tid & 31);
            if (VEC && kr < k && col + 3 < n) {
                float4 v = *reinterpret_cast<const float4 *>(b + kr * n + col);
                t.b[it][0] = v.x; t.b[it][1] = v.y; t.b[it][2] = v.z; t.b[it][3] = v.w;
            } else {
#pragma unroll
                for (int e = 0; e < 4; e++)
                    t.b[it][e] = (kr < k && col + e < n) ? b[kr * n + col + e] : 0.0f;
            }
        }
    } else {
        // W: 128 rows (output columns) x 16 k, loaded like A: four adjacent k
        // of one row per thread (16 bytes of f32, 8 of bf16/f16), widened
#pragma unroll
        for (int it = 0; it < 2; it++) {
            const int64_t col = n0 + (tid >> 2) + 64 * it;
            const int64_t kk = k0 + 4 * (tid & 3);
            if (VEC && col < n && kk + 3 < k) {
                if (BT == QLL_W_F32) {
                    const float4 v = *reinterpret_cast<const float4 *>(static_cast<const float *>(bv) + col * k + kk);
                    t.b[it][0] = v.x; t.b[it][1] = v.y; t.b[it][2] = v.z; t.b[it][3] = v.w;
                } else {
                    const uint2 v = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(bv) + col * k + kk);
                    const uint32_t h[4] = {v.x & 0xffffu, v.x >> 16, v.y & 0xffffu, v.y >> 16};
#pragma unroll
                    for (int e = 0; e < 4; e++)
                        t.b[it][e] = BT == QLL_W_BF16 ? __builtin_bit_cast(float, h[e] << 16) : half_bits_to_float(h[e]);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; e++)
                    t.b[it][e] = (col < n && kk + e < k) ? sgemm_w_elem<BT>(bv, col * k + kk + e) : 0.0f;
            }
        }
    }
}

template <int BT>
__device__ __forceinline__ void sgemm_store_tile(const SgemmTileRegs &t, float (*As)[BM + APAD],
                                                 float (*Bs)[BN + BPAD])
{
    const int tid = threadIdx.x;
#pragma unroll
    for (int it = 0; it < 2; it++) {
        const int row = (tid >> 2) + 64 * it;
        const int kq = 4 * (tid & 3);
#pragma unroll
        for (int e = 0; e < 4; e++)
            As[kq + e][row] = t.a[it][e];
    }
    if (BT == kBNN) {
#pragma unroll
        for (int it = 0; it < 2; it++) {
            const int kr = (tid >> 5) + 8 * it;
            const int col = 4 * (tid & 31);
            *reinterpret_cast<float4 *>(&Bs[kr][col]) = make_float4(t.b[it][0], t.b[it][1], t.b[it][2], t.b[it][3]);
        }
    } else { // k-major, like A
#pragma unroll
        for (int it = 0; it < 2; it++) {
            const int col = (tid >> 2) + 64 * it;
            const int kq = 4 * (tid & 3);
#pragma unroll
            for (int e = 0; e < 4; e++)
                Bs[kq + e][col] = t.b[it][e];
        }
    }
}

template <bool VEC, int BT, bool FULL>
__global__ __launch_bounds__(kSgemmThreads) void sgemm_mfma_kernel(const float *__restrict__ a,
                                                                   const void *__restrict__ b,
                                                                   float *__restrict__ c, int64_t m, int64_t n,
                                                                   int64_t k)
{
    __shared__ __attribute__((aligned(16))) float As[2][BK][BM + APAD];
    __shared__ __attribute__((aligned(16))) float Bs[2][BK][BN + BPAD];

    // Tile order: workgroups are dealt to the eight XCDs in turn (L2 is per
    // XCD), so when the grid allows, XCD x takes a contiguous run of tiles,
    // read in groups of eight row tiles: its resident workgroups then share
    // 8 row panels of A and tiles / 64 column panels of B instead of every
    // row panel (4096^3: 812 -> 700 MB of HBM traffic, the same time).
    int64_t m0, n0;
    {
        const int64_t ntx = gridDim.x, nty = gridDim.y, tiles = ntx * nty;
        const int64_t lin = blockIdx.x + ntx * (int64_t)blockIdx.y;
        if (tiles % 64 == 0 && nty % 8 == 0) {
            const int64_t t = (lin % 8) * (tiles / 8) + lin / 8;
            const int64_t grp = t / (8 * ntx), in = t % (8 * ntx);
            m0 = (grp * 8 + in % 8) * BM;
            n0 = (in / 8) * BN;
        } else {
            m0 = (int64_t)blockIdx.y * BM;
            n0 = (int64_t)blockIdx.x * BN;
        }
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64; // wave tile origin inside the block tile
    const int li = lane & 31, lh = lane >> 5;

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int v = 0; v < 16; v++)
                acc[i][j][v] = 0.0f;

    const int64_t nkt = (k + BK - 1) / BK;
    SgemmTileRegs regs;
    sgemm_load_tile<VEC, BT, FULL>(a, b, m, n, k, m0, n0, 0, regs);
    sgemm_store_tile<BT>(regs, As[0], Bs[0]);
    __syncthreads();

    for (int64_t kt = 0; kt < nkt; kt++) {
        const int cur = (int)(kt & 1);
        if (kt + 1 < nkt)
            sgemm_load_tile<VEC, BT, FULL>(a, b, m, n, k, m0, n0, (kt + 1) * BK, regs);
        // the MFMA phase at raised priority: with four workgroups per CU the
        // SIMD's arbiter then prefers a wave that feeds the matrix core over
        // one that writes the next tile (1064 against 1071 us at 4096^3)
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int s = 0; s < BK / 2; s++) {
            const int kk = 2 * s + lh; // lanes 0-31 take k = 2s, lanes 32-63 k = 2s+1
            float av[2], bv[2];
#pragma unroll
            for (int i = 0; i < 2; i++)
                av[i] = As[cur][kk][wm + 32 * i + li];
#pragma unroll
            for (int j = 0; j < 2; j++)
                bv[j] = Bs[cur][kk][wn + 32 * j + li];
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int j = 0; j < 2; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[i], bv[j], acc[i][j], 0, 0, 0);
        }
        __builtin_amdgcn_s_setprio(0);
        if (kt + 1 < nkt)
            sgemm_store_tile<BT>(regs, As[cur ^ 1], Bs[cur ^ 1]);
        __syncthreads();
    }

    // D layout of a 32x32 MFMA tile: lane l, register v holds
    // row 8*(v/4) + 4*(l/32) + v%4, column l%32.
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const int64_t row = m0 + wm + 32 * i + 8 * (v >> 2) + 4 * lh + (v & 3);
                const int64_t col = n0 + wn + 32 * j + li;
                if (FULL || (row < m && col < n))
                    c[row * n + col] = acc[i][j][v];
            }
}

hipError_t launch_sgemm(const float *a, const float *b, float *c, int64_t m, int64_t n, int64_t k, hipStream_t s)
{
    dim3 grid((unsigned)((n + BN - 1) / BN), (unsigned)((m + BM - 1) / BM));
    if (m % BM == 0 && n % BN == 0 && k % BK == 0)
        hipLaunchKernelGGL((sgemm_mfma_kernel<true, kBNN, true>), grid, dim3(kSgemmThreads), 0, s, a, b, c, m, n, k);
    else if (k % 4 == 0 && n % 4 == 0)
        hipLaunchKernelGGL((sgemm_mfma_kernel<true, kBNN, false>), grid, dim3(kSgemmThreads), 0, s, a, b, c, m, n, k);
    else
        hipLaunchKernelGGL((sgemm_mfma_kernel<false, kBNN, false>), grid, dim3(kSgemmThreads), 0, s, a, b, c, m, n, k);
    return hipGetLastError();
}

template <int BT>
static hipError_t launch_sgemm_nt_t(const float *a, const void *w, float *c, int64_t m, int64_t n, int64_t k,
                                    hipStream_t s)
{
    dim3 grid((unsigned)((n + BN - 1) / BN), (unsigned)((m + BM - 1) / BM));
    if (m % BM == 0 && n % BN == 0 && k % BK == 0)
        hipLaunchKernelGGL((sgemm_mfma_kernel<true, BT, true>), grid, dim3(kSgemmThreads), 0, s, a, w, c, m, n, k);
    else if (k % 4 == 0)
        hipLaunchKernelGGL((sgemm_mfma_kernel<true, BT, false>), grid, dim3(kSgemmThreads), 0, s, a, w, c, m, n, k);
    else
        hipLaunchKernelGGL((sgemm_mfma_kernel<false, BT, false>), grid, dim3(kSgemmThreads), 0, s, a, w, c, m, n, k);
    return hipGetLastError();
}

hipError_t launch_sgemm_nt(const float *a, const void *w, int wfmt, float *c, int64_t m, int64_t n, int64_t k,
                           hipStream_t s)
{
    if (wfmt == QLL_W_F32)
        return launch_sgemm_nt_t<QLL_W_F32>(a, w, c, m, n, k, s);
    if (wfmt == QLL_W_BF16)
        return launch_sgemm_nt_t<QLL_W_BF16>(a, w, c, m, n, k, s);
    return launch_sgemm_nt_t<QLL_W_F16>(a, w, c, m, n, k, s);
}

} // namespace qll
