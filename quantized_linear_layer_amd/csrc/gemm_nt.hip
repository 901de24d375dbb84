// Transposed-B GEMV, y[j] = sum_p x[p] * W[j][p] with W stored [n][k] -- the
// linear layer's own orientation, a two-stream dot per output (Fucina course
// "Chapter 06 -- Going fast on CPUs", 6.6) -- for f32, bf16 or f16 weights,
// widened exactly in registers and accumulated in f32 (the same chapter on
// reduced precision: bf16 is the top half of an f32, widened by a 16-bit
// shift; f16 is converted once per load; f32 activations are never rounded).
//
// Decode is bound by reading W once.  L lanes share a row (64/L rows per
// wave); a lane reads 16-byte vectors of its row (4 f32 or 8 halves) at
// stride L, U of them in flight, and the next chunk's weight loads are issued
// before the current chunk's fmas.  The activation vector is read through the
// cache (every row of a workgroup reads the same addresses).  Rows whose byte
// length is not a multiple of 16 take a scalar variant.
#include "common.h"

namespace qll {

constexpr int kGemvNtThreads = 256;

template <int WFMT>
struct NtW {
    static constexpr int ES = WFMT == QLL_W_F32 ? 4 : 2; // bytes per weight
    static constexpr int V = 16 / ES;                    // weights per 16-byte vector
};

__device__ __forceinline__ float bf16_to_float(uint32_t h) { return __builtin_bit_cast(float, h << 16); }
__device__ __forceinline__ float f16_to_float(uint32_t h) { return half_bits_to_float(h); }

// Weight e (0 <= e < V) of a 16-byte vector.
template <int WFMT>
__device__ __forceinline__ float nt_weight(const u32x4 &v, int e)
{
    if (WFMT == QLL_W_F32) {
        // the element is copied out first: a bit_cast applied to the vector
        // subscript itself compiled to the same element for every e
        const uint32_t word = v[e];
        return __builtin_bit_cast(float, word);
    }
    const uint32_t word = v[e >> 1];
    const uint32_t h = (e & 1) ? (word >> 16) : (word & 0xffffu);
    return WFMT == QLL_W_BF16 ? bf16_to_float(h) : f16_to_float(h);
}

template <int WFMT>
__device__ __forceinline__ float nt_weight_scalar(const uint8_t *w, int64_t idx)
{
    if (WFMT == QLL_W_F32)
        return reinterpret_cast<const float *>(w)[idx];
    const uint32_t h = reinterpret_cast<const uint16_t *>(w)[idx];
    return WFMT == QLL_W_BF16 ? bf16_to_float(h) : f16_to_float(h);
}

template <int WFMT, int U>
struct NtRaw {
    u32x4 w[U];
    float4 x[U][NtW<WFMT>::V / 4];
};

// A chunk's activation pieces are requested with its weights, one chunk
// ahead: loads retire in order, so activation loads issued inside the dot
// would wait for the next chunk's weights (4096^2: f32 weights 15.3 -> 13.5
// us, bf16 9.0 -> 8.3 us).
template <int WFMT, int L, int U>
__device__ __forceinline__ void nt_load(const float *__restrict__ x, const uint8_t *wr, int64_t nv, int64_t c0, int r,
                                        NtRaw<WFMT, U> &raw)
{
    constexpr int V = NtW<WFMT>::V;
#pragma unroll
    for (int i = 0; i < U; i++) {
        int64_t v = c0 + r + (int64_t)i * L;
        v = v < nv ? v : 0; // past the row: reload vector 0 (masked in nt_dot)
#pragma unroll
        for (int q = 0; q < V / 4; q++)
            raw.x[i][q] = *reinterpret_cast<const float4 *>(x + v * V + 4 * q);
        raw.w[i] = *reinterpret_cast<const u32x4 *>(wr + v * 16);
    }
}

template <int WFMT, int L, int U>
__device__ __forceinline__ float nt_dot(int64_t nv, int64_t c0, int r, const NtRaw<WFMT, U> &raw)
{
    constexpr int V = NtW<WFMT>::V;
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < U; i++) {
        const int64_t v = c0 + r + (int64_t)i * L;
        if (v < nv) {
#pragma unroll
            for (int q = 0; q < V / 4; q++) {
                const float4 xs = raw.x[i][q];
                acc = fmaf(xs.x, nt_weight<WFMT>(raw.w[i], 4 * q + 0), acc);
                acc = fmaf(xs.y, nt_weight<WFMT>(raw.w[i], 4 * q + 1), acc);
                acc = fmaf(xs.z, nt_weight<WFMT>(raw.w[i], 4 * q + 2), acc);
                acc = fmaf(xs.w, nt_weight<WFMT>(raw.w[i], 4 * q + 3), acc);
            }
        }
    }
    return acc;
}

template <int WFMT, int L, int U, bool VEC>
__global__ __launch_bounds__(kGemvNtThreads) void gemv_nt_kernel(const float *__restrict__ x,
                                                                 const uint8_t *__restrict__ w,
                                                                 float *__restrict__ y, int64_t n, int64_t k)
{
    constexpr int R = 64 / L, ES = NtW<WFMT>::ES;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane / L, r = lane % L;
    const int64_t row = ((int64_t)blockIdx.x * (kGemvNtThreads / 64) + wave) * R + g;
    const int64_t rowc = row < n ? row : n - 1; // rows past n load row n - 1; never stored
    const uint8_t *wr = w + rowc * k * ES;
    float acc = 0.0f;
    if (VEC) {
        const int64_t nv = k / NtW<WFMT>::V;
        const int64_t step = (int64_t)L * U;
        NtRaw<WFMT, U> cur, nxt;
        nt_load<WFMT, L, U>(x, wr, nv, 0, r, cur);
        for (int64_t c0 = 0; c0 < nv; c0 += step) {
            if (c0 + step < nv)
                nt_load<WFMT, L, U>(x, wr, nv, c0 + step, r, nxt);
            acc += nt_dot<WFMT, L, U>(nv, c0, r, cur);
            cur = nxt;
        }
    } else {
        for (int64_t p = r; p < k; p += L)
            acc = fmaf(x[p], nt_weight_scalar<WFMT>(wr, p), acc);
    }
#pragma unroll
    for (int off = L / 2; off > 0; off >>= 1)
        acc += __shfl_xor(acc, off);
    if (row < n && r == 0)
        y[row] = acc;
}

template <int WFMT, int L, int U, bool VEC>
static hipError_t launch_nt_l(const float *x, const uint8_t *w, float *y, int64_t n, int64_t k, hipStream_t s)
{
    constexpr int R = 64 / L;
    const int64_t rows_per_wg = R * (kGemvNtThreads / 64);
    const int64_t grid = (n + rows_per_wg - 1) / rows_per_wg;
    if (grid > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((gemv_nt_kernel<WFMT, L, U, VEC>), dim3((unsigned)grid), dim3(kGemvNtThreads), 0, s, x, w, y,
                       n, k);
    return hipGetLastError();
}

// Lanes per row: one pass of 4 vectors per lane for short rows, 64 lanes
// (several chunks) for long ones.
template <int WFMT>
static hipError_t launch_nt(const float *x, const uint8_t *w, float *y, int64_t n, int64_t k, hipStream_t s)
{
    constexpr int V = NtW<WFMT>::V;
    if (k % V != 0)
        return launch_nt_l<WFMT, 64, 1, false>(x, w, y, n, k, s);
    const int64_t nv = k / V;
    if (nv <= 32)
        return launch_nt_l<WFMT, 8, 4, true>(x, w, y, n, k, s);
    if (nv <= 64)
        return launch_nt_l<WFMT, 16, 4, true>(x, w, y, n, k, s);
    if (nv <= 128)
        return launch_nt_l<WFMT, 32, 4, true>(x, w, y, n, k, s);
    return launch_nt_l<WFMT, 64, 4, true>(x, w, y, n, k, s);
}

// ------------------------------------------------------------------ bf16 weights, m > 1
// The bf16-weight GEMM on the bf16 matrix cores (v_mfma_f32_32x32x16_bf16)
// without rounding the activations: every f32 activation is split exactly
// into three bf16 parts, x = x1 + x2 + x3 (x1 = bf16(x), x2 = bf16(x - x1),
// x3 = x - x1 - x2: the residuals have at most 16 and 8 significant bits), and
// each product of two bf16 values is exact in f32, so the three MFMAs per K
// step accumulate exactly the products the f32 path forms, in f32.  A
// prepass writes the three parts in the tile layout the kernel reads; the
// weights are read as they are ([n][k] bf16, never widened in memory).
//
// Tiles: 128 x 128 outputs per workgroup, 4 waves of 64 x 64 (2 x 2 MFMA
// tiles), K steps of 16, three LDS buffers filled by global_load_lds two
// steps ahead.  A row of a 16-wide K step is 32 bytes (two 16-byte halves,
// the two lane halves' operands); half h of row r sits at h ^ ((r >> 3) & 1),
// so the 16 rows one ds_read_b128 serves fall in distinct banks.

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
#define QLL_LDS_NT __attribute__((address_space(3)))

constexpr int kNbM = 128, kNbK = 16, kNbBuf = 3, kNbThreads = 256;
constexpr int kNbPlane = kNbM * kNbK * 2;  // 4096 bytes: one part of a 128-row K step
constexpr int kNbAChunk = 3 * kNbPlane;    // the three parts
// NJ = 32-column tiles per wave: the workgroup covers 64 NJ weight rows
// NW weight planes: 1 for bf16 weights (used as stored), 2 for f16 weights
// and 3 for f32 weights (each split exactly into that many bf16 parts by
// nt_w_split_kernel).
template <int NJ, int NW>
struct NbCfg {
    static constexpr int BN = 64 * NJ;
    static constexpr int WChunk = BN * kNbK * 2; // bytes of one weight plane per K step
    static constexpr int Dma = 3 + NW * NJ / 2;   // loads per wave and stage (3 of activations, NJ/2 per plane)
};

struct NbPrep {
    uint8_t *a; // [mp / 128][kp / 16] chunks of kNbAChunk bytes
    int64_t mp, kp;
};

__device__ __forceinline__ int nb_half(int r, int h) { return h ^ ((r >> 3) & 1); }

__device__ __forceinline__ uint32_t bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Three exact bf16 parts of 8 activations, packed two per dword per part.
__device__ __forceinline__ void nb_split8(const float v[8], uint32_t part[3][4])
{
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        uint32_t b[3][2];
#pragma unroll
        for (int q = 0; q < 2; q++) {
            const float x0 = v[e + q];
            const uint32_t h1 = bf16_bits(x0);
            const float r1 = x0 - __builtin_bit_cast(float, h1 << 16); // exact
            const uint32_t h2 = bf16_bits(r1);
            const float r2 = r1 - __builtin_bit_cast(float, h2 << 16); // exact, at most 8 significant bits
            b[0][q] = h1;
            b[1][q] = h2;
            b[2][q] = bf16_bits(r2); // exact
        }
#pragma unroll
        for (int pp = 0; pp < 3; pp++)
            part[pp][e >> 1] = b[pp][0] | (b[pp][1] << 16);
    }
}


// One workgroup per chunk (128 rows x 16 k); thread (row r, half h) splits
// the 8 activations x[row][16 kt + 8 h ..] (zero past m or k).
__global__ __launch_bounds__(256) void nt_bf16_prep_kernel(const float *__restrict__ x, NbPrep p, int64_t m,
                                                           int64_t k)
{
    const int64_t kts = p.kp / kNbK;
    const int64_t mt = blockIdx.x / kts, kt = blockIdx.x % kts;
    const int r = threadIdx.x >> 1, h = threadIdx.x & 1;
    const int64_t row = mt * kNbM + r, k0 = kt * kNbK + 8 * h;
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; e++)
        v[e] = (row < m && k0 + e < k) ? x[row * k + k0 + e] : 0.0f;
    uint32_t part[3][4];
    nb_split8(v, part);
    uint8_t *chunk = p.a + (size_t)blockIdx.x * kNbAChunk + r * 32 + 16 * nb_half(r, h);
#pragma unroll
    for (int pp = 0; pp < 3; pp++)
        *reinterpret_cast<u32x4 *>(chunk + pp * kNbPlane) = u32x4{part[pp][0], part[pp][1], part[pp][2], part[pp][3]};
}

// Whole-tile form (m % 128 == 0, k % 32 == 0): one workgroup per pair of
// chunks (128 rows x 32 k); thread (row r, half h) reads x[row][32 q + 16 h ..
// + 15] with four 16-byte loads (a thread pair covers the row's 128-byte
// line, where the form above splits it between two workgroups and loads it
// one float at a time) and writes both of its 8-activation halves to chunk
// 2 q + h, laid out as above.
__global__ __launch_bounds__(256) void nt_bf16_prep_full_kernel(const float *__restrict__ x, NbPrep p, int64_t k)
{
    const int64_t kts = p.kp / kNbK, pairs = kts / 2;
    const int64_t mt = blockIdx.x / pairs, q = blockIdx.x % pairs;
    const int r = threadIdx.x >> 1, h = threadIdx.x & 1;
    const float *src = x + (mt * kNbM + r) * k + 32 * q + 16 * h;
    float v[16];
#pragma unroll
    for (int c = 0; c < 4; c++) {
        const float4 f = *reinterpret_cast<const float4 *>(src + 4 * c);
        v[4 * c] = f.x; v[4 * c + 1] = f.y; v[4 * c + 2] = f.z; v[4 * c + 3] = f.w;
    }
    uint8_t *chunk = p.a + (size_t)(mt * kts + 2 * q + h) * kNbAChunk + r * 32;
#pragma unroll
    for (int hh = 0; hh < 2; hh++) {
        uint32_t part[3][4];
        nb_split8(v + 8 * hh, part);
#pragma unroll
        for (int pp = 0; pp < 3; pp++)
            *reinterpret_cast<u32x4 *>(chunk + 16 * nb_half(r, hh) + pp * kNbPlane) =
                u32x4{part[pp][0], part[pp][1], part[pp][2], part[pp][3]};
    }
}

template <int NJ, int NW>
struct NbLds {
    uint8_t a[kNbAChunk];
    uint8_t w[NW][NbCfg<NJ, NW>::WChunk];
};

__device__ __forceinline__ void nb_dma16(const void *base, uint32_t off, const QLL_LDS_NT void *lds)
{
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base),
                 "s"((uint32_t)(uintptr_t)lds)
                 : "memory", "m0");
}

// K step kt into buffer s: the activation chunk (12 KB, three 1 KB loads per
// wave) and the weight rows of each plane (32 bytes each, two lanes per row,
// 32 rows per load; rows past n load row n - 1, whose outputs are dropped).
// Plane ww starts at w + ww * plane bytes.
template <int NJ, int NW>
__device__ __forceinline__ void nb_load(const uint8_t *__restrict__ w, int64_t plane, const NbPrep &p, int64_t mt,
                                        int64_t n0, int64_t n, int64_t k, int64_t kt, NbLds<NJ, NW> &s)
{
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint8_t *ab = p.a + (mt * (p.kp / kNbK) + kt) * kNbAChunk;
    const QLL_LDS_NT char *as = (const QLL_LDS_NT char *)&s.a[0];
#pragma unroll
    for (int j = 0; j < 3; j++) {
        const int region = 3 * wave + j;
        nb_dma16(ab + region * 1024, 16u * lane, as + region * 1024);
    }
#pragma unroll
    for (int ww = 0; ww < NW; ww++)
#pragma unroll
        for (int j = 0; j < NJ / 2; j++) {
            const int q = wave * (NJ / 2) + j; // 32-row group
            const int row = 32 * q + (lane >> 1);
            const int64_t grow = n0 + row < n ? n0 + row : n - 1;
            const uint32_t off = (uint32_t)((grow - n0) * k * 2 + kt * 32 + 16 * nb_half(row, lane & 1));
            nb_dma16(w + ww * plane + n0 * k * 2, off, (const QLL_LDS_NT char *)&s.w[ww][0] + 1024 * q);
        }
}

template <int N>
__device__ __forceinline__ void nb_sync()
{
    __builtin_amdgcn_s_waitcnt((N & 0xf) | (0x7 << 4)); // vmcnt(N) expcnt(7) lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// blockIdx.y = split: K steps [split * per, min(kts, (split + 1) * per)),
// written to y + split * m * n (the workspace's partials when splitting).
template <int NJ, int NW>
__global__ __launch_bounds__(kNbThreads) void nt_bf16_gemm_kernel(const uint8_t *__restrict__ w, int64_t plane,
                                                                  NbPrep p, float *__restrict__ y, int64_t m,
                                                                  int64_t n, int64_t k, int64_t per)
{
    constexpr int BN = NbCfg<NJ, NW>::BN, DMA = NbCfg<NJ, NW>::Dma;
    __shared__ NbLds<NJ, NW> lds[kNbBuf];
    // consecutive workgroups share a weight tile (the row tiles of one column
    // tile run together and meet its weights in L2)
    const int64_t mtc = p.mp / kNbM;
    const int64_t mt = blockIdx.x % mtc, ntile = blockIdx.x / mtc;
    const int64_t m0 = mt * kNbM, n0 = ntile * BN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lr = lane & 31, lh = lane >> 5;
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 32 * NJ;
    const int64_t kts_all = p.kp / kNbK;
    const int64_t kb = (int64_t)blockIdx.y * per;
    const int64_t ke = kb + per < kts_all ? kb + per : kts_all;
    y += (int64_t)blockIdx.y * m * n;

    f32x16 acc[2][NJ];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < NJ; j++)
            acc[i][j] = f32x16{};

    // per-lane LDS offsets of the operands (rows of the wave's tiles)
    uint32_t ao[2], bo[NJ];
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int r = wm + 32 * i + lr;
        ao[i] = (uint32_t)(r * 32 + 16 * nb_half(r, lh));
    }
#pragma unroll
    for (int j = 0; j < NJ; j++) {
        const int c = wn + 32 * j + lr;
        using Lds = NbLds<NJ, NW>;
        bo[j] = (uint32_t)(offsetof(Lds, w) + c * 32 + 16 * nb_half(c, lh));
    }

    nb_load<NJ, NW>(w, plane, p, mt, n0, n, k, kb, lds[0]);
    nb_load<NJ, NW>(w, plane, p, mt, n0, n, k, kb + 1 < ke ? kb + 1 : ke - 1, lds[1]);
    nb_sync<DMA>();
    int cur = 0;
    for (int64_t kt = kb; kt < ke; kt++) {
        const int nx2 = cur == 0 ? 2 : cur - 1;
        // steps past the range reload its last one (never computed)
        nb_load<NJ, NW>(w, plane, p, mt, n0, n, k, kt + 2 < ke ? kt + 2 : ke - 1, lds[nx2]);
        const QLL_LDS_NT char *base = (const QLL_LDS_NT char *)&lds[cur];
        u32x4 a[2][3], b[NW][NJ];
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int pp = 0; pp < 3; pp++)
                a[i][pp] = *reinterpret_cast<const QLL_LDS_NT u32x4 *>(base + ao[i] + pp * kNbPlane);
#pragma unroll
        for (int ww = 0; ww < NW; ww++)
#pragma unroll
            for (int j = 0; j < NJ; j++)
                b[ww][j] = *reinterpret_cast<const QLL_LDS_NT u32x4 *>(base + bo[j] + ww * NbCfg<NJ, NW>::WChunk);
        // activation part pp against weight plane ww, for pp + ww <= 2: the
        // products left out (x3 w2 for f16 weights; x2 w3, x3 w2, x3 w3 for
        // f32 weights) are each at most 2^-27 of x * w, an eighth of one f32
        // rounding of the sum
#pragma unroll
        for (int ww = 0; ww < NW; ww++)
#pragma unroll
            for (int pp = 0; pp < 3 - ww; pp++)
#pragma unroll
                for (int i = 0; i < 2; i++)
#pragma unroll
                    for (int j = 0; j < NJ; j++)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[i][pp]),
                                                                             __builtin_bit_cast(bf16x8, b[ww][j]),
                                                                             acc[i][j], 0, 0, 0);
        nb_sync<DMA>();
        cur = cur == 2 ? 0 : cur + 1;
    }
    __builtin_amdgcn_s_waitcnt(0x7 << 4); // no load may still be writing this workgroup's LDS

#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < NJ; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const int64_t row = m0 + wm + 32 * i + 8 * (v >> 2) + 4 * lh + (v & 3);
                const int64_t col = n0 + wn + 32 * j + lr;
                if (row < m && col < n)
                    y[row * n + col] = acc[i][j][v];
            }
}

// The bf16 matrix-core path needs m > 1, k % 16 == 0 (weight rows then
// 32-byte aligned and the K steps whole) and k < 2^23.
bool gemm_nt_bf16_core_shape(int64_t m, int64_t k)
{
    return m > 1 && k % 16 == 0 && k < ((int64_t)1 << 23);
}

// 256-column tiles (one 64 x 128 tile per wave) when they still give two
// workgroups per CU and there is one weight plane, else 128-column tiles (two
// planes of 256-column tiles would leave room for one workgroup per CU); K is
// split (partials summed in a fixed order by a second kernel) while the tiles
// leave workgroup slots idle (two per CU), each split keeping at least 32 K
// steps.  Workspace: the split activations, the two weight planes (f16
// weights), then the partials.
struct NbPlan {
    int nj, nw, splits;
    int64_t mp, per, tiles;
    size_t w_off, parts_off, total;
};

static NbPlan nb_plan(int64_t m, int64_t n, int64_t k, int nw)
{
    NbPlan p;
    p.nw = nw;
    p.mp = (m + kNbM - 1) / kNbM * kNbM;
    const int64_t mt = p.mp / kNbM, kts = k / kNbK;
    const int64_t tiles4 = mt * ((n + 255) / 256);
    p.nj = nw == 1 && tiles4 >= 512 ? 4 : 2;
    p.tiles = p.nj == 4 ? tiles4 : mt * ((n + 127) / 128);
    int64_t splits = 512 / p.tiles;
    if (splits > kts / 32)
        splits = kts / 32;
    if (splits > 8)
        splits = 8;
    if (splits < 2)
        splits = 1;
    p.per = (kts + splits - 1) / splits;
    p.splits = (int)((kts + p.per - 1) / p.per);
    auto up = [](size_t v) { return (v + 255) / 256 * 256; };
    p.w_off = up((size_t)mt * (size_t)kts * kNbAChunk);
    p.parts_off = p.w_off + (nw > 1 ? up((size_t)nw * (size_t)n * (size_t)k * 2) : 0);
    p.total = p.parts_off + (p.splits > 1 ? up((size_t)p.splits * (size_t)(m * n) * sizeof(float)) : 0);
    return p;
}

static int nb_planes(int wfmt) { return wfmt == QLL_W_BF16 ? 1 : wfmt == QLL_W_F16 ? 2 : 3; }

size_t gemm_nt_workspace(int wfmt, int64_t m, int64_t n, int64_t k)
{
    if (!gemm_nt_bf16_core_shape(m, k))
        return 0;
    return nb_plan(m, n, k, nb_planes(wfmt)).total;
}

// Weights -> NW bf16 planes whose sum is the weight exactly.  f16 (NW = 2):
// the first part keeps 8 of the 11 significant bits, the rest (at most 4 bits,
// within bf16's exponent range since f16's is narrower) is the second.  f32
// (NW = 3): 8 + 8 + 8 of the 24 bits, as for the activations.  Eight weights
// per thread.
template <int NW>
__global__ __launch_bounds__(256) void nt_w_split_kernel(const void *__restrict__ w, uint8_t *__restrict__ planes,
                                                         int64_t plane, int64_t count8)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= count8)
        return;
    float f[8];
    if (NW == 2) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(w) + 8 * i);
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const uint32_t word = v[e];
            f[2 * e] = half_bits_to_float(word & 0xffffu);
            f[2 * e + 1] = half_bits_to_float(word >> 16);
        }
    } else {
        const float *src = static_cast<const float *>(w) + 8 * i;
        const float4 a = *reinterpret_cast<const float4 *>(src), b = *reinterpret_cast<const float4 *>(src + 4);
        f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
        f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
    }
    uint32_t out[NW][4];
#pragma unroll
    for (int e = 0; e < 4; e++) {
        uint32_t b[NW][2];
#pragma unroll
        for (int q = 0; q < 2; q++) {
            float r = f[2 * e + q];
#pragma unroll
            for (int pp = 0; pp < NW; pp++) {
                b[pp][q] = bf16_bits(r);
                r -= __builtin_bit_cast(float, b[pp][q] << 16); // exact
            }
        }
#pragma unroll
        for (int pp = 0; pp < NW; pp++)
            out[pp][e] = b[pp][0] | (b[pp][1] << 16);
    }
#pragma unroll
    for (int pp = 0; pp < NW; pp++)
        *reinterpret_cast<u32x4 *>(planes + pp * plane + 16 * i) = u32x4{out[pp][0], out[pp][1], out[pp][2], out[pp][3]};
}

// The plain orientation's B[k][n] (f32) -> three bf16 planes laid out as
// W[n][k] = B^T, split like nt_w_split_kernel<3>.  64 x 64 tiles through LDS:
// rows of B are read 16 bytes per thread along n, and each thread writes 16
// consecutive k of one output row per plane (32 bytes, four threads per row).
__global__ __launch_bounds__(256) void nn_b_split_t_kernel(const float *__restrict__ b, uint8_t *__restrict__ planes,
                                                           int64_t plane, int64_t n, int64_t k)
{
    __shared__ float t[64][65];
    const int64_t n0 = (int64_t)blockIdx.x * 64, k0 = (int64_t)blockIdx.y * 64;
    const int tid = threadIdx.x;
#pragma unroll
    for (int it = 0; it < 4; it++) {
        const int r = (tid >> 4) + 16 * it, c = 4 * (tid & 15);
        const int64_t kr = k0 + r, nc = n0 + c;
        float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (kr < k) {
            if (nc + 3 < n && n % 4 == 0) {
                const float4 f = *reinterpret_cast<const float4 *>(b + kr * n + nc);
                v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
            } else {
#pragma unroll
                for (int e = 0; e < 4; e++)
                    v[e] = nc + e < n ? b[kr * n + nc + e] : 0.0f;
            }
        }
#pragma unroll
        for (int e = 0; e < 4; e++)
            t[r][c + e] = v[e];
    }
    __syncthreads();
    const int nr = tid >> 2, kq = 16 * (tid & 3);
    const int64_t row = n0 + nr, kk = k0 + kq;
    if (row >= n || kk >= k) // k is a multiple of 16, so a 16-wide piece is whole
        return;
    uint32_t out[3][8];
#pragma unroll
    for (int e = 0; e < 8; e++) {
        uint32_t bb[3][2];
#pragma unroll
        for (int q = 0; q < 2; q++) {
            float r = t[kq + 2 * e + q][nr];
#pragma unroll
            for (int pp = 0; pp < 3; pp++) {
                bb[pp][q] = bf16_bits(r);
                r -= __builtin_bit_cast(float, bb[pp][q] << 16); // exact
            }
        }
#pragma unroll
        for (int pp = 0; pp < 3; pp++)
            out[pp][e] = bb[pp][0] | (bb[pp][1] << 16);
    }
#pragma unroll
    for (int pp = 0; pp < 3; pp++) {
        uint8_t *dst = planes + pp * plane + (row * k + kk) * 2;
        *reinterpret_cast<u32x4 *>(dst) = u32x4{out[pp][0], out[pp][1], out[pp][2], out[pp][3]};
        *reinterpret_cast<u32x4 *>(dst + 16) = u32x4{out[pp][4], out[pp][5], out[pp][6], out[pp][7]};
    }
}

// b_kn: w is the plain orientation's B[k][n] (f32), transposed by the split.
hipError_t launch_gemm_nt_bf16_mfma(const float *x, const void *w, int wfmt, float *y, int64_t m, int64_t n,
                                    int64_t k, void *ws, hipStream_t s, bool b_kn)
{
    const NbPlan plan = nb_plan(m, n, k, nb_planes(wfmt));
    NbPrep p;
    p.a = static_cast<uint8_t *>(ws);
    p.mp = plan.mp;
    p.kp = k;
    const int64_t chunks = (p.mp / kNbM) * (k / kNbK);
    const int64_t count8 = n * k / 8;
    if (chunks > 0x7fffffff || plan.tiles > 0x7fffffff || (count8 + 255) / 256 > 0x7fffffff ||
        (b_kn && ((n + 63) / 64 > 0x7fffffff || (k + 63) / 64 > 65535)))
        return hipErrorInvalidConfiguration;
    if (m % kNbM == 0 && k % (2 * kNbK) == 0)
        hipLaunchKernelGGL(nt_bf16_prep_full_kernel, dim3((unsigned)(chunks / 2)), dim3(256), 0, s, x, p, k);
    else
        hipLaunchKernelGGL(nt_bf16_prep_kernel, dim3((unsigned)chunks), dim3(256), 0, s, x, p, m, k);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const uint8_t *wb = static_cast<const uint8_t *>(w);
    int64_t plane = 0;
    if (plan.nw > 1) {
        uint8_t *planes = static_cast<uint8_t *>(ws) + plan.w_off;
        plane = n * k * 2;
        const dim3 g((unsigned)((count8 + 255) / 256));
        if (b_kn)
            hipLaunchKernelGGL(nn_b_split_t_kernel, dim3((unsigned)((n + 63) / 64), (unsigned)((k + 63) / 64)),
                               dim3(256), 0, s, static_cast<const float *>(w), planes, plane, n, k);
        else if (plan.nw == 2)
            hipLaunchKernelGGL(nt_w_split_kernel<2>, g, dim3(256), 0, s, w, planes, plane, count8);
        else
            hipLaunchKernelGGL(nt_w_split_kernel<3>, g, dim3(256), 0, s, w, planes, plane, count8);
        e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        wb = planes;
    }
    float *out = plan.splits > 1 ? reinterpret_cast<float *>(static_cast<uint8_t *>(ws) + plan.parts_off) : y;
    const dim3 grid((unsigned)plan.tiles, (unsigned)plan.splits);
    if (plan.nw == 3)
        hipLaunchKernelGGL((nt_bf16_gemm_kernel<2, 3>), grid, dim3(kNbThreads), 0, s, wb, plane, p, out, m, n, k,
                           plan.per);
    else if (plan.nw == 2)
        hipLaunchKernelGGL((nt_bf16_gemm_kernel<2, 2>), grid, dim3(kNbThreads), 0, s, wb, plane, p, out, m, n, k,
                           plan.per);
    else if (plan.nj == 4)
        hipLaunchKernelGGL((nt_bf16_gemm_kernel<4, 1>), grid, dim3(kNbThreads), 0, s, wb, plane, p, out, m, n, k,
                           plan.per);
    else
        hipLaunchKernelGGL((nt_bf16_gemm_kernel<2, 1>), grid, dim3(kNbThreads), 0, s, wb, plane, p, out, m, n, k,
                           plan.per);
    e = hipGetLastError();
    if (e != hipSuccess || plan.splits == 1)
        return e;
    return launch_sum_splits(out, y, m * n, plan.splits, s);
}

hipError_t launch_gemv_nt(const float *x, const void *w, int wfmt, float *y, int64_t n, int64_t k, hipStream_t s)
{
    const uint8_t *wb = static_cast<const uint8_t *>(w);
    if (wfmt == QLL_W_F32)
        return launch_nt<QLL_W_F32>(x, wb, y, n, k, s);
    if (wfmt == QLL_W_BF16)
        return launch_nt<QLL_W_BF16>(x, wb, y, n, k, s);
    return launch_nt<QLL_W_F16>(x, wb, y, n, k, s);
}

} // namespace qll
