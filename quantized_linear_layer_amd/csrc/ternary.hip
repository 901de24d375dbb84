// BitNet ternary linear layer (Loom "Plan 9 SIMD Forward", "BitNet ternary
// MAD kernel"): weights in {-1, 0, +1} stored as 2-bit codes c = w + 1, 16 per
// uint32; int8 activations with act_scale = 127 / max|x| per row; the dot
// uses the ternary identity
//     sum_t (c_t - 1) q_t = sum_t c_t q_t - sum_t q_t,
// with sum_t q_t (act_sum) computed once per activation row, and the output
// is dot * w_scale / act_scale.
//
// Unlike the page's CPU design (a byte-per-weight code cache built once), the
// codes are unpacked in registers on every call, so W is read at 2 bits per
// weight: (word >> 2j) & 0x03030303 puts codes j, 4+j, 8+j, 12+j of the word
// into the four bytes of a dword.  The activation bytes are transposed to the
// same order once per workgroup when they are staged in LDS, and
// v_dot4_i32_i8 multiplies the two (codes are 0..2, valid signed bytes).
#include "common.h"

namespace qll {

#define QLL_LDS_T __attribute__((address_space(3)))

// 16 activation bytes (dwords D0..D3, byte e of Dr = x[4r + e]) -> A0..A3 with
// byte r of Aj = x[4r + j], the order of the code unpack: a 4x4 byte transpose
// in two rounds of byte permutes (interleave pairs of dwords, then pairs of
// halves).
__device__ __forceinline__ u32x4 transpose_4x4_bytes(u32x4 d)
{
    const uint32_t p0 = __builtin_amdgcn_perm(d[1], d[0], 0x05010400u); // D0.b0 D1.b0 D0.b1 D1.b1
    const uint32_t p1 = __builtin_amdgcn_perm(d[1], d[0], 0x07030602u); // D0.b2 D1.b2 D0.b3 D1.b3
    const uint32_t p2 = __builtin_amdgcn_perm(d[3], d[2], 0x05010400u);
    const uint32_t p3 = __builtin_amdgcn_perm(d[3], d[2], 0x07030602u);
    return u32x4{__builtin_amdgcn_perm(p2, p0, 0x05040100u), __builtin_amdgcn_perm(p2, p0, 0x07060302u),
                 __builtin_amdgcn_perm(p3, p1, 0x05040100u), __builtin_amdgcn_perm(p3, p1, 0x07060302u)};
}

__device__ __forceinline__ int ternary_word_dot(uint32_t word, u32x4 a, int acc)
{
    acc = sdot4(word & 0x03030303u, a[0], acc);
    acc = sdot4((word >> 2) & 0x03030303u, a[1], acc);
    acc = sdot4((word >> 4) & 0x03030303u, a[2], acc);
    acc = sdot4((word >> 6) & 0x03030303u, a[3], acc);
    return acc;
}

__device__ __forceinline__ float ternary_output(int dot_c, int asum, float w_scale, float s)
{
    if (s == 0.0f)
        return 0.0f;
    return (float)(dot_c - asum) * w_scale / s;
}

constexpr int kTerGemvThreads = 64;
constexpr int kTerUnroll = 8;

// m = 1.  VEC: 4 words (one dwordx4) per unit when k % 64 == 0, else 1 word.
// Each lane issues the weight loads of its first row group before the
// activation staging, so the two memory round trips overlap.
template <int L, int VEC>
__global__ __launch_bounds__(kTerGemvThreads) void ternary_gemv_kernel(
    const uint32_t *__restrict__ w, float w_scale, const int8_t *__restrict__ xq, const float *__restrict__ act_scale,
    const int32_t *__restrict__ act_sum, float *__restrict__ y, int64_t n, int nw)
{
    extern __shared__ u32x4 s_x[]; // [nw] transposed activation words
    constexpr int R = 64 / L;
    constexpr int WAVES = kTerGemvThreads / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane / L, r = lane % L;
    const int nu = nw / VEC;
    const int64_t stride = (int64_t)gridDim.x * WAVES * R;
    int64_t row0 = ((int64_t)blockIdx.x * WAVES + wave) * R;

    // first kTerUnroll units of this lane's first row, in flight during the staging
    uint32_t pre[kTerUnroll][VEC];
    {
        const int64_t row = row0 + g;
        const uint32_t *wr = w + (row < n ? row : 0) * nw;
#pragma unroll
        for (int i = 0; i < kTerUnroll; i++) {
            const int u = r + i * L;
            const int uc = u < nu ? u : 0;
            if (VEC == 4) {
                const u32x4 v = reinterpret_cast<const u32x4 *>(wr)[uc];
#pragma unroll
                for (int e = 0; e < VEC; e++)
                    pre[i][e] = v[e];
            } else {
                pre[i][0] = wr[uc];
            }
        }
    }
    // activation staging: all of a lane's loads first, then the transposes
    {
        constexpr int kStage = 8; // words per lane per round (k up to 8192 in one round)
        for (int i0 = threadIdx.x; i0 < nw; i0 += kStage * kTerGemvThreads) {
            u32x4 t[kStage];
#pragma unroll
            for (int j = 0; j < kStage; j++) {
                const int i = i0 + j * kTerGemvThreads;
                t[j] = reinterpret_cast<const u32x4 *>(xq)[i < nw ? i : 0];
            }
#pragma unroll
            for (int j = 0; j < kStage; j++) {
                const int i = i0 + j * kTerGemvThreads;
                if (i < nw)
                    s_x[i] = transpose_4x4_bytes(t[j]);
            }
        }
    }
    __syncthreads();

    const float s = act_scale[0];
    const int asum = act_sum[0];
    bool first = true;
    for (; row0 < n; row0 += stride) {
        const int64_t row = row0 + g;
        int acc = 0;
        if (row < n) {
            const uint32_t *wr = w + row * nw;
            for (int u0 = r; u0 < nu; u0 += kTerUnroll * L) {
                uint32_t wd[kTerUnroll][VEC];
#pragma unroll
                for (int i = 0; i < kTerUnroll; i++) {
                    const int u = u0 + i * L;
                    if (first && u0 == r) {
#pragma unroll
                        for (int e = 0; e < VEC; e++)
                            wd[i][e] = pre[i][e];
                    } else if (u < nu) {
                        if (VEC == 4) {
                            u32x4 v = reinterpret_cast<const u32x4 *>(wr)[u];
#pragma unroll
                            for (int e = 0; e < VEC; e++)
                                wd[i][e] = v[e];
                        } else {
                            wd[i][0] = wr[u];
                        }
                    }
                }
#pragma unroll
                for (int i = 0; i < kTerUnroll; i++) {
                    const int u = u0 + i * L;
                    if (u < nu) {
#pragma unroll
                        for (int e = 0; e < VEC; e++)
                            acc = ternary_word_dot(wd[i][e], s_x[u * VEC + e], acc);
                    }
                }
            }
        }
        first = false;
#pragma unroll
        for (int off = L / 2; off > 0; off >>= 1)
            acc += __shfl_xor(acc, off);
        if (row < n && r == 0)
            y[row] = ternary_output(acc, asum, w_scale, s);
    }
}

template <int L, int VEC>
static hipError_t launch_ter_l(const uint32_t *w, float w_scale, const int8_t *xq, const float *act_scale,
                               const int32_t *act_sum, float *y, int64_t n, int nw, hipStream_t st)
{
    constexpr int R = 64 / L;
    const int64_t waves = (n + R - 1) / R;
    int64_t grid = (waves + kTerGemvThreads / 64 - 1) / (kTerGemvThreads / 64);
    if (grid > 16384)
        grid = 16384;
    hipLaunchKernelGGL((ternary_gemv_kernel<L, VEC>), dim3((unsigned)grid), dim3(kTerGemvThreads),
                       (size_t)nw * 16, st, w, w_scale, xq, act_scale, act_sum, y, n, nw);
    return hipGetLastError();
}

// m = 1, k % 64 == 0: 256-thread workgroups, so the activation staging is
// shared by four waves and each lane transposes at most a few 16-byte
// pieces.  Per lane, in issue order: its activation pieces (so that waiting
// for them does not wait for the weights: loads retire in order), the
// weight units of its first chunk, then the transposes into LDS while the
// weights are in flight.  L lanes per row (R = 64 / L rows per wave), U
// units of four words per lane and chunk; the next chunk's weights are
// loaded while the current one is dotted, into four independent
// accumulators (one per dword of a word's activation) rather than one chain.
constexpr int kTg2Threads = 256;
constexpr int kTg2ActRegs = 4; // activation pieces per thread held in registers (k <= 16384)

template <int L, int U>
__global__ __launch_bounds__(kTg2Threads) void ternary_gemv2_kernel(
    const uint32_t *__restrict__ w, float w_scale, const int8_t *__restrict__ xq, const float *__restrict__ act_scale,
    const int32_t *__restrict__ act_sum, float *__restrict__ y, int64_t n, int nw)
{
    // transposed activation words, word 4u + e at [e][u]: the lanes of a row
    // read consecutive 16-byte slots (with [4u + e] they were 64 bytes apart:
    // 6.7 bank-conflict cycles per read; 3.11 -> 3.04 us at 2560 -> 6912)
    extern __shared__ u32x4 s_x[];
    constexpr int R = 64 / L, WAVES = kTg2Threads / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane / L, r = lane % L;
    const int nu = nw / 4;
    const int chunk = U * L, chunks = (nu + chunk - 1) / chunk;
    const int64_t row = ((int64_t)blockIdx.x * WAVES + wave) * R + g;
    const u32x4 *wr = reinterpret_cast<const u32x4 *>(w + (row < n ? row : 0) * nw);
    const u32x4 *xv = reinterpret_cast<const u32x4 *>(xq);
    const float s = act_scale[0];
    const int asum = act_sum[0];

    u32x4 a[kTg2ActRegs];
#pragma unroll
    for (int j = 0; j < kTg2ActRegs; j++) {
        const int i = threadIdx.x + j * kTg2Threads;
        // unconditional (waits stay countable); pieces past the row reload
        // word i % nw rather than all word 0: 3.64 against 3.83 us at 2560 -> 6912
        a[j] = xv[i < nw ? i : i % nw];
    }
    asm volatile("" ::: "memory"); // the activation loads go out first

    u32x4 cur[U], nxt[U];
    const auto load = [&](u32x4 (&d)[U], int c) {
#pragma unroll
        for (int i = 0; i < U; i++) {
            const int u = c * chunk + r + i * L;
            d[i] = wr[u < nu ? u : 0];
        }
    };
    load(cur, 0);

#pragma unroll
    for (int j = 0; j < kTg2ActRegs; j++) {
        const int i = threadIdx.x + j * kTg2Threads;
        if (i < nw)
            s_x[(i & 3) * nu + (i >> 2)] = transpose_4x4_bytes(a[j]);
    }
    for (int i = threadIdx.x + kTg2ActRegs * kTg2Threads; i < nw; i += kTg2Threads)
        s_x[(i & 3) * nu + (i >> 2)] = transpose_4x4_bytes(xv[i]);
    __syncthreads();

    int acc[4] = {0, 0, 0, 0};
    for (int c = 0; c < chunks; c++) {
        if (c + 1 < chunks)
            load(nxt, c + 1);
#pragma unroll
        for (int i = 0; i < U; i++) {
            const int u = c * chunk + r + i * L;
            if (u < nu) {
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const u32x4 t = s_x[e * nu + u];
                    const uint32_t word = cur[i][e];
                    acc[0] = sdot4(word & 0x03030303u, t[0], acc[0]);
                    acc[1] = sdot4((word >> 2) & 0x03030303u, t[1], acc[1]);
                    acc[2] = sdot4((word >> 4) & 0x03030303u, t[2], acc[2]);
                    acc[3] = sdot4((word >> 6) & 0x03030303u, t[3], acc[3]);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < U; i++)
            cur[i] = nxt[i];
    }
    int dot = (acc[0] + acc[1]) + (acc[2] + acc[3]);
#pragma unroll
    for (int off = L / 2; off > 0; off >>= 1)
        dot += __shfl_xor(dot, off);
    if (row < n && r == 0)
        y[row] = ternary_output(dot, asum, w_scale, s);
}

template <int L, int U>
static hipError_t launch_tg2(const uint32_t *w, float w_scale, const int8_t *xq, const float *act_scale,
                             const int32_t *act_sum, float *y, int64_t n, int nw, hipStream_t st)
{
    constexpr int R = 64 / L, RPW = R * (kTg2Threads / 64);
    const int64_t grid = (n + RPW - 1) / RPW;
    if (grid > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((ternary_gemv2_kernel<L, U>), dim3((unsigned)grid), dim3(kTg2Threads), (size_t)nw * 16, st, w,
                       w_scale, xq, act_scale, act_sum, y, n, nw);
    return hipGetLastError();
}

template <int VEC>
static hipError_t launch_ter_vec(const uint32_t *w, float w_scale, const int8_t *xq, const float *act_scale,
                                 const int32_t *act_sum, float *y, int64_t n, int nw, hipStream_t st)
{
    const int nu = nw / VEC;
    if (nu >= 256)
        return launch_ter_l<64, VEC>(w, w_scale, xq, act_scale, act_sum, y, n, nw, st);
    if (nu >= 128)
        return launch_ter_l<32, VEC>(w, w_scale, xq, act_scale, act_sum, y, n, nw, st);
    if (nu >= 64)
        return launch_ter_l<16, VEC>(w, w_scale, xq, act_scale, act_sum, y, n, nw, st);
    return launch_ter_l<8, VEC>(w, w_scale, xq, act_scale, act_sum, y, n, nw, st);
}

hipError_t launch_ternary_gemv(const uint32_t *w, float w_scale, const int8_t *xq, const float *act_scale,
                               const int32_t *act_sum, float *y, int64_t n, int64_t k, hipStream_t st)
{
    const int nw = (int)(k / 16);
    if (nw % 4 == 0) {
        // units of four words per row, about three per lane (2560 -> 6912:
        // 16 lanes x 3 units 3.9 us; 32 x 2 4.1, 64 x 1 4.4, 8 x 5 4.0,
        // 16 x 4 4.0, 8 x 8 4.2)
        const int nu = nw / 4;
        if (nu > 96)
            return launch_tg2<64, 3>(w, w_scale, xq, act_scale, act_sum, y, n, nw, st);
        if (nu > 48)
            return launch_tg2<32, 3>(w, w_scale, xq, act_scale, act_sum, y, n, nw, st);
        if (nu > 24)
            return launch_tg2<16, 3>(w, w_scale, xq, act_scale, act_sum, y, n, nw, st);
        return launch_tg2<8, 3>(w, w_scale, xq, act_scale, act_sum, y, n, nw, st);
    }
    return launch_ter_vec<1>(w, w_scale, xq, act_scale, act_sum, y, n, nw, st);
}

// ------------------------------------------------------------------ GEMM (m > 1), any k
// The general kernel (k % 64 != 0, or operands beyond 32-bit offsets; the
// k-split kernel further down takes the rest).
// v_mfma_i32_16x16x64_i8: one MFMA covers 64 codes = 4 weight words.  The
// k range is walked in chunks of kTerKC codes (32 words).  Within a chunk,
// lane group h of an operand (lanes 16h..16h+15) takes words 8h..8h+7 in
// successive k-steps, so a lane's weight words are contiguous (two 16-byte
// loads per chunk) and the activation bytes of the same words, transposed
// like the code unpack, are its A operand.  Words past the end of the row
// meet zero activation, so the codes there do not matter.
// Workgroup tile: 64 activation rows x 32 weight rows; wave w owns rows
// 16w..16w+15 and both 16-column halves.  The activation chunk (64 rows x
// 512 bytes) is loaded with consecutive lanes on consecutive 16-byte pieces
// of a row and double buffered in LDS; rows are padded by 16 bytes so the 16
// rows read by one MFMA operand fall in distinct banks.

constexpr int TBM = 64, TBN = 32, kTerKC = 512, kTerWPC = kTerKC / 16; // words per chunk
constexpr int kTerGemmThreads = 256;
constexpr int kTerPieces = TBM * kTerWPC / kTerGemmThreads;             // 16-byte pieces per thread

struct TerStage {
    u32x4 x[kTerPieces];
    uint32_t w[2][8];
};

template <bool VEC>
__device__ __forceinline__ void ternary_gemm_load(const uint32_t *__restrict__ w, const int8_t *__restrict__ xq,
                                                  int64_t m, int64_t n, int nw, int64_t m0, int64_t n0, int chunk,
                                                  TerStage &st)
{
    const int lane = threadIdx.x & 63;
    const int lr = lane & 15, lh = lane >> 4;
#pragma unroll
    for (int i = 0; i < kTerPieces; i++) {
        const int piece = threadIdx.x + i * kTerGemmThreads;
        const int row = piece / kTerWPC, word = chunk * kTerWPC + piece % kTerWPC;
        const int64_t gi = m0 + row;
        st.x[i] = (gi < m && word < nw)
                      ? *reinterpret_cast<const u32x4 *>(xq + gi * (int64_t)nw * 16 + (int64_t)word * 16)
                      : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < 2; j++) {
        const int64_t col = n0 + 16 * j + lr;
        const int word0 = chunk * kTerWPC + 8 * lh;
        const uint32_t *wr = w + col * nw;
        if (VEC && col < n && word0 + 8 <= nw) {
            const u32x4 a = *reinterpret_cast<const u32x4 *>(wr + word0);
            const u32x4 b = *reinterpret_cast<const u32x4 *>(wr + word0 + 4);
#pragma unroll
            for (int e = 0; e < 4; e++) {
                st.w[j][e] = a[e];
                st.w[j][4 + e] = b[e];
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; e++)
                st.w[j][e] = (col < n && word0 + e < nw) ? wr[word0 + e] : 0u;
        }
    }
}

template <bool VEC>
__global__ __launch_bounds__(kTerGemmThreads) void ternary_gemm_kernel(
    const uint32_t *__restrict__ w, float w_scale, const int8_t *__restrict__ xq, const float *__restrict__ act_scale,
    const int32_t *__restrict__ act_sum, float *__restrict__ y, int64_t m, int64_t n, int nw)
{
    __shared__ u32x4 xs[2][TBM][kTerWPC + 1];
    const int64_t m0 = (int64_t)blockIdx.y * TBM, n0 = (int64_t)blockIdx.x * TBN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lr = lane & 15, lh = lane >> 4;
    const int nchunks = (nw + kTerWPC - 1) / kTerWPC;

    i32x4 acc[2] = {i32x4{0, 0, 0, 0}, i32x4{0, 0, 0, 0}};
    TerStage st;
    ternary_gemm_load<VEC>(w, xq, m, n, nw, m0, n0, 0, st);
    for (int c = 0; c < nchunks; c++) {
        const int buf = c & 1;
#pragma unroll
        for (int i = 0; i < kTerPieces; i++) {
            const int piece = threadIdx.x + i * kTerGemmThreads;
            xs[buf][piece / kTerWPC][piece % kTerWPC] = transpose_4x4_bytes(st.x[i]);
        }
        uint32_t wcur[2][8];
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int e = 0; e < 8; e++)
                wcur[j][e] = st.w[j][e];
        __syncthreads();
        if (c + 1 < nchunks)
            ternary_gemm_load<VEC>(w, xq, m, n, nw, m0, n0, c + 1, st);
#pragma unroll
        for (int s = 0; s < 8; s++) {
            const i32x4 a = __builtin_bit_cast(i32x4, xs[buf][16 * wave + lr][8 * lh + s]);
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const uint32_t cw = wcur[j][s];
                const i32x4 b = {(int)(cw & 0x03030303u), (int)((cw >> 2) & 0x03030303u),
                                 (int)((cw >> 4) & 0x03030303u), (int)((cw >> 6) & 0x03030303u)};
                acc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[j], 0, 0, 0);
            }
        }
    }
    // D layout of a 16x16 tile: lane l, register v -> row 4*(l/16)+v, column l%16
#pragma unroll
    for (int v = 0; v < 4; v++) {
        const int64_t row = m0 + 16 * wave + 4 * lh + v;
        if (row >= m)
            continue;
        const float s = act_scale[row];
        const int asum = act_sum[row];
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int64_t col = n0 + 16 * j + lr;
            if (col < n)
                y[row * n + col] = ternary_output(acc[j][v], asum, w_scale, s);
        }
    }
}

// ------------------------------------------------------------------ GEMM, k % 64 == 0
// At the workload's size (m = 64, 4.4 MB of weights, 2.3 GOP) the GEMM is
// bound neither by bytes nor by the matrix core but by each SIMD's
// instruction stream and by memory round trips, so this kernel spends few
// instructions per multiply-add and spreads k over the waves:
//   * 32x32x32 int8 MFMA.  Per instruction a lane brings 16 activation bytes
//     (one code word's worth, transposed into the unpack order) and one
//     code word, so each transposed activation fragment feeds two MFMAs of
//     32K multiply-adds (the wave's two 32-row weight groups) and each
//     unpacked word a 32-row product.
//   * Tile 32 activation rows x 64 weight rows per workgroup; the row's
//     32-word chunks (512 codes) are dealt round-robin to its KS waves,
//     each with its own LDS region; the exact int32 partial tiles are added
//     in LDS in a fixed order at the end, so the result does not depend on
//     KS.  KS is chosen so that the grid has about a wave per SIMD.
//   * Operands go memory -> LDS by 16-byte DMA (global_load_lds), coalesced
//     in 128-byte runs; per-lane loads of the MFMA fragments themselves
//     would touch 64 cache lines per instruction.  Lane (r, h) at step s
//     takes word 16h + s of the chunk, so half p of the chunk (steps 8p ..
//     8p + 7) is words 8p .. 8p + 7 and 16 + 8p .. 16 + 8p + 7 of each row:
//     both halves are requested at once and the first is dotted while the
//     second lands.  The lane offsets (row, slot swizzle, clamps for ragged
//     m and n) are computed once; chunk and half enter only through the
//     scalar base address.
//   * LDS slot swizzles: activation slot ^ (row & 15) and code group ^
//     ((row >> 2) & 3), so the 16 rows one fragment read touches fall in
//     distinct banks.
// Words past the end of a row (a partial last chunk) are loaded from
// clamped addresses and their code word is zeroed: code 0 adds nothing to
// sum c q, and act_sum counts the row's real words only.
__device__ __forceinline__ void ter_dma16(const void *base, uint32_t off, const QLL_LDS_T void *lds)
{
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base),
                 "s"((uint32_t)(uintptr_t)lds)
                 : "memory", "m0");
}

// Wait until at most N vector-memory operations of this wave are
// outstanding (and all LDS operations have completed).
template <int N>
__device__ __forceinline__ void ter_wait()
{
    static_assert(N < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | (0x7 << 4)); // vmcnt(N) expcnt(7) lgkmcnt(0)
    asm volatile("" ::: "memory");
}

constexpr int kTerKsRows = 32, kTerKsCols = 64, kTerKsMaxSplit = 6; // 24 KB of LDS per wave
constexpr int64_t kTerKsTargetWaves = 1024;

struct TerKsLds {
    u32x4 x[2][kTerKsRows][16]; // [half][row][slot]: slot ^ (row & 15) = 8 hh + s8 -> word 32c + 16 hh + 8 half + s8
    u32x4 w[2][kTerKsCols][4];  // [half][row][group]: group ^ ((row >> 2) & 3) = 2 hh + g2 -> words 32c + 16 hh + 8 half + 4 g2 ..
};

struct TerKsOff {
    uint32_t x[8]; // byte offset of the lane's 16 bytes in activation load q (rows 4q .. 4q + 3), first half of chunk 0
    uint32_t w[4]; // the same for code load q (rows 16q .. 16q + 15)
};

__device__ __forceinline__ void ter_ks_offsets(int64_t m, int64_t n, int nw, int64_t m0, int64_t n0, TerKsOff &o)
{
    const int lane = threadIdx.x & 63;
    // m * k and n * k / 4 are below 2^32 - 4096 (checked at launch)
    const uint32_t xrow = (uint32_t)nw * 16u, wrow = (uint32_t)nw * 4u;
#pragma unroll
    for (int q = 0; q < 8; q++) { // 16 lanes per row
        const int row = 4 * q + (lane >> 4), lam = (lane & 15) ^ (row & 15);
        const uint32_t gi = (uint32_t)(m0 + row < m ? m0 + row : m - 1);
        o.x[q] = gi * xrow + (uint32_t)(16 * (lam >> 3) + (lam & 7)) * 16u;
    }
#pragma unroll
    for (int q = 0; q < 4; q++) { // 4 lanes per row
        const int row = 16 * q + (lane >> 2), gam = (lane & 3) ^ ((row >> 2) & 3);
        const uint32_t gj = (uint32_t)(n0 + row < n ? n0 + row : n - 1);
        o.w[q] = gj * wrow + (uint32_t)(16 * (gam >> 1) + 4 * (gam & 1)) * 4u;
    }
}

// Half p of chunk c into s.  FULL: the chunk lies in the row; the half's
// first word goes into the scalar base and the lane offsets are used as they
// are.  Otherwise (the row's last, partial chunk) each word is clamped to the
// row and addressed from the tensor's base: a clamped word can precede the
// half's first word, and the hardware adds the 32-bit lane offset unsigned.
template <bool FULL>
__device__ __forceinline__ void ter_ks_load(const uint32_t *__restrict__ w, const int8_t *__restrict__ xq, int nw,
                                            int c, int p, const TerKsOff &o, TerKsLds &s)
{
    const int lane = threadIdx.x & 63;
    const int w0 = 32 * c + 8 * p; // first word of the half's first run
    const QLL_LDS_T char *xs = (const QLL_LDS_T char *)&s.x[p][0][0];
    const QLL_LDS_T char *ws = (const QLL_LDS_T char *)&s.w[p][0][0];
#pragma unroll
    for (int q = 0; q < 8; q++) {
        if (FULL) {
            ter_dma16(xq + (int64_t)w0 * 16, o.x[q], xs + 1024 * q);
        } else {
            const int lam = (lane & 15) ^ ((4 * q + (lane >> 4)) & 15);
            const int rel = 16 * (lam >> 3) + (lam & 7); // word within the half's runs
            const int word = w0 + rel < nw ? w0 + rel : nw - 1;
            ter_dma16(xq, o.x[q] - (uint32_t)rel * 16u + (uint32_t)word * 16u, xs + 1024 * q);
        }
    }
#pragma unroll
    for (int q = 0; q < 4; q++) {
        if (FULL) {
            ter_dma16(w + w0, o.w[q], ws + 1024 * q);
        } else {
            const int row = 16 * q + (lane >> 2), gam = (lane & 3) ^ ((row >> 2) & 3);
            const int rel = 16 * (gam >> 1) + 4 * (gam & 1);
            const int word = w0 + rel + 4 <= nw ? w0 + rel : nw - 4;
            ter_dma16(w, o.w[q] - (uint32_t)rel * 4u + (uint32_t)word * 4u, ws + 1024 * q);
        }
    }
}

// Steps 8p .. 8p + 7 of chunk c from the LDS region into the two 32x32
// accumulators.
template <bool FULL>
__device__ __forceinline__ void ter_ks_half(const TerKsLds &s, int nw, int c, int p, int r, int h, i32x16 *acc)
{
#pragma unroll
    for (int g2 = 0; g2 < 2; g2++) {
        u32x4 wv[2];
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int wr = 32 * j + r;
            wv[j] = s.w[p][wr][(2 * h + g2) ^ ((wr >> 2) & 3)];
        }
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const int s8 = 4 * g2 + e;
            const i32x4 a = __builtin_bit_cast(i32x4, transpose_4x4_bytes(s.x[p][r][(8 * h + s8) ^ (r & 15)]));
#pragma unroll
            for (int j = 0; j < 2; j++) {
                uint32_t cw = wv[j][e];
                if (!FULL && 32 * c + 16 * h + 8 * p + s8 >= nw)
                    cw = 0u;
                const i32x4 b = {(int)(cw & 0x03030303u), (int)((cw >> 2) & 0x03030303u),
                                 (int)((cw >> 4) & 0x03030303u), (int)((cw >> 6) & 0x03030303u)};
                acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[j], 0, 0, 0);
            }
        }
    }
}

template <bool FULL>
__device__ __forceinline__ void ter_ks_chunk(const uint32_t *__restrict__ w, const int8_t *__restrict__ xq, int nw,
                                             int c, int r, int h, const TerKsOff &o, TerKsLds &s, i32x16 *acc)
{
    constexpr int D = 12; // loads per half
    ter_wait<0>();        // the previous chunk's fragment reads have completed
    ter_ks_load<FULL>(w, xq, nw, c, 0, o, s);
    ter_ks_load<FULL>(w, xq, nw, c, 1, o, s);
    ter_wait<D>();
    ter_ks_half<FULL>(s, nw, c, 0, r, h, acc);
    ter_wait<0>();
    ter_ks_half<FULL>(s, nw, c, 1, r, h, acc);
}

template <int KS>
__global__ __launch_bounds__(64 * KS) void ternary_gemm_ks_kernel(const uint32_t *__restrict__ w, float w_scale,
                                                                  const int8_t *__restrict__ xq,
                                                                  const float *__restrict__ act_scale,
                                                                  const int32_t *__restrict__ act_sum,
                                                                  float *__restrict__ y, int64_t m, int64_t n, int nw)
{
    constexpr int PAD = kTerKsCols + 8; // the two lane halves of a partial-tile store land 32 banks apart
    static_assert(kTerKsRows * PAD * 4 <= (int)sizeof(TerKsLds), "a wave's partial tile fits in its region");
    __shared__ TerKsLds lds[KS];
    const int lane = threadIdx.x & 63, r = lane & 31, h = lane >> 5;
    const int ks = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t m0 = (int64_t)blockIdx.y * kTerKsRows, n0 = (int64_t)blockIdx.x * kTerKsCols;
    const int nch = (nw + 31) / 32;

    // Epilogue: wave ks writes tile rows ks, ks + KS, ... (lane = column),
    // so each output row's scale and code sum are wave-uniform; requested
    // first.
    constexpr int PER = (kTerKsRows + KS - 1) / KS;
    float scs[PER];
    int asums[PER];
#pragma unroll
    for (int i = 0; i < PER; i++) {
        const int64_t rw = m0 + ks + KS * i;
        const int64_t rc = rw < m ? rw : m - 1;
        scs[i] = act_scale[rc];
        asums[i] = act_sum[rc];
    }
    TerKsOff o;
    ter_ks_offsets(m, n, nw, m0, n0, o);

    i32x16 acc[2] = {i32x16{}, i32x16{}};
    for (int c = ks; c < nch; c += KS) {
        if (32 * (c + 1) <= nw) // uniform
            ter_ks_chunk<true>(w, xq, nw, c, r, h, o, lds[ks], acc);
        else
            ter_ks_chunk<false>(w, xq, nw, c, r, h, o, lds[ks], acc);
    }
    if (KS == 1) {
        // D layout of a 32x32 tile: lane l, register v -> row 8 (v / 4) + 4 (l / 32) + v % 4, column l % 32
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const int64_t row = m0 + 8 * (v >> 2) + 4 * h + (v & 3), col = n0 + 32 * j + r;
                if (row < m && col < n)
                    y[row * n + col] = ternary_output(acc[j][v], act_sum[row], w_scale, act_scale[row]);
            }
        return;
    }
    __syncthreads(); // every wave is done with its region
    int *part = reinterpret_cast<int *>(&lds[ks]);
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
        for (int v = 0; v < 16; v++)
            part[(8 * (v >> 2) + 4 * h + (v & 3)) * PAD + 32 * j + r] = acc[j][v];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PER; i++) {
        const int rr = ks + KS * i;
        if (rr >= kTerKsRows)
            break;
        const int64_t row = m0 + rr, col = n0 + lane;
        int dot = 0;
#pragma unroll
        for (int q = 0; q < KS; q++)
            dot += reinterpret_cast<const int *>(&lds[q])[rr * PAD + lane];
        if (row < m && col < n)
            y[row * n + col] = ternary_output(dot, asums[i], w_scale, scs[i]);
    }
}

// ------------------------------------------------------------------ GEMM, about one workgroup per CU, 128 <= k <= 3072
// The k-split kernel's tile (32 activation rows x 64 weight rows) and MFMA,
// arranged for grids that fit on the CUs at once (the BitNet layer at
// m = 64: 216 workgroups).  There, 32-word chunks dealt to five waves leave
// one SIMD with two waves' MFMAs and unpacking while the others have one.
// Here eight waves, two per SIMD: the row's 128-code steps are cut into
// four equal shares, one per SIMD, and SIMD s's share into a first part for
// wave s and the rest for wave s + 4 (the waves of a workgroup are placed
// on the SIMDs in turn), so every SIMD dots the same number of steps and always
// has a second wave to cover one wave's dependency and LDS latencies.  A
// wave requests its whole part in one burst into its own LDS region, its
// 64 weight rows' words first and then the activation step by step, and
// dots each step as soon as it has landed; no barrier until the end.
// Layout of a region:
//   * x[step][row][slot]: the step's 128 activation bytes of the row as
//     eight 16-byte pieces (piece p = word p of the step), piece p in slot
//     p ^ f(row), f(row) = (row & 7) ^ ((row >> 3) & 1): the 8 or 16 lanes
//     that one pass of a fragment read serves fall in distinct banks.  A
//     DMA instruction fills rows 8i .. 8i + 7 with whole 128-byte lines.
//   * w[row][piece]: the weight row's words of the part, row-major (2 NQ
//     pieces of 4 words for a part of NQ steps), so each DMA instruction
//     reads whole runs of 2 NQ x 16 bytes.
// Step j: lane (r, h) reads word 4h + u of activation row r (transposed to
// the unpack order) for MFMA u = 0..3 and words 4h .. 4h + 3 of weight rows
// r and 32 + r (one 16-byte read each).  The exact int32 partial tiles are
// added in LDS in a fixed order at the end.
constexpr int kTbSimds = 4, kTbWaves = 2 * kTbSimds, kTbMaxShare = 6; // parts of <= 3 steps: 18 KB of LDS per wave
constexpr int64_t kTbMaxTiles = 256; // the grid fits on the 256 CUs at once

template <int NQ>
struct TbLds {
    u32x4 x[NQ][kTerKsRows][8];
    u32x4 w[kTerKsCols * 2 * NQ];
};

template <int NQ>
struct TbOff {
    uint32_t x[4];      // activation DMA i: row 8i + lane / 8 (clamped to m), its piece for slot lane % 8
    uint32_t w[2 * NQ]; // weight DMA i: row (64i + lane) / 2NQ (clamped to n), 16-byte half of the step
    int wq[2 * NQ];     // the step of the part that weight DMA i's piece belongs to
};

template <int NQ>
__device__ __forceinline__ void tb_offsets(int64_t m, int64_t n, int nw, int64_t m0, int64_t n0, TbOff<NQ> &o)
{
    const int lane = threadIdx.x & 63;
    // m * k and n * k / 4 are below 2^32 - 4096 (checked at launch)
    const uint32_t xrow = (uint32_t)nw * 16u, wrow = (uint32_t)nw * 4u;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int row = 8 * i + (lane >> 3);
        const int piece = (lane & 7) ^ (row & 7) ^ ((row >> 3) & 1);
        const uint32_t gi = (uint32_t)(m0 + row < m ? m0 + row : m - 1);
        o.x[i] = gi * xrow + 16u * (uint32_t)piece;
    }
#pragma unroll
    for (int i = 0; i < 2 * NQ; i++) {
        const int p = 64 * i + lane, row = p / (2 * NQ), pc = p % (2 * NQ);
        const uint32_t gj = (uint32_t)(n0 + row < n ? n0 + row : n - 1);
        o.w[i] = gj * wrow + 16u * (uint32_t)(pc & 1);
        o.wq[i] = pc >> 1;
    }
}

// Step j of a part of NQ steps (in a region for NR) into the two 32x32
// accumulators.
template <int NQ, int NR>
__device__ __forceinline__ void tb_step(const TbLds<NR> &s, int j, int r, int h, i32x16 *acc)
{
    const int f = (r & 7) ^ ((r >> 3) & 1);
    u32x4 wv[2];
#pragma unroll
    for (int jj = 0; jj < 2; jj++)
        wv[jj] = s.w[(32 * jj + r) * 2 * NQ + 2 * j + h];
#pragma unroll
    for (int u = 0; u < 4; u++) {
        const i32x4 a = __builtin_bit_cast(i32x4, transpose_4x4_bytes(s.x[j][r][(4 * h + u) ^ f]));
#pragma unroll
        for (int jj = 0; jj < 2; jj++) {
            const uint32_t cw = wv[jj][u];
            const i32x4 b = {(int)(cw & 0x03030303u), (int)((cw >> 2) & 0x03030303u),
                             (int)((cw >> 4) & 0x03030303u), (int)((cw >> 6) & 0x03030303u)};
            acc[jj] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[jj], 0, 0, 0);
        }
    }
}

// Wait until steps 0 .. j of a burst of NQ steps have landed (the weights
// first, then four activation loads per step).
template <int NQ>
__device__ __forceinline__ void tb_wait(int j)
{
    static_assert(NQ <= 3, "waits below");
    switch (4 * (NQ - 1 - j)) {
    case 4: ter_wait<4>(); break;
    case 8: ter_wait<8>(); break;
    default: ter_wait<0>(); break;
    }
}

// One wave's part, steps qa .. qb - 1 (at most NQ), into its region: the
// burst of loads, then each step dotted as soon as it has landed.  Steps
// past a shorter part re-read its last step (the wait counts stay static).
template <int NQ, int NR>
__device__ __forceinline__ void tb_part(const uint32_t *__restrict__ w, const int8_t *__restrict__ xq, int64_t m,
                                        int64_t n, int nw, int64_t m0, int64_t n0, int qa, int qb, TbLds<NR> &s, int r,
                                        int h, i32x16 *acc)
{
    static_assert(NQ <= NR, "the part fits in the region");
    TbOff<NQ> o;
    tb_offsets<NQ>(m, n, nw, m0, n0, o);
#pragma unroll
    for (int i = 0; i < 2 * NQ; i++) {
        const int qg = qa + o.wq[i] < qb ? qa + o.wq[i] : qb - 1;
        ter_dma16(w, o.w[i] + 32u * (uint32_t)qg, (const QLL_LDS_T char *)&s.w[0] + 1024 * i);
    }
#pragma unroll
    for (int j = 0; j < NQ; j++) {
        const int qg = qa + j < qb ? qa + j : qb - 1;
#pragma unroll
        for (int i = 0; i < 4; i++)
            ter_dma16(xq + 128 * (int64_t)qg, o.x[i], (const QLL_LDS_T char *)&s.x[j][0][0] + 1024 * i);
    }
    if (qb - qa == NQ) { // uniform; no branch between the steps of a whole part
#pragma unroll
        for (int j = 0; j < NQ; j++) {
            tb_wait<NQ>(j);
            tb_step<NQ, NR>(s, j, r, h, acc);
        }
    } else {
        const int cnt = qb - qa;
#pragma unroll
        for (int j = 0; j < NQ; j++) {
            tb_wait<NQ>(j);
            if (j < cnt) // uniform
                tb_step<NQ, NR>(s, j, r, h, acc);
        }
    }
}

// SHARE = steps per SIMD, ceil(k / 128 / 4): the first wave of a SIMD takes
// NA = ceil(SHARE / 2) of them, the second the other NB.
template <int SHARE>
__global__ __launch_bounds__(64 * kTbWaves) void ternary_gemm_burst_kernel(const uint32_t *__restrict__ w,
                                                                           float w_scale,
                                                                           const int8_t *__restrict__ xq,
                                                                           const float *__restrict__ act_scale,
                                                                           const int32_t *__restrict__ act_sum,
                                                                           float *__restrict__ y, int64_t m,
                                                                           int64_t n, int nw)
{
    constexpr int NA = (SHARE + 1) / 2, NB = SHARE - NA, NR = NA < 2 ? 2 : NA;
    constexpr int PAD = kTerKsCols + 8; // the two lane halves of a partial-tile store land 32 banks apart
    static_assert(kTerKsRows * PAD * 4 <= (int)sizeof(TbLds<NR>), "a wave's partial tile fits in its region");
    __shared__ TbLds<NR> lds[kTbWaves];
    const int lane = threadIdx.x & 63, r = lane & 31, h = lane >> 5;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t m0 = (int64_t)blockIdx.y * kTerKsRows, n0 = (int64_t)blockIdx.x * kTerKsCols;
    const int nq = nw >> 3;                           // 128-code steps per row: ceil(nq / 4) == SHARE
    const int sa = (wv % kTbSimds) * SHARE;           // the SIMD's share: steps sa .. se - 1
    const int se = sa + SHARE < nq ? sa + SHARE : nq;
    const int qa = wv < kTbSimds ? sa : sa + NA;      // this wave's part: steps qa .. qb - 1
    const int qb0 = wv < kTbSimds ? sa + NA : se;
    const int qb = qb0 < se ? qb0 : se;

    // Epilogue: wave wv writes tile rows wv, wv + 8, ...; their scales and
    // code sums are wave-uniform and requested first.
    constexpr int PER = kTerKsRows / kTbWaves;
    float scs[PER];
    int asums[PER];
#pragma unroll
    for (int i = 0; i < PER; i++) {
        const int64_t rw = m0 + wv + kTbWaves * i;
        const int64_t rc = rw < m ? rw : m - 1;
        scs[i] = act_scale[rc];
        asums[i] = act_sum[rc];
    }

    i32x16 acc[2] = {i32x16{}, i32x16{}};
    if (qa < qb) { // uniform
        if (wv < kTbSimds)
            tb_part<NA, NR>(w, xq, m, n, nw, m0, n0, qa, qb, lds[wv], r, h, acc);
        else if constexpr (NB > 0)
            tb_part<NB, NR>(w, xq, m, n, nw, m0, n0, qa, qb, lds[wv], r, h, acc);
    }

    __syncthreads(); // every wave is done with its region
    int *part = reinterpret_cast<int *>(&lds[wv]);
#pragma unroll
    for (int jj = 0; jj < 2; jj++)
#pragma unroll
        for (int v = 0; v < 16; v++)
            part[(8 * (v >> 2) + 4 * h + (v & 3)) * PAD + 32 * jj + r] = acc[jj][v];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PER; i++) {
        const int rr = wv + kTbWaves * i;
        const int64_t row = m0 + rr, col = n0 + lane;
        int dot = 0;
#pragma unroll
        for (int q = 0; q < kTbWaves; q++)
            dot += reinterpret_cast<const int *>(&lds[q])[rr * PAD + lane];
        if (row < m && col < n)
            y[row * n + col] = ternary_output(dot, asums[i], w_scale, scs[i]);
    }
}

hipError_t launch_ternary_gemm(const uint32_t *w, float w_scale, const int8_t *xq, const float *act_scale,
                               const int32_t *act_sum, float *y, int64_t m, int64_t n, int64_t k, hipStream_t st)
{
    const int nw = (int)(k / 16);
    // the k-split kernel addresses both operands with 32-bit lane offsets
    const bool small = m * k + 4096 < ((int64_t)1 << 32) && n * (k / 4) + 4096 < ((int64_t)1 << 32);
    const int64_t tiles = ((n + kTerKsCols - 1) / kTerKsCols) * ((m + kTerKsRows - 1) / kTerKsRows);
    if (nw % 8 == 0 && nw / 8 <= kTbSimds * kTbMaxShare && small && tiles <= kTbMaxTiles) {
        const int share = (nw / 8 + kTbSimds - 1) / kTbSimds;
        const dim3 grid((unsigned)((n + kTerKsCols - 1) / kTerKsCols), (unsigned)((m + kTerKsRows - 1) / kTerKsRows));
#define QLL_TB(S)                                                                                                      \
    hipLaunchKernelGGL((ternary_gemm_burst_kernel<S>), grid, dim3(64 * kTbWaves), 0, st, w, w_scale, xq, act_scale,    \
                       act_sum, y, m, n, nw)
        switch (share) {
        case 1: QLL_TB(1); break;
        case 2: QLL_TB(2); break;
        case 3: QLL_TB(3); break;
        case 4: QLL_TB(4); break;
        case 5: QLL_TB(5); break;
        default: QLL_TB(6); break;
        }
#undef QLL_TB
        return hipGetLastError();
    }
    if (nw % 4 == 0 && small) {
        const int nch = (nw + 31) / 32;
        // about one wave per SIMD (1024), at most one chunk per wave
        int64_t split = (kTerKsTargetWaves + tiles - 1) / tiles;
        split = split < nch ? split : nch;
        split = split < kTerKsMaxSplit ? split : kTerKsMaxSplit;
        const dim3 grid((unsigned)((n + kTerKsCols - 1) / kTerKsCols), (unsigned)((m + kTerKsRows - 1) / kTerKsRows));
#define QLL_TKS(KS)                                                                                                    \
    hipLaunchKernelGGL((ternary_gemm_ks_kernel<KS>), grid, dim3(64 * KS), 0, st, w, w_scale, xq, act_scale, act_sum, y, \
                       m, n, nw)
        switch (split) {
        case 1: QLL_TKS(1); break;
        case 2: QLL_TKS(2); break;
        case 3: QLL_TKS(3); break;
        case 4: QLL_TKS(4); break;
        case 5: QLL_TKS(5); break;
        default: QLL_TKS(6); break;
        }
#undef QLL_TKS
        return hipGetLastError();
    }
    dim3 grid((unsigned)((n + TBN - 1) / TBN), (unsigned)((m + TBM - 1) / TBM));
    if (nw % 4 == 0)
        hipLaunchKernelGGL(ternary_gemm_kernel<true>, grid, dim3(kTerGemmThreads), 0, st, w, w_scale, xq, act_scale,
                           act_sum, y, m, n, nw);
    else
        hipLaunchKernelGGL(ternary_gemm_kernel<false>, grid, dim3(kTerGemmThreads), 0, st, w, w_scale, xq,
                           act_scale, act_sum, y, m, n, nw);
    return hipGetLastError();
}

} // namespace qll
