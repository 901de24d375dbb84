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
    extern __shared__ u32x4 s_x[]; // [nw] transposed activation words
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
        a[j] = xv[i < nw ? i : 0];
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
            s_x[i] = transpose_4x4_bytes(a[j]);
    }
    for (int i = threadIdx.x + kTg2ActRegs * kTg2Threads; i < nw; i += kTg2Threads)
        s_x[i] = transpose_4x4_bytes(xv[i]);
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
                    const u32x4 t = s_x[4 * u + e];
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

// ------------------------------------------------------------------ GEMM (m > 1)
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
// The same MFMA and operand orders as above, restructured for latency: at the
// workload's size (m = 64, 4.4 MB of weights) the kernel is bound by memory
// round trips, not bytes or MFMAs.  One wave per workgroup owns 16 activation
// rows x 32 weight rows (four times as many workgroups as the 64 x 32 tile
// above), so no workgroup barrier is needed; every operand goes memory -> LDS
// (global_load_lds) into a ring of kTer2Buf chunk buffers, issued
// kTer2Buf - 1 chunks ahead, and the wave waits only for its own loads.  In
// LDS the activation word w of row r sits in slot w ^ (r & 15) and weight
// group g (4 words) of row r in group g ^ ((r >> 1) & 7), so the 16 rows an
// MFMA operand reads fall in distinct banks; the 4x4 byte transpose of the
// activation is applied after the LDS read.  Words past the end of the row
// (a partial last chunk) are loaded from clamped addresses and their
// activation operand is zeroed.
constexpr int kTer2BM = 16, kTer2BN = 32, kTer2Buf = 3;
constexpr int kTer2Dma = 12; // per chunk: 8 KB of activations + 4 KB of weights, 1 KB per wave-wide load

struct Ter2Lds {
    u32x4 x[kTer2BM][kTerWPC];  // [row][slot]
    u32x4 w[kTer2BN][kTerWPC / 4]; // [row][group]
};

__device__ __forceinline__ void ter2_dma16(const void *base, uint32_t off, const QLL_LDS_T void *lds)
{
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base),
                 "s"((uint32_t)(uintptr_t)lds)
                 : "memory", "m0");
}

// Chunk c (activation words 32c .. 32c + 31 of every row) into buffer s.
__device__ __forceinline__ void ter2_load(const uint32_t *__restrict__ w, const int8_t *__restrict__ xq, int64_t m,
                                          int64_t n, int nw, int64_t m0, int64_t n0, int c, Ter2Lds &s)
{
    const int lane = threadIdx.x;
    const QLL_LDS_T char *xs = (const QLL_LDS_T char *)&s.x[0][0];
    const QLL_LDS_T char *ws = (const QLL_LDS_T char *)&s.w[0][0];
#pragma unroll
    for (int q = 0; q < 8; q++) { // rows 2q, 2q + 1: lane -> (row, slot)
        const int rr = 2 * q + (lane >> 5), slot = lane & 31;
        const int64_t gi = m0 + rr < m ? m0 + rr : m - 1;
        int word = 32 * c + (slot ^ (rr & 15));
        word = word < nw ? word : nw - 1;
        ter2_dma16(xq, (uint32_t)((gi * nw + word) * 16), xs + 1024 * q);
    }
#pragma unroll
    for (int q = 0; q < 4; q++) { // rows 8q .. 8q + 7: lane -> (row, group)
        const int wr = 8 * q + (lane >> 3), grp = lane & 7;
        const int64_t gj = n0 + wr < n ? n0 + wr : n - 1;
        int word = 32 * c + 4 * (grp ^ ((wr >> 1) & 7));
        word = word + 4 <= nw ? word : nw - 4;
        ter2_dma16(w, (uint32_t)((gj * nw + word) * 4), ws + 1024 * q);
    }
}

template <int N>
__device__ __forceinline__ void ter2_wait()
{
    static_assert(N < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | (0x7 << 4)); // vmcnt(N) expcnt(7) lgkmcnt(0)
    asm volatile("" ::: "memory");
}

__global__ __launch_bounds__(64) void ternary_gemm2_kernel(const uint32_t *__restrict__ w, float w_scale,
                                                           const int8_t *__restrict__ xq,
                                                           const float *__restrict__ act_scale,
                                                           const int32_t *__restrict__ act_sum, float *__restrict__ y,
                                                           int64_t m, int64_t n, int nw)
{
    __shared__ Ter2Lds lds[kTer2Buf];
    const int64_t m0 = (int64_t)blockIdx.y * kTer2BM, n0 = (int64_t)blockIdx.x * kTer2BN;
    const int lane = threadIdx.x, lr = lane & 15, lh = lane >> 4;
    const int nch = (nw + kTerWPC - 1) / kTerWPC;

    i32x4 acc[2] = {i32x4{0, 0, 0, 0}, i32x4{0, 0, 0, 0}};
#pragma unroll
    for (int c = 0; c < kTer2Buf - 1; c++)
        if (c < nch)
            ter2_load(w, xq, m, n, nw, m0, n0, c, lds[c]);
    for (int c = 0; c < nch; c++) {
        const int ahead = c + kTer2Buf - 1;
        if (ahead < nch)
            ter2_load(w, xq, m, n, nw, m0, n0, ahead, lds[ahead % kTer2Buf]);
        // chunk c has landed once at most the loads of the later chunks remain
        const int later = (nch - 1 - c) < (kTer2Buf - 1) ? (nch - 1 - c) : (kTer2Buf - 1);
        if (later >= 2)
            ter2_wait<2 * kTer2Dma>();
        else if (later == 1)
            ter2_wait<kTer2Dma>();
        else
            ter2_wait<0>();
        const Ter2Lds &s = lds[c % kTer2Buf];
        u32x4 wv[2][2];
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int wr = 16 * j + lr, sw = (wr >> 1) & 7;
            wv[j][0] = s.w[wr][(2 * lh) ^ sw];
            wv[j][1] = s.w[wr][(2 * lh + 1) ^ sw];
        }
#pragma unroll
        for (int st = 0; st < 8; st++) {
            const int word = 32 * c + 8 * lh + st;
            i32x4 a = __builtin_bit_cast(i32x4, transpose_4x4_bytes(s.x[lr][(8 * lh + st) ^ lr]));
            if (word >= nw)
                a = i32x4{0, 0, 0, 0};
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const uint32_t cw = wv[j][st >> 2][st & 3];
                const i32x4 b = {(int)(cw & 0x03030303u), (int)((cw >> 2) & 0x03030303u),
                                 (int)((cw >> 4) & 0x03030303u), (int)((cw >> 6) & 0x03030303u)};
                acc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[j], 0, 0, 0);
            }
        }
    }
    // D layout of a 16x16 tile: lane l, register v -> row 4*(l/16)+v, column l%16
#pragma unroll
    for (int v = 0; v < 4; v++) {
        const int64_t row = m0 + 4 * lh + v;
        if (row >= m)
            continue;
        const float sc = act_scale[row];
        const int asum = act_sum[row];
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int64_t col = n0 + 16 * j + lr;
            if (col < n)
                y[row * n + col] = ternary_output(acc[j][v], asum, w_scale, sc);
        }
    }
}

// The same tile per wave (16 activation rows x 32 weight rows, the same
// MFMA and LDS layouts) with WN waves per workgroup side by side, so the
// activation chunk a workgroup loads serves WN * 32 weight rows (a quarter
// or half of the activation bytes the one-wave kernel reads per output), and
// a ring of NB chunk buffers, all filled at the start: with the workload's
// five chunks every load is requested before the first wait, so the kernel
// pays one memory round trip instead of one per ring turn.  The loads of a
// chunk are spread over the waves (per wave: its share of the activation
// rows and its own weight rows), so each wave waits for its own loads of the
// chunk and the workgroup then meets; after that meeting every wave is done
// with the previous chunk, whose buffer then takes the next chunk past the
// ring.
template <int WN>
struct Ter3Lds {
    u32x4 x[kTer2BM][kTerWPC];          // [row][slot]
    u32x4 w[WN * kTer2BN][kTerWPC / 4]; // [row][group]
};

template <int WN>
__device__ __forceinline__ void ter3_load(const uint32_t *__restrict__ w, const int8_t *__restrict__ xq, int64_t m,
                                          int64_t n, int nw, int64_t m0, int64_t n0, int c, int wave, Ter3Lds<WN> &s)
{
    const int lane = threadIdx.x & 63;
    const QLL_LDS_T char *xs = (const QLL_LDS_T char *)&s.x[0][0];
    const QLL_LDS_T char *ws = (const QLL_LDS_T char *)&s.w[0][0];
#pragma unroll
    for (int q0 = 0; q0 < 8 / WN; q0++) { // activation rows 2q, 2q + 1 for q = wave, wave + WN, ...
        const int q = wave + WN * q0;
        const int rr = 2 * q + (lane >> 5), slot = lane & 31;
        const int64_t gi = m0 + rr < m ? m0 + rr : m - 1;
        int word = 32 * c + (slot ^ (rr & 15));
        word = word < nw ? word : nw - 1;
        ter2_dma16(xq, (uint32_t)((gi * nw + word) * 16), xs + 1024 * q);
    }
#pragma unroll
    for (int q = 0; q < 4; q++) { // this wave's weight rows 32 wave + 8q .. + 7
        const int wr = 8 * q + (lane >> 3), grp = lane & 7;
        const int64_t gj = n0 + 32 * wave + wr < n ? n0 + 32 * wave + wr : n - 1;
        int word = 32 * c + 4 * (grp ^ ((wr >> 1) & 7));
        word = word + 4 <= nw ? word : nw - 4;
        ter2_dma16(w, (uint32_t)((gj * nw + word) * 4), ws + 4096 * wave + 1024 * q);
    }
}

// Wait until at most `later` chunks of this wave's loads are outstanding.
template <int D, int NB>
__device__ __forceinline__ void ter3_wait(int later)
{
    static_assert(D * (NB - 1) < 64, "vmcnt field");
    switch (later) {
    case 0: ter2_wait<0>(); break;
    case 1: ter2_wait<D>(); break;
    case 2: ter2_wait<(NB > 2 ? 2 * D : 0)>(); break;
    case 3: ter2_wait<(NB > 3 ? 3 * D : 0)>(); break;
    default: ter2_wait<(NB > 4 ? 4 * D : 0)>(); break;
    }
}

template <int WN, int NB>
__global__ __launch_bounds__(64 * WN) void ternary_gemm3_kernel(const uint32_t *__restrict__ w, float w_scale,
                                                                 const int8_t *__restrict__ xq,
                                                                 const float *__restrict__ act_scale,
                                                                 const int32_t *__restrict__ act_sum,
                                                                 float *__restrict__ y, int64_t m, int64_t n, int nw)
{
    static_assert(NB >= 2 && NB <= 5, "ring depth");
    constexpr int D = 8 / WN + 4; // loads per wave and chunk
    __shared__ Ter3Lds<WN> lds[NB];
    const int64_t m0 = (int64_t)blockIdx.y * kTer2BM, n0 = (int64_t)blockIdx.x * (kTer2BN * WN);
    const int lane = threadIdx.x & 63, lr = lane & 15, lh = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nch = (nw + kTerWPC - 1) / kTerWPC;

    i32x4 acc[2] = {i32x4{0, 0, 0, 0}, i32x4{0, 0, 0, 0}};
    // the scales and code sums of this lane's four output rows, requested
    // first so that the epilogue does not wait for another round trip
    float scs[4];
    int asums[4];
#pragma unroll
    for (int v = 0; v < 4; v++) {
        const int64_t rw = m0 + 4 * lh + v < m ? m0 + 4 * lh + v : m - 1;
        scs[v] = act_scale[rw];
        asums[v] = act_sum[rw];
    }
#pragma unroll
    for (int c = 0; c < NB; c++)
        if (c < nch)
            ter3_load<WN>(w, xq, m, n, nw, m0, n0, c, wave, lds[c]);
    for (int c = 0; c < nch; c++) {
        // chunks requested so far: the first NB, then one more per turn from c = 1
        const int issued = (NB + (c > 0 ? c - 1 : 0)) < nch ? NB + (c > 0 ? c - 1 : 0) : nch;
        ter3_wait<D, NB>(issued - c - 1);
        __syncthreads();
        if (c > 0 && c - 1 + NB < nch)
            ter3_load<WN>(w, xq, m, n, nw, m0, n0, c - 1 + NB, wave, lds[(c - 1) % NB]);
        const Ter3Lds<WN> &s = lds[c % NB];
        u32x4 wv[2][2];
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int wr = 32 * wave + 16 * j + lr, sw = ((16 * j + lr) >> 1) & 7;
            wv[j][0] = s.w[wr][(2 * lh) ^ sw];
            wv[j][1] = s.w[wr][(2 * lh + 1) ^ sw];
        }
#pragma unroll
        for (int st = 0; st < 8; st++) {
            const int word = 32 * c + 8 * lh + st;
            i32x4 a = __builtin_bit_cast(i32x4, transpose_4x4_bytes(s.x[lr][(8 * lh + st) ^ lr]));
            if (word >= nw)
                a = i32x4{0, 0, 0, 0};
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const uint32_t cw = wv[j][st >> 2][st & 3];
                const i32x4 b = {(int)(cw & 0x03030303u), (int)((cw >> 2) & 0x03030303u),
                                 (int)((cw >> 4) & 0x03030303u), (int)((cw >> 6) & 0x03030303u)};
                acc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[j], 0, 0, 0);
            }
        }
    }
    // no load may still be writing this workgroup's LDS when it ends
    ter2_wait<0>();
    // D layout of a 16x16 tile: lane l, register v -> row 4*(l/16)+v, column l%16
#pragma unroll
    for (int v = 0; v < 4; v++) {
        const int64_t row = m0 + 4 * lh + v;
        if (row >= m)
            continue;
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int64_t col = n0 + 32 * wave + 16 * j + lr;
            if (col < n)
                y[row * n + col] = ternary_output(acc[j][v], asums[v], w_scale, scs[v]);
        }
    }
}

hipError_t launch_ternary_gemm(const uint32_t *w, float w_scale, const int8_t *xq, const float *act_scale,
                               const int32_t *act_sum, float *y, int64_t m, int64_t n, int64_t k, hipStream_t st)
{
    const int nw = (int)(k / 16);
    // the restructured kernel addresses both operands with 32-bit offsets
    const bool small = m * k < ((int64_t)1 << 32) && n * (k / 4) < ((int64_t)1 << 32);
    if (nw % 4 == 0 && small) {
        constexpr int WN = 2, NB = 5;
        dim3 grid3((unsigned)((n + WN * kTer2BN - 1) / (WN * kTer2BN)), (unsigned)((m + kTer2BM - 1) / kTer2BM));
        hipLaunchKernelGGL((ternary_gemm3_kernel<WN, NB>), grid3, dim3(64 * WN), 0, st, w, w_scale, xq, act_scale,
                           act_sum, y, m, n, nw);
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
