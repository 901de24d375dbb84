// Q4_0 x Q8_0 for a handful of activation rows (speculative or batched
// decode, short prompts: 2 <= m <= 32; the GEMM entry runs 33 <= m <= 64 as
// groups of at most 32 rows) on the int8 matrix core.  For every
// activation row i, weight row j and block b the arithmetic is that of
// llama.cpp visual guide lesson 31 "CPU backend" ("How the quantized dot
// product works"):
//     P = sum_t (q_w[j,b,t] - 8) * q_x[i,b,t]          exact integer
//     Y[i,j] += (f32(d_w[j,b]) * f32(d_x[i,b])) * P       f32
// -- per block the same exact sum and the same f32 product as the decode
// GEMV kernels.
//
// Tile.  K = 32 of v_mfma_i32_16x16x32_i8 is one block, so one instruction
// forms the block sums of 16 weight rows x 16 activation rows.  Lane l holds
// operand bytes for row l % 16 and lane group g = l / 16: its eight weight
// bytes come from the two nibbles of dword g of the block's codes (codes
// 4g..4g+3 and 16+4g..16+4g+3) and its eight activation bytes are the same
// codes of the activation row, so both operands put the same code at the
// same byte and the matrix core pairs every weight code with its own
// activation code whatever order it gives K.  The scale tile d_w d_x^T is a
// second, f16 MFMA; the vector ALU converts each sum and does one fma per
// output and block.
//
// Work split (the tall-matrix form that shares activation stages between
// waves is described at its kernel below).  A workgroup owns one or two
// 16-row weight tiles (two on tall matrices, so that each activation
// fragment feeds two block sums).  Its KS
// waves take KS contiguous runs of the row's blocks, and each wave streams
// its run -- its weight rows and every activation row, eight blocks a stage,
// exactly as stored -- from memory into two LDS stage buffers of its own
// (global_load_lds, whole contiguous 16-byte pieces), the next stage in
// flight while the current one is computed.  No wave waits for another
// until the end, where the KS partial tiles are added in LDS in wave order,
// so the result does not depend on timing.  Weight rows past n and
// activation rows past m load the last valid row instead (their outputs are
// dropped); the row's last stage starts at block nb - 8 and computes only
// the blocks the stage before did not.
#include "common.h"

namespace qll {

#define QLL_LDS_M __attribute__((address_space(3)))
typedef float f32x4_m __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4_m __attribute__((ext_vector_type(4)));

constexpr int kSmSB = 8;    // blocks per stage
constexpr int kSmNS = 2;    // stage buffers per wave (1 or 2)
constexpr int kSmGroup = 8; // block products (times tiles) formed before their sums

// 16-column activation tiles for MP staged activation rows.
constexpr int sm_mt(int mp) { return mp > 16 ? mp / 16 : 1; }

// Byte layout of one stage buffer for T 16-row weight tiles (1 or 2) and MP
// activation rows (4, 8, 16 or 32): the stage's eight blocks of each row
// exactly as stored (144 bytes of weights, 272 of activations: whole 16-byte
// pieces), rows one after another (so every load instruction reads
// contiguous runs), each region padded to whole 1 KB loads.
template <int T, int MP>
struct SmLayout {
    static constexpr int WR = 16 * T;                          // weight rows
    static constexpr int WROW = 18 * kSmSB, XROW = 34 * kSmSB; // bytes per row
    static constexpr int WP = WROW / 16, XP = XROW / 16;       // 16-byte pieces per row: 9 and 17
    // wave-wide loads per stage (64 lanes of 16 bytes each)
    static constexpr int NW = (WR * WP + 63) / 64, NX = (MP * XP + 63) / 64;
    static constexpr int DMA = NW + NX;
    static constexpr int W = 0;             // [WR weight rows][144 B], then padding
    static constexpr int X = W + 1024 * NW; // [MP activation rows][272 B], then padding
    static constexpr int STAGE = X + 1024 * NX;
};

// Byte offset of each lane's 16-byte piece in each load of a stage, relative
// to the stage's first block (weights: of the workgroup's first row).  Lane l
// of load i writes LDS bytes 16 (64 i + l) of its region, so it fetches
// piece 64 i + l of the rows laid end to end; lanes past the last piece
// fetch the first piece again into the padding.
template <int T, int MP>
struct SmOff {
    uint32_t w[SmLayout<T, MP>::NW], x[SmLayout<T, MP>::NX];
};

template <int T, int MP>
__device__ __forceinline__ void sm_offsets(int64_t m, int64_t n, int nb, int64_t row0, SmOff<T, MP> &o)
{
    using L = SmLayout<T, MP>;
    const int lane = threadIdx.x & 63;
    // n, m < 2^31 and k < 2^24 at the boundary: 32 rows of weights or of
    // activations span far less than 4 GiB
    const uint32_t rb = (uint32_t)nb * 18u, xr = (uint32_t)nb * 34u;
#pragma unroll
    for (int i = 0; i < L::NW; i++) {
        const int p = 64 * i + lane < L::WR * L::WP ? 64 * i + lane : 0, r = p / L::WP, c = p % L::WP;
        const uint32_t rr = (uint32_t)(row0 + r < n ? r : n - 1 - row0);
        o.w[i] = rr * rb + 16u * (uint32_t)c;
    }
#pragma unroll
    for (int i = 0; i < L::NX; i++) {
        const int p = 64 * i + lane < MP * L::XP ? 64 * i + lane : 0, a = p / L::XP, c = p % L::XP;
        const uint32_t ac = (uint32_t)(a < m ? a : m - 1);
        o.x[i] = ac * xr + 16u * (uint32_t)c;
    }
}

// One wave-wide global -> LDS load: lane l reads 16 bytes at base + off and
// the wave writes them to LDS at lds + 16 l.  The addresses need only be
// 2-byte aligned.  Inline assembly keeps these loads out of the compiler's
// wait bookkeeping; the waits below count them.
__device__ __forceinline__ void sm_dma16(const void *base, uint32_t off, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(lds)
                 : "memory", "m0");
}

// Wait until at most N of this wave's vector-memory operations are
// outstanding and all its LDS operations have completed.
template <int N>
__device__ __forceinline__ void sm_wait()
{
    static_assert(N < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | (0x7 << 4));
    asm volatile("" ::: "memory");
}

// Wait for this wave's LDS operations only (vmcnt left at its maximum).
__device__ __forceinline__ void sm_wait_lds()
{
    __builtin_amdgcn_s_waitcnt(0xf | (0x3 << 14) | (0x7 << 4));
    asm volatile("" ::: "memory");
}

// The loads of the stage whose first block is be (be + 8 <= nb), into the
// buffer at lds: L::DMA wave-wide loads, all lanes active.
template <int T, int MP>
__device__ __forceinline__ void sm_load(const uint8_t *wt, const uint8_t *xq, int be, const SmOff<T, MP> &o,
                                        uint32_t lds)
{
    using L = SmLayout<T, MP>;
    const uint8_t *wb = wt + 18 * (int64_t)be, *xb = xq + 34 * (int64_t)be;
#pragma unroll
    for (int i = 0; i < L::NX; i++)
        sm_dma16(xb, o.x[i], lds + L::X + 1024 * i);
#pragma unroll
    for (int i = 0; i < L::NW; i++)
        sm_dma16(wb, o.w[i], lds + L::W + 1024 * i);
}

// A stage's weight rows and activation rows in LDS.
struct SmBufs {
    const QLL_LDS_M char *w, *x;
};

template <typename V>
__device__ __forceinline__ V sm_lds(const QLL_LDS_M char *p)
{
    return *reinterpret_cast<const QLL_LDS_M V *>(p);
}

// The four bytes at p in LDS, p = 2 (mod 4) when TWO, else a multiple of 4.
template <bool TWO>
__device__ __forceinline__ uint32_t sm_word(const QLL_LDS_M char *p)
{
    if constexpr (TWO)
        return funnel(sm_lds<uint32_t>(p + 2), sm_lds<uint32_t>(p - 2), 16);
    else
        return sm_lds<uint32_t>(p);
}

// The binary16 at p in LDS (p even; HIGH: p = 2 mod 4), zero-extended, in
// lanes whose width is 16 (and 0 in lanes whose width is 0).
template <bool HIGH>
__device__ __forceinline__ uint32_t sm_half_bits(const QLL_LDS_M char *p, uint32_t width)
{
    if constexpr (HIGH)
        return __builtin_amdgcn_ubfe(sm_lds<uint32_t>(p - 2), 16, width);
    else
        return __builtin_amdgcn_ubfe(sm_lds<uint32_t>(p), 0, width);
}

// Products of block bl of a stage buffer: for weight tile u and activation
// tile t, p[u MT + t] = 16 P and sc[u MT + t] = S on the 16 x 16 output
// layout (lane l, register i: weight row 16 u + 4 (l / 16) + i, activation
// row 16 t + l % 16).  In a row, block bl's scale sits at 18 bl (weights)
// or 34 bl (activations) and its codes 2 bytes later, so for even bl the
// code words straddle dwords and for odd bl the scales sit in the high half
// of a dword.
//   Weight operand: t = w ^ 0x88888888 flips the top bit of both nibbles of
// every byte, so (t & 0xf0f0f0f0) holds the bytes 16 (q - 8) of the high
// nibbles as signed 8-bit values ((16 q) ^ 0x80 = 16 q - 128), and
// ((t << 4) & 0xf0f0f0f0) those of the low nibbles; the block sum comes out
// as 16 P, exact in int32 and in f32 (|16 P| < 2^24), and the final outputs
// are divided by 16, which is exact, so every result equals that of P.
//   Scales: the tile S = d_w d_x^T is formed on the matrix core
// (v_mfma_f32_16x16x16_f16 with only k = 0 nonzero: lanes 0..15 hold their
// row's d_w and d_x, the others zeros), every entry the exact f32 product of
// two halves.
template <int T, int MP, int BL>
__device__ __forceinline__ void sm_mfma(const SmBufs &s, uint32_t width, i32x4 (&p)[T * sm_mt(MP)],
                                        f32x4_m (&sc)[T * sm_mt(MP)])
{
    using L = SmLayout<T, MP>;
    constexpr bool ODD = BL & 1;
    constexpr int MT = sm_mt(MP);
    const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
    // activation rows past MP (columns of the tile past m): any staged row
    const int ra = r < MP ? r : MP - 1;
    long aop[T];
    f16x4_m sa[T];
#pragma unroll
    for (int u = 0; u < T; u++) {
        const QLL_LDS_M char *wrow = s.w + (16 * u + r) * L::WROW + 18 * BL;
        const uint32_t wt = sm_word<!ODD>(wrow + 2 + 4 * g) ^ 0x88888888u;
        aop[u] = (long)(((uint64_t)(wt & 0xf0f0f0f0u) << 32) | ((wt << 4) & 0xf0f0f0f0u));
        sa[u] = __builtin_bit_cast(f16x4_m, (uint64_t)sm_half_bits<ODD>(wrow, width));
    }
#pragma unroll
    for (int t = 0; t < MT; t++) {
        const QLL_LDS_M char *xrow = s.x + (16 * t + ra) * L::XROW + 34 * BL;
        const uint32_t x0 = sm_word<!ODD>(xrow + 2 + 4 * g), x1 = sm_word<!ODD>(xrow + 18 + 4 * g);
        const long bop = (long)(((uint64_t)x1 << 32) | x0);
        const f16x4_m sb = __builtin_bit_cast(f16x4_m, (uint64_t)sm_half_bits<ODD>(xrow, width));
#pragma unroll
        for (int u = 0; u < T; u++) {
            p[u * MT + t] = __builtin_amdgcn_mfma_i32_16x16x32_i8(aop[u], bop, i32x4{0, 0, 0, 0}, 0, 0, 0);
            sc[u * MT + t] = __builtin_amdgcn_mfma_f32_16x16x16f16(sa[u], sb, f32x4_m{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        }
    }
}

template <int N>
__device__ __forceinline__ void sm_apply(const i32x4 (&p)[N], const f32x4_m (&sc)[N], float (&acc)[N][4])
{
#pragma unroll
    for (int t = 0; t < N; t++)
#pragma unroll
        for (int i = 0; i < 4; i++)
            acc[t][i] += sc[t][i] * (float)p[t][i];
}

template <int T, int MP, int BL>
__device__ __forceinline__ void sm_block(const SmBufs &s, uint32_t width, float (&acc)[T * sm_mt(MP)][4])
{
    i32x4 p[T * sm_mt(MP)];
    f32x4_m sc[T * sm_mt(MP)];
    sm_mfma<T, MP, BL>(s, width, p, sc);
    sm_apply(p, sc, acc);
}

// Blocks B0 .. B0 + G - 1: every block's products first, then their sums
// in block order (the matrix core's latency covered by the later blocks).
template <int T, int MP, int B0, int G>
__device__ __forceinline__ void sm_group(const SmBufs &s, uint32_t width, float (&acc)[T * sm_mt(MP)][4])
{
    constexpr int N = T * sm_mt(MP);
    i32x4 p[G][N];
    f32x4_m sc[G][N];
    if constexpr (G > 0) sm_mfma<T, MP, B0 + 0>(s, width, p[0], sc[0]);
    if constexpr (G > 1) sm_mfma<T, MP, B0 + 1>(s, width, p[1], sc[1]);
    if constexpr (G > 2) sm_mfma<T, MP, B0 + 2>(s, width, p[2], sc[2]);
    if constexpr (G > 3) sm_mfma<T, MP, B0 + 3>(s, width, p[3], sc[3]);
    if constexpr (G > 4) sm_mfma<T, MP, B0 + 4>(s, width, p[4], sc[4]);
    if constexpr (G > 5) sm_mfma<T, MP, B0 + 5>(s, width, p[5], sc[5]);
    if constexpr (G > 6) sm_mfma<T, MP, B0 + 6>(s, width, p[6], sc[6]);
    if constexpr (G > 7) sm_mfma<T, MP, B0 + 7>(s, width, p[7], sc[7]);
#pragma unroll
    for (int b = 0; b < G; b++)
        sm_apply(p[b], sc[b], acc);
}

// Blocks lo .. 7 of a stage buffer (lo > 0 only for a row's last stage,
// which starts inside the one before).
template <int T, int MP>
__device__ __forceinline__ void sm_stage(const SmBufs &s, int lo, uint32_t width, float (&acc)[T * sm_mt(MP)][4])
{
    if (lo == 0) { // uniform
        constexpr int G = kSmGroup / (T * sm_mt(MP)); // 8, 4 or 2 blocks
        static_assert(G >= 1 && kSmSB % G == 0, "whole groups per stage");
        sm_group<T, MP, 0, G>(s, width, acc);
        if constexpr (G < kSmSB) sm_group<T, MP, G % kSmSB, G>(s, width, acc);
        if constexpr (3 * G <= kSmSB) sm_group<T, MP, (2 * G) % kSmSB, G>(s, width, acc);
        if constexpr (4 * G <= kSmSB) sm_group<T, MP, (3 * G) % kSmSB, G>(s, width, acc);
        return;
    }
    if (lo <= 1) sm_block<T, MP, 1>(s, width, acc);
    if (lo <= 2) sm_block<T, MP, 2>(s, width, acc);
    if (lo <= 3) sm_block<T, MP, 3>(s, width, acc);
    if (lo <= 4) sm_block<T, MP, 4>(s, width, acc);
    if (lo <= 5) sm_block<T, MP, 5>(s, width, acc);
    if (lo <= 6) sm_block<T, MP, 6>(s, width, acc);
    sm_block<T, MP, 7>(s, width, acc);
}

template <int T, int MP, int KS>
__global__ __launch_bounds__(64 * KS) void q4_0_small_m_mfma_kernel(const uint8_t *__restrict__ w,
                                                                    const uint8_t *__restrict__ xq,
                                                                    float *__restrict__ y, int64_t m, int64_t n,
                                                                    int nb)
{
    using L = SmLayout<T, MP>;
    constexpr int MT = sm_mt(MP), N = T * MT;
    static_assert(N * 4 * 64 * 4 <= kSmNS * L::STAGE, "a wave's partial tile fits in its stage buffers");
    static_assert(kSmNS == 1 || kSmNS == 2, "one stage in flight at most");
    __shared__ __attribute__((aligned(16))) char stage[KS][kSmNS][L::STAGE];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t row0 = (int64_t)blockIdx.x * L::WR;
    const uint8_t *wt = w + row0 * ((int64_t)nb * 18);
    // this wave's stages: s0 .. s1 - 1 of the row's nst
    const int nst = (nb + kSmSB - 1) / kSmSB;
    const int s0 = nst * wave / KS, s1 = nst * (wave + 1) / KS;
    const int blast = nb - kSmSB; // first block of the row's last stage
    SmOff<T, MP> o;
    sm_offsets<T, MP>(m, n, nb, row0, o);
    const QLL_LDS_M char *buf = (const QLL_LDS_M char *)&stage[wave][0][0];
    const uint32_t lds = (uint32_t)(uintptr_t)buf;

    const uint32_t width = lane < 16 ? 16u : 0u; // the scale operands live in lanes 0..15
    float acc[N][4];
#pragma unroll
    for (int t = 0; t < N; t++)
#pragma unroll
        for (int i = 0; i < 4; i++)
            acc[t][i] = 0.0f;
    // kSmNS stage buffers in a ring: stage s in buffer s % kSmNS, the
    // kSmNS - 1 stages after it in flight while it is computed
#pragma unroll
    for (int j = 0; j < kSmNS; j++)
        if (s0 + j < s1)
            sm_load<T, MP>(wt, xq, min((s0 + j) * kSmSB, blast), o, lds + j * L::STAGE);
    for (int s2 = s0; s2 < s1; s2 += kSmNS) {
#pragma unroll
        for (int j = 0; j < kSmNS; j++) { // buffer j: a constant offset
            const int s = s2 + j;
            if (s >= s1)
                break;
            if (kSmNS > 1 && s + 1 < s1)
                sm_wait<(kSmNS - 1) * L::DMA>(); // stage s has landed, the one after may not have
            else
                sm_wait<0>();
            const SmBufs sb{buf + j * L::STAGE + L::W, buf + j * L::STAGE + L::X};
            sm_stage<T, MP>(sb, s * kSmSB - min(s * kSmSB, blast), width, acc);
            if (s + kSmNS < s1) {
                sm_wait_lds(); // this buffer's reads have completed
                sm_load<T, MP>(wt, xq, min((s + kSmNS) * kSmSB, blast), o, lds + j * L::STAGE);
            }
        }
    }

    // Partial tiles, each in its wave's own stage buffers (the wave's loads
    // have all landed: its last wait counted zero), as part[4 (u MT + t) +
    // i][lane]; then each output summed over the waves in order.
    typedef float Part[N * 4][64];
#pragma unroll
    for (int t = 0; t < N; t++)
#pragma unroll
        for (int i = 0; i < 4; i++)
            (*reinterpret_cast<Part *>(&stage[wave][0][0]))[4 * t + i][lane] = acc[t][i];
    __syncthreads();
    for (int oi = threadIdx.x; oi < 256 * N; oi += 64 * KS) {
        // activation row col and weight row row of the workgroup's tile
        const int col = oi / L::WR, row = oi % L::WR;
        const int u = row >> 4, t = col >> 4;
        const int reg = 4 * (u * MT + t) + (row & 3), ln = 16 * ((row & 15) >> 2) + (col & 15);
        float v = (*reinterpret_cast<const Part *>(&stage[0][0][0]))[reg][ln];
#pragma unroll
        for (int q = 1; q < KS; q++)
            v += (*reinterpret_cast<const Part *>(&stage[q][0][0]))[reg][ln];
        if (col < m && row0 + row < n)
            y[(int64_t)col * n + row0 + row] = v * 0.0625f; // the sums were of 16 P
    }
}

// Wait until at most n (0 .. 15) of this wave's vector-memory operations
// are outstanding (n uniform), and all its LDS operations have completed.
__device__ __forceinline__ void sm_wait_n(int n)
{
    switch (n) {
    case 0: sm_wait<0>(); break;
    case 1: sm_wait<1>(); break;
    case 2: sm_wait<2>(); break;
    case 3: sm_wait<3>(); break;
    case 4: sm_wait<4>(); break;
    case 5: sm_wait<5>(); break;
    case 6: sm_wait<6>(); break;
    case 7: sm_wait<7>(); break;
    case 8: sm_wait<8>(); break;
    case 9: sm_wait<9>(); break;
    case 10: sm_wait<10>(); break;
    case 11: sm_wait<11>(); break;
    case 12: sm_wait<12>(); break;
    case 13: sm_wait<13>(); break;
    case 14: sm_wait<14>(); break;
    default: sm_wait<15>(); break;
    }
}

// Tall matrices: R waves, each with its own T weight tiles and the whole
// row of blocks, share one activation stage.  Wave w loads its weight rows
// and the activation loads i = w, w + R, ...; after its own loads have
// landed it meets the others at a barrier (then every load of the stage has
// landed), computes, and meets them again before the buffer it read is
// refilled.  The activation rows are read from L2 once per R T weight tiles
// instead of once per tile, and a wave needs only its weight rows' LDS.
template <int T, int MP, int R>
__global__ __launch_bounds__(64 * R) void q4_0_small_m_shared_kernel(const uint8_t *__restrict__ w,
                                                                     const uint8_t *__restrict__ xq,
                                                                     float *__restrict__ y, int64_t m, int64_t n,
                                                                     int nb)
{
    using L = SmLayout<T, MP>;
    constexpr int MT = sm_mt(MP), N = T * MT, WB = 1024 * L::NW, XB = 1024 * L::NX;
    static_assert(N * 4 * 64 * 4 <= WB, "a wave's output tile fits in its weight buffer");
    static_assert(L::NW + (L::NX + R - 1) / R <= 15, "loads per wave and stage");
    __shared__ __attribute__((aligned(16))) char wst[2][R][WB];
    __shared__ __attribute__((aligned(16))) char xst[2][XB];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t row0 = ((int64_t)blockIdx.x * R + wave) * L::WR;
    // a last workgroup's waves past n load row n - 1 (outputs dropped)
    const int64_t lrow0 = row0 < n ? row0 : n - 1;
    const uint8_t *wt = w + lrow0 * ((int64_t)nb * 18);
    const int nst = (nb + kSmSB - 1) / kSmSB, blast = nb - kSmSB;
    SmOff<T, MP> o;
    sm_offsets<T, MP>(m, n, nb, lrow0, o);
    const int nxw = (L::NX - wave + R - 1) / R; // this wave's activation loads per stage (may be 0)
    const int dma = L::NW + nxw;
    const uint32_t wl[2] = {(uint32_t)(uintptr_t)&wst[0][wave][0], (uint32_t)(uintptr_t)&wst[1][wave][0]};
    const uint32_t xl[2] = {(uint32_t)(uintptr_t)&xst[0][0], (uint32_t)(uintptr_t)&xst[1][0]};
    auto load = [&](int st, int j) {
        const int be = min(st * kSmSB, blast);
        const uint8_t *wb = wt + 18 * (int64_t)be, *xb = xq + 34 * (int64_t)be;
#pragma unroll
        for (int i = 0; i < L::NX; i++)
            if (i % R == wave) // uniform
                sm_dma16(xb, o.x[i], xl[j] + 1024 * i);
#pragma unroll
        for (int i = 0; i < L::NW; i++)
            sm_dma16(wb, o.w[i], wl[j] + 1024 * i);
    };

    const uint32_t width = lane < 16 ? 16u : 0u; // the scale operands live in lanes 0..15
    float acc[N][4];
#pragma unroll
    for (int t = 0; t < N; t++)
#pragma unroll
        for (int i = 0; i < 4; i++)
            acc[t][i] = 0.0f;
    load(0, 0);
    if (1 < nst)
        load(1, 1);
    for (int s2 = 0; s2 < nst; s2 += 2) {
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int st = s2 + j;
            if (st >= nst)
                break;
            sm_wait_n(st + 1 < nst ? dma : 0); // this wave's loads of stage st have landed
            __syncthreads();                    // and every wave's
            const SmBufs sb{(const QLL_LDS_M char *)&wst[j][wave][0], (const QLL_LDS_M char *)&xst[j][0]};
            sm_stage<T, MP>(sb, st * kSmSB - min(st * kSmSB, blast), width, acc);
            if (st + 2 < nst) {
                __syncthreads(); // every wave is done reading buffer j
                load(st + 2, j);
            }
        }
    }

    // The wave's tile through its own weight buffer (its loads have all
    // landed), as part[4 t + i][lane], then stored row-contiguously.
    typedef float Part[N * 4][64];
    Part &part = *reinterpret_cast<Part *>(&wst[0][wave][0]);
#pragma unroll
    for (int t = 0; t < N; t++)
#pragma unroll
        for (int i = 0; i < 4; i++)
            part[4 * t + i][lane] = acc[t][i];
    for (int oi = lane; oi < 256 * N; oi += 64) {
        const int col = oi / L::WR, row = oi % L::WR;
        const int u = row >> 4, t = col >> 4;
        const int reg = 4 * (u * MT + t) + (row & 3), ln = 16 * ((row & 15) >> 2) + (col & 15);
        if (col < m && row0 + row < n)
            y[(int64_t)col * n + row0 + row] = part[reg][ln] * 0.0625f; // the sums were of 16 P
    }
}

// Workgroups of one split that fit on a CU at once (the LDS bounds them).
template <int T, int MP>
constexpr int sm_per_cu(int ks)
{
    return 160 * 1024 / (ks * kSmNS * SmLayout<T, MP>::STAGE);
}

template <int T, int MP, int KS>
static void launch_sm(const uint8_t *w, const uint8_t *xq, float *y, int64_t m, int64_t n, int nb, hipStream_t s)
{
    // splits whose workgroup does not fit are never chosen
    if constexpr (sm_per_cu<T, MP>(KS) >= 1) {
        const unsigned tiles = (unsigned)((n + 16 * T - 1) / (16 * T));
        hipLaunchKernelGGL((q4_0_small_m_mfma_kernel<T, MP, KS>), dim3(tiles), dim3(64 * KS), 0, s, w, xq, y, m, n,
                           nb);
    }
}

// Activation rows staged for m: 4, 8, 16 or 32.
static int sm_rows(int64_t m) { return m <= 4 ? 4 : m <= 8 ? 8 : m <= 16 ? 16 : 32; }

// 16-row weight tiles per wave, where the activation stages are the wave's
// own: two (each activation fragment feeding two block sums, so the
// activation rows, re-read for every weight tile, cost half as much per
// weight byte) from n = 8192 at m > 16; one elsewhere, where the extra
// workgroups matter more (measured, 4096 -> 14336 at m = 32: 19.4 -> 17.3
// us, at m = 16: 13.9 -> 14.9 us).
static int small_m_mfma_row_tiles(int64_t m, int64_t n, int64_t k)
{
    (void)k;
    return n >= 8192 && m > 16 ? 2 : 1;
}

static int sm_per_cu_1(int mp, int ks)
{
    return mp == 4 ? sm_per_cu<1, 4>(ks) : mp == 8 ? sm_per_cu<1, 8>(ks) : mp == 16 ? sm_per_cu<1, 16>(ks)
                                                                                     : sm_per_cu<1, 32>(ks);
}

// Waves per row tile: the largest split (at most 8, or 2 with two-tile
// waves) whose workgroups all fit on the chip at once and that leaves every
// wave at least two stages; one wave per row tile when even that is more
// workgroups than fit.
static int small_m_mfma_split(int64_t m, int64_t n, int64_t k)
{
    const int rt = small_m_mfma_row_tiles(m, n, k), mp = sm_rows(m);
    const int64_t tiles = (n + 16 * rt - 1) / (16 * rt), nst = (k / 32 + kSmSB - 1) / kSmSB;
    for (int ks = rt == 2 ? 2 : 8; ks > 1; ks /= 2) {
        const int per_cu = rt == 2 ? sm_per_cu<2, 32>(ks) : sm_per_cu_1(mp, ks); // two tiles: m > 16
        if (nst >= 2 * ks && tiles <= 256 * per_cu)
            return ks;
    }
    return 1;
}

template <int MP>
static void launch_sm_ks(int ks, const uint8_t *w, const uint8_t *xq, float *y, int64_t m, int64_t n, int nb,
                         hipStream_t s)
{
    switch (ks) {
    case 1: launch_sm<1, MP, 1>(w, xq, y, m, n, nb, s); break;
    case 2: launch_sm<1, MP, 2>(w, xq, y, m, n, nb, s); break;
    case 4: launch_sm<1, MP, 4>(w, xq, y, m, n, nb, s); break;
    default: launch_sm<1, MP, 8>(w, xq, y, m, n, nb, s); break;
    }
}

// Tall matrices (n >= 32768) at m > 4 share each activation stage among the
// waves of a workgroup: kShR waves of kShT weight tiles (measured on
// 4096 -> 128256 at m = 8 / 16 / 32 / 48: 78 / 80 / 126 / 194 us with
// one-wave stages, 72 / 76 / 103 / 173 us with four waves of two tiles;
// one tile or two waves were slower).
constexpr int kShT = 2, kShR = 4;

static bool small_m_mfma_shared(int64_t m, int64_t n, int64_t k)
{
    (void)k;
    return n >= 32768 && m > 4;
}

template <int MP>
static void launch_sh(const uint8_t *w, const uint8_t *xq, float *y, int64_t m, int64_t n, int nb, hipStream_t s)
{
    const unsigned groups = (unsigned)((n + 16 * kShT * kShR - 1) / (16 * kShT * kShR));
    hipLaunchKernelGGL((q4_0_small_m_shared_kernel<kShT, MP, kShR>), dim3(groups), dim3(64 * kShR), 0, s, w, xq, y,
                       m, n, nb);
}

hipError_t launch_q4_0_q8_0_small_m_mfma(const uint8_t *w, const uint8_t *xq, float *y, int64_t m, int64_t n,
                                         int64_t k, hipStream_t s)
{
    if (m < 1 || m > kMaxMMfma || k < kMinKMfma || k >= kMaxKMfma)
        return hipErrorInvalidValue;
    if ((n + 15) / 16 > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    const int nb = (int)(k / 32), mp = sm_rows(m);
    if (small_m_mfma_shared(m, n, k)) { // m > 4: 8, 16 or 32 staged rows
        if (mp == 8)
            launch_sh<8>(w, xq, y, m, n, nb, s);
        else if (mp == 16)
            launch_sh<16>(w, xq, y, m, n, nb, s);
        else
            launch_sh<32>(w, xq, y, m, n, nb, s);
    } else if (small_m_mfma_row_tiles(m, n, k) == 2) { // m > 16: 32 staged rows
        if (small_m_mfma_split(m, n, k) == 1)
            launch_sm<2, 32, 1>(w, xq, y, m, n, nb, s);
        else
            launch_sm<2, 32, 2>(w, xq, y, m, n, nb, s);
    } else {
        const int ks = small_m_mfma_split(m, n, k);
        switch (mp) {
        case 4: launch_sm_ks<4>(ks, w, xq, y, m, n, nb, s); break;
        case 8: launch_sm_ks<8>(ks, w, xq, y, m, n, nb, s); break;
        case 16: launch_sm_ks<16>(ks, w, xq, y, m, n, nb, s); break;
        default: launch_sm_ks<32>(ks, w, xq, y, m, n, nb, s); break;
        }
    }
    return hipGetLastError();
}

} // namespace qll
