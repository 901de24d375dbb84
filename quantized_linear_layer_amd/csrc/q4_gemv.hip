// Q4_0 x Q8_0 decode GEMV, m = 1 (llama.cpp visual guide lesson 31 "CPU
// backend", "How the quantized dot product works"): for each weight row j and
// 32-block b,
//     sumi = sum_t (q_w - 8) * q_x          exact int32
//     y_j += f32(d_w) * f32(d_x) * sumi     f32
// Decode is bandwidth-bound (Fucina course "Chapter 06", 6.1: each weight
// byte feeds one multiply-add), so the kernel is built to stream W once:
//
//  * The activation row is decoded once per workgroup into LDS as aligned
//    structure-of-arrays: 32 code bytes, d_x as f32 and the correction
//    c8 = -8 * sum_t q_x per block, so that sum_t (q_w - 8) q_x =
//    c8 + sum_t q_w q_x needs no per-weight subtraction.
//  * A row of W is n_b * 18 bytes.  When n_b is even each lane takes a PAIR of
//    blocks (36 bytes = 9 dwords, dword aligned: two dwordx4 loads and one
//    dword load, every byte used); otherwise one block through a 5-dword
//    window.  L lanes share a row (64/L rows per wave); unit u of a row goes to
//    lane u mod L, four units in flight per lane.
//  * The nibbles are unpacked in registers (mask / shift-mask) and fed to
//    v_dot4_i32_i8 against the activation dwords: low nibbles of qs dword i are
//    elements 4i..4i+3, high nibbles elements 16+4i..16+4i+3.
//  * A row's partial sums are combined across its L lanes by xor-shuffles.
#include "common.h"

namespace qll {

struct Q4Unit {
    uint32_t d[2];
    uint32_t qs[2][4];
};

// Pair of Q4_0 blocks from 9 dwords starting at a dword-aligned address.
__device__ __forceinline__ void load_q4_pair(const uint8_t *p, uint32_t w[9])
{
    u32x4 a = load4_a4(p), b = load4_a4(p + 16);
    w[0] = a[0]; w[1] = a[1]; w[2] = a[2]; w[3] = a[3];
    w[4] = b[0]; w[5] = b[1]; w[6] = b[2]; w[7] = b[3];
    w[8] = *reinterpret_cast<const uint32_t *>(p + 32);
}

__device__ __forceinline__ void decode_q4_pair(const uint32_t w[9], Q4Unit &u)
{
    // block A: bytes 0..17 -> d = bytes 0..1, qs = bytes 2..17
    u.d[0] = w[0] & 0xffffu;
#pragma unroll
    for (int i = 0; i < 4; i++)
        u.qs[0][i] = funnel(w[i + 1], w[i], 16);
    // block B: bytes 18..35 -> d = bytes 18..19 (high half of dword 4), qs = dwords 5..8
    u.d[1] = w[4] >> 16;
#pragma unroll
    for (int i = 0; i < 4; i++)
        u.qs[1][i] = w[5 + i];
}

// One Q4_0 block at byte offset o (o % 4 is 0 or 2) of `base`.  Reads only the
// block's bytes and, when o % 4 == 2, the two bytes before it (o >= 18 then).
__device__ __forceinline__ void load_q4_single(const uint8_t *base, int64_t o, uint32_t w[5])
{
    if ((o & 3) == 0) {
        u32x4 a = load4_a4(base + o);
        w[0] = a[0]; w[1] = a[1]; w[2] = a[2]; w[3] = a[3];
        w[4] = *reinterpret_cast<const uint16_t *>(base + o + 16);
    } else {
        u32x4 a = load4_a4(base + o - 2);
        w[0] = a[0]; w[1] = a[1]; w[2] = a[2]; w[3] = a[3];
        w[4] = *reinterpret_cast<const uint32_t *>(base + o + 14);
    }
}

__device__ __forceinline__ void decode_q4_single(const uint32_t w[5], bool odd, Q4Unit &u)
{
    if (!odd) {
        u.d[0] = w[0] & 0xffffu;
#pragma unroll
        for (int i = 0; i < 4; i++)
            u.qs[0][i] = funnel(w[i + 1], w[i], 16);
    } else {
        u.d[0] = w[0] >> 16;
#pragma unroll
        for (int i = 0; i < 4; i++)
            u.qs[0][i] = w[i + 1];
    }
}

struct ActLds {
    const u32x4 *qs; // [nb][2] : elements 0..15, 16..31
    const float *dx; // [nb]
    const int *c8;   // [nb]  -8 * sum_t q_x
};

__device__ __forceinline__ float q4_block_dot(uint32_t dbits, const uint32_t qs[4], const ActLds &a, int b)
{
    const u32x4 xlo = a.qs[2 * b], xhi = a.qs[2 * b + 1];
    int s = a.c8[b];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        s = sdot4(qs[i] & 0x0f0f0f0fu, xlo[i], s);
        s = sdot4((qs[i] >> 4) & 0x0f0f0f0fu, xhi[i], s);
    }
    return half_bits_to_float(dbits) * a.dx[b] * (float)s;
}

// Decode the Q8_0 activation row into LDS (all threads of the workgroup).
// Split in two so that a kernel can issue the activation loads BEFORE its
// weight loads: loads retire in order, so waiting for activation bytes that
// were requested after the weights would also wait for the weights.
constexpr int kStageRegs = 2; // blocks per thread held in registers (nb <= 2 * blockDim)

struct ActRaw {
    uint32_t w[kStageRegs][9]; // raw dword window of each block, decoded later
    uint32_t tail[kStageRegs]; // the block's last two bytes
};

// Block b starts at byte 34b: dword aligned for even b, 2 bytes past a dword
// for odd b.  Every block loads the nine dwords from floor(34b / 4) with the
// same code (no divergent branch, so nothing waits for these loads until
// stage_q8_finish), plus the block's last two bytes as a u16.  An even block
// uses that u16 in place of its ninth dword, which for the last block of the
// row would lie past the end of the buffer (its index is clamped here).
__device__ __forceinline__ void stage_q8_load(const uint8_t *xq, int nb, ActRaw &raw)
{
    const uint32_t *p = reinterpret_cast<const uint32_t *>(xq);
    const int64_t max_dw = (int64_t)nb * 34 / 4 - 1;
#pragma unroll
    for (int i = 0; i < kStageRegs; i++) {
        // unconditional loads (threads past the row end reload the last block,
        // which stage_q8_finish then ignores): a branch here would make the
        // compiler wait for these loads at its join
        int b = threadIdx.x + i * blockDim.x;
        b = b < nb ? b : nb - 1;
        const int64_t a = ((int64_t)b * 34 - 2 * (b & 1)) / 4;
#pragma unroll
        for (int e = 0; e < 8; e++)
            raw.w[i][e] = p[a + e];
        raw.w[i][8] = p[a + 8 <= max_dw ? a + 8 : max_dw];
        raw.tail[i] = *reinterpret_cast<const uint16_t *>(xq + (int64_t)b * 34 + 32);
    }
}

__device__ __forceinline__ void decode_q8_window(const uint32_t w[9], bool odd, uint32_t &d, uint32_t q[8])
{
    // even block: d = low half of dword 0, codes shifted by two bytes;
    // odd block: d = high half of dword 0, codes are dwords 1..8
    const uint32_t sh = odd ? 0u : 16u;
    d = odd ? (w[0] >> 16) : (w[0] & 0xffffu);
#pragma unroll
    for (int i = 0; i < 8; i++)
        q[i] = funnel(w[i + 1], odd ? w[i + 1] : w[i], sh);
}

__device__ __forceinline__ void stage_q8_store_block(int b, uint32_t d, const uint32_t q[8], int nb, bool store,
                                                     void *smem)
{
    u32x4 *s_qs = reinterpret_cast<u32x4 *>(smem);
    float *s_dx = reinterpret_cast<float *>(s_qs + 2 * nb);
    int *s_c8 = reinterpret_cast<int *>(s_dx + nb);
    int sx = 0;
#pragma unroll
    for (int i = 0; i < 8; i++)
        sx = sdot4(q[i], 0x01010101u, sx);
    const float dx = half_bits_to_float(d);
    if (store) {
        s_qs[2 * b] = u32x4{q[0], q[1], q[2], q[3]};
        s_qs[2 * b + 1] = u32x4{q[4], q[5], q[6], q[7]};
        s_dx[b] = dx;
        s_c8[b] = -8 * sx;
    }
}

// Writes the blocks held in `raw`, stages any remaining blocks directly (only
// when nb > kStageRegs * blockDim), and synchronises the workgroup.
__device__ __forceinline__ ActLds stage_q8_finish(const uint8_t *xq, int nb, const ActRaw &raw,
                                                  void *smem)
{
    // decode unconditionally (only the stores are guarded): a use inside a
    // branch would let the compiler sink the loads past the weight loads
#pragma unroll
    for (int i = 0; i < kStageRegs; i++) {
        const int b = threadIdx.x + i * blockDim.x;
        const int bc = b < nb ? b : nb - 1;
        uint32_t w9[9];
#pragma unroll
        for (int e = 0; e < 9; e++)
            w9[e] = raw.w[i][e];
        w9[8] = (bc & 1) ? w9[8] : raw.tail[i];
        uint32_t d, q[8];
        decode_q8_window(w9, (bc & 1) != 0, d, q);
        stage_q8_store_block(bc, d, q, nb, b < nb, smem);
    }
    for (int b = threadIdx.x + kStageRegs * blockDim.x; b < nb; b += blockDim.x) {
        uint32_t d, q[8];
        load_q8_0_block(xq, (int64_t)b * 34, d, q);
        stage_q8_store_block(b, d, q, nb, true, smem);
    }
    __syncthreads();
    u32x4 *s_qs = reinterpret_cast<u32x4 *>(smem);
    float *s_dx = reinterpret_cast<float *>(s_qs + 2 * nb);
    int *s_c8 = reinterpret_cast<int *>(s_dx + nb);
    return ActLds{s_qs, s_dx, s_c8};
}

// The f32 activation row of the quantize-fused entry, quantized to Q8_0
// while it is staged, with exactly the arithmetic of quantize_q8_0_kernel:
// eight lanes per block (four values each; groups of eight consecutive
// threads share a block), amax by xor-shuffles over the eight, d = amax / 127
// and codes round-half-away(x / d) in IEEE f32, the stored binary16 d widened
// back to f32 for the dot.  The LDS layout is stage_q8_finish's, so the dot
// that follows sees the same values as after qll_quantize_q8_0.
constexpr int kStageF32Regs = 4; // 16-byte pieces per thread held in registers (k <= 4096 at 256 threads)

struct ActRawF32 {
    u32x4 v[kStageF32Regs];
};

__device__ __forceinline__ void stage_f32_load(const float *x, int nb, ActRawF32 &raw)
{
    const u32x4 *xv = reinterpret_cast<const u32x4 *>(x);
    const int pieces = nb * 8;
#pragma unroll
    for (int j = 0; j < kStageF32Regs; j++) {
        const int p = threadIdx.x + j * blockDim.x;
        raw.v[j] = xv[p < pieces ? p : 0]; // unconditional (see stage_q8_load)
    }
}

__device__ __forceinline__ void stage_f32_piece(u32x4 raw, int p, int nb, void *smem)
{
    u32x4 *s_qs = reinterpret_cast<u32x4 *>(smem);
    float *s_dx = reinterpret_cast<float *>(s_qs + 2 * nb);
    int *s_c8 = reinterpret_cast<int *>(s_dx + nb);
    const int b = p >> 3, sub = p & 7;
    const bool ok = b < nb;
    // named components: a bit-cast of raw[e] inside an unrolled loop read
    // component 0 for every e in this compiler's output
    const float v[4] = {ok ? __uint_as_float(raw.x) : 0.0f, ok ? __uint_as_float(raw.y) : 0.0f,
                        ok ? __uint_as_float(raw.z) : 0.0f, ok ? __uint_as_float(raw.w) : 0.0f};
    float a = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
    a = fmaxf(a, __shfl_xor(a, 1));
    a = fmaxf(a, __shfl_xor(a, 2));
    a = fmaxf(a, __shfl_xor(a, 4));
    const float d = a / 127.0f;
    uint32_t q = 0u;
#pragma unroll
    for (int e = 0; e < 4; e++)
        q |= ((uint32_t)quant_code(v[e], d) & 0xffu) << (8 * e);
    int sx = sdot4(q, 0x01010101u, 0);
    sx += __shfl_xor(sx, 1);
    sx += __shfl_xor(sx, 2);
    sx += __shfl_xor(sx, 4);
    if (ok) {
        reinterpret_cast<uint32_t *>(s_qs)[8 * b + sub] = q; // codes 4 sub .. 4 sub + 3 of block b
        if (sub == 0) {
            s_dx[b] = half_bits_to_float(float_to_half_bits(d));
            s_c8[b] = -8 * sx;
        }
    }
}

__device__ __forceinline__ ActLds stage_f32_finish(const float *x, int nb, const ActRawF32 &raw, void *smem)
{
#pragma unroll
    for (int j = 0; j < kStageF32Regs; j++)
        stage_f32_piece(raw.v[j], threadIdx.x + j * blockDim.x, nb, smem);
    // every thread of the workgroup runs the same trip count, so the
    // eight-lane shuffles always see whole groups
    const u32x4 *xv = reinterpret_cast<const u32x4 *>(x);
    const int pieces = nb * 8;
    for (int p0 = kStageF32Regs * blockDim.x; p0 < pieces; p0 += blockDim.x) {
        const int p = p0 + threadIdx.x;
        stage_f32_piece(xv[p < pieces ? p : 0], p, nb, smem);
    }
    __syncthreads();
    u32x4 *s_qs = reinterpret_cast<u32x4 *>(smem);
    float *s_dx = reinterpret_cast<float *>(s_qs + 2 * nb);
    int *s_c8 = reinterpret_cast<int *>(s_dx + nb);
    return ActLds{s_qs, s_dx, s_c8};
}

constexpr int kGemvThreads = 256;

// One work item of a wave: a group of R = 64/L rows and a chunk of U * L
// consecutive units of those rows (U per lane).
template <int U>
struct GemvRaw {
    uint32_t w[U][9];
};

template <int L, int U, bool PAIR>
__device__ __forceinline__ void gemv_load(const uint8_t *__restrict__ w, int64_t row, int64_t n, int64_t row_bytes,
                                          int nu, int ubase, int r, GemvRaw<U> &raw)
{
#pragma unroll
    for (int i = 0; i < U; i++) {
        // Units outside the matrix load the first unit of row 0 instead (and
        // are masked in gemv_compute): unconditional loads let the compiler
        // count them, so waits for earlier loads do not drain these.
        int u = ubase + r + i * L;
        const bool ok = row < n && u < nu;
        const int64_t rr = ok ? row : 0;
        u = ok ? u : 0;
        if (PAIR) {
            load_q4_pair(w + rr * row_bytes + (int64_t)u * 36, raw.w[i]);
        } else {
            load_q4_single(w, rr * row_bytes + (int64_t)u * 18, raw.w[i]);
        }
    }
}

template <int L, int U, bool PAIR>
__device__ __forceinline__ float gemv_compute(const GemvRaw<U> &raw, int64_t row, int64_t n, int64_t row_bytes,
                                              int nu, int ubase, int r, const ActLds &act)
{
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < U; i++) {
        const int u = ubase + r + i * L;
        if (row < n && u < nu) {
            Q4Unit unit;
            if (PAIR) {
                decode_q4_pair(raw.w[i], unit);
                acc += q4_block_dot(unit.d[0], unit.qs[0], act, 2 * u);
                acc += q4_block_dot(unit.d[1], unit.qs[1], act, 2 * u + 1);
            } else {
                const int64_t o = row * row_bytes + (int64_t)u * 18;
                decode_q4_single(raw.w[i], (o & 3) != 0, unit);
                acc += q4_block_dot(unit.d[0], unit.qs[0], act, u);
            }
        }
    }
    return acc;
}

// Persistent over work items: each wave walks the row groups
// wave_id, wave_id + total_waves, ... and, within a row group, its chunks in
// order; the next item's weight bytes are loaded while the current one is
// computed.  The activation loads are issued first, then the first item's
// weight loads, then the activation is decoded into LDS: loads complete in
// order, so the staging waits only for its own bytes and HBM traffic starts
// at once.  (xq is deliberately not __restrict__: with it, the compiler may
// move the activation loads past the barrier that keeps them ahead.)
template <int L, int U, bool PAIR, bool F32>
__global__ __launch_bounds__(kGemvThreads) void q4_0_q8_0_gemv_kernel(const uint8_t *__restrict__ w,
                                                                      const void *xin,
                                                                      float *__restrict__ y, int64_t n, int nb)
{
    extern __shared__ u32x4 smem[];
    constexpr int R = 64 / L; // rows per wave
    constexpr int WAVES = kGemvThreads / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane / L, r = lane % L;
    const int nu = PAIR ? nb / 2 : nb;
    const int chunk_units = U * L;
    const int chunks = (nu + chunk_units - 1) / chunk_units;
    const int64_t row_bytes = (int64_t)nb * 18;
    const int64_t n_groups = (n + R - 1) / R;
    const int64_t stride = (int64_t)gridDim.x * WAVES;

    const uint8_t *xq = static_cast<const uint8_t *>(xin);
    const float *xf = static_cast<const float *>(xin);
    ActRaw araw;
    ActRawF32 fraw;
    if (F32)
        stage_f32_load(xf, nb, fraw);
    else
        stage_q8_load(xq, nb, araw);
    asm volatile("" ::: "memory"); // keep these loads ahead of the weight loads

    int64_t grp = (int64_t)blockIdx.x * WAVES + wave;
    int c = 0;
    GemvRaw<U> cur;
    // unconditional (a wave without work loads masked dummies): see gemv_load
    gemv_load<L, U, PAIR>(w, grp * R + g, n, row_bytes, nu, 0, r, cur);

    const ActLds act = F32 ? stage_f32_finish(xf, nb, fraw, smem) : stage_q8_finish(xq, nb, araw, smem);

    float acc = 0.0f;
    while (grp < n_groups) {
        int64_t grp2 = grp;
        int c2 = c + 1;
        if (c2 == chunks) {
            c2 = 0;
            grp2 += stride;
        }
        GemvRaw<U> nxt;
        if (grp2 < n_groups)
            gemv_load<L, U, PAIR>(w, grp2 * R + g, n, row_bytes, nu, c2 * chunk_units, r, nxt);
        const int64_t row = grp * R + g;
        acc += gemv_compute<L, U, PAIR>(cur, row, n, row_bytes, nu, c * chunk_units, r, act);
        if (c == chunks - 1) {
#pragma unroll
            for (int off = L / 2; off > 0; off >>= 1)
                acc += __shfl_xor(acc, off);
            if (row < n && r == 0)
                y[row] = acc;
            acc = 0.0f;
        }
        cur = nxt;
        grp = grp2;
        c = c2;
    }
}

size_t q4_gemv_lds_bytes(int nb) { return (size_t)nb * 40; }

constexpr int64_t kF32GemvGrid = 512;

// One work item per wave: the dispatcher starts new workgroups as others
// finish, which measured faster on the 296 MB vocabulary projection than
// looping resident waves over items (47 vs 53 us), and equal on one-pass
// shapes.  The kernel still loops if the grid limit were ever reached.
template <int L, int U, bool PAIR, bool F32>
static hipError_t launch_l(const uint8_t *w, const void *xin, float *y, int64_t n, int nb, hipStream_t s)
{
    constexpr int R = 64 / L;
    const int64_t groups = (n + R - 1) / R;
    int64_t grid = (groups + kGemvThreads / 64 - 1) / (kGemvThreads / 64);
    // f32 rows: every workgroup quantizes the whole row, so at most two
    // workgroups per CU, each looping over its rows, quantize it (measured
    // against one item per wave: 11 vs 14 us on 4096 -> 14336, 57 vs 72 us
    // on the 296 MB vocabulary projection)
    if (F32 && grid > kF32GemvGrid)
        grid = kF32GemvGrid;
    if (grid > 0x7fffffff)
        grid = 0x7fffffff;
    hipLaunchKernelGGL((q4_0_q8_0_gemv_kernel<L, U, PAIR, F32>), dim3((unsigned)grid), dim3(kGemvThreads),
                       q4_gemv_lds_bytes(nb), s, w, xin, y, n, nb);
    return hipGetLastError();
}

template <bool PAIR, bool F32 = false>
static hipError_t launch_pair(const uint8_t *w, const void *xq, float *y, int64_t n, int nb, hipStream_t s)
{
    const int nu = PAIR ? nb / 2 : nb;
    // Lanes per row (8..64).  A matrix that fits in one pass of the resident
    // waves gets about two units per lane (more, lighter waves: a shorter
    // compute tail after the last bytes land); a larger one about four (less
    // per-row overhead in the persistent loop).
    if (n <= 16384) {
        if (nu > 64)
            return launch_l<64, 4, PAIR, F32>(w, xq, y, n, nb, s);
        if (nu > 32)
            return launch_l<32, 2, PAIR, F32>(w, xq, y, n, nb, s);
        if (nu > 16)
            return launch_l<16, 2, PAIR, F32>(w, xq, y, n, nb, s);
        return launch_l<8, 2, PAIR, F32>(w, xq, y, n, nb, s);
    }
    if (nu > 128)
        return launch_l<64, 4, PAIR, F32>(w, xq, y, n, nb, s);
    if (nu > 64)
        return launch_l<32, 4, PAIR, F32>(w, xq, y, n, nb, s);
    if (nu > 32)
        return launch_l<16, 4, PAIR, F32>(w, xq, y, n, nb, s);
    return launch_l<8, 4, PAIR, F32>(w, xq, y, n, nb, s);
}

hipError_t launch_q4_0_q8_0_gemv(const uint8_t *w, const uint8_t *xq, float *y, int64_t n, int64_t k,
                                 hipStream_t s)
{
    const int nb = (int)(k / 32);
    if (nb % 2 == 0)
        return launch_pair<true>(w, xq, y, n, nb, s);
    return launch_pair<false>(w, xq, y, n, nb, s);
}

// ------------------------------------------------------------------ decode-packed Q4_0 weights
// A load-time layout for the decode GEMV (the packed right-hand side of the
// Fucina reference "Backends", 9.7, rewritten once and reused by every
// call; aligned 128-bit loads in place of the 18-byte block stride): each
// row as two planes -- the nb blocks' 16 nibble bytes (Q4_0 order), 16 * nb
// bytes, then their nb binary16 scales, padded to a multiple of 16 bytes
// (8 scales) with zeros.  A row stays at 18 bytes per block when nb % 8 == 0.
// In the GEMV, lane r of the L lanes of a row takes blocks r, r + L, ...,
// so each load instruction of a wave reads consecutive 16-byte nibble
// pieces (and consecutive 2-byte scales): the whole instruction is a few
// cache lines, where a lane-private stride (an AoS unit or an interleaved
// group per lane) spreads one instruction over tens of lines.
__host__ __device__ inline int64_t q4p_row_bytes(int nb) { return 16 * (int64_t)nb + 16 * (int64_t)((nb + 7) / 8); }

template <int U>
struct Q4pRaw {
    u32x4 q[U];    // nibbles of the lane's U blocks
    uint32_t d[U]; // their binary16 scales (low half)
};

template <int L, int U>
__device__ __forceinline__ void q4p_load(const uint8_t *__restrict__ w, int64_t row, int64_t n, int64_t row_bytes,
                                         int nb, int bbase, int r, Q4pRaw<U> &raw)
{
#pragma unroll
    for (int i = 0; i < U; i++) {
        // blocks outside the matrix load block 0 of row 0 instead (masked in
        // q4p_compute): unconditional loads keep the wait counts exact
        int b = bbase + r + i * L;
        const bool ok = row < n && b < nb;
        const int64_t rr = ok ? row : 0;
        b = ok ? b : 0;
        const uint8_t *base = w + rr * row_bytes;
        raw.q[i] = *reinterpret_cast<const u32x4 *>(base + 16 * (int64_t)b);
        raw.d[i] = *reinterpret_cast<const uint16_t *>(base + 16 * (int64_t)nb + 2 * b);
    }
}

template <int L, int U>
__device__ __forceinline__ float q4p_compute(const Q4pRaw<U> &raw, int64_t row, int64_t n, int nb, int bbase, int r,
                                             const ActLds &act)
{
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < U; i++) {
        const int b = bbase + r + i * L;
        if (row < n && b < nb) {
            const uint32_t qs[4] = {raw.q[i][0], raw.q[i][1], raw.q[i][2], raw.q[i][3]};
            acc += q4_block_dot(raw.d[i], qs, act, b);
        }
    }
    return acc;
}

// The GEMV kernel's structure on the packed layout: L lanes per row, U
// blocks per lane and work item, the next item's bytes in flight while the
// current one is dotted.
template <int L, int U>
__global__ __launch_bounds__(kGemvThreads) void q4_0_packed_gemv_kernel(const uint8_t *__restrict__ w, const void *xin,
                                                                        float *__restrict__ y, int64_t n, int nb)
{
    extern __shared__ u32x4 smem[];
    constexpr int R = 64 / L, WAVES = kGemvThreads / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane / L, r = lane % L;
    const int chunk = U * L;
    const int chunks = (nb + chunk - 1) / chunk;
    const int64_t row_bytes = q4p_row_bytes(nb);
    const int64_t n_groups = (n + R - 1) / R;
    const int64_t stride = (int64_t)gridDim.x * WAVES;

    const uint8_t *xq = static_cast<const uint8_t *>(xin);
    ActRaw araw;
    stage_q8_load(xq, nb, araw);
    asm volatile("" ::: "memory"); // keep these loads ahead of the weight loads

    int64_t grp = (int64_t)blockIdx.x * WAVES + wave;
    int c = 0;
    Q4pRaw<U> cur;
    q4p_load<L, U>(w, grp * R + g, n, row_bytes, nb, 0, r, cur);

    const ActLds act = stage_q8_finish(xq, nb, araw, smem);

    float acc = 0.0f;
    while (grp < n_groups) {
        int64_t grp2 = grp;
        int c2 = c + 1;
        if (c2 == chunks) {
            c2 = 0;
            grp2 += stride;
        }
        Q4pRaw<U> nxt;
        if (grp2 < n_groups)
            q4p_load<L, U>(w, grp2 * R + g, n, row_bytes, nb, c2 * chunk, r, nxt);
        const int64_t row = grp * R + g;
        acc += q4p_compute<L, U>(cur, row, n, nb, c * chunk, r, act);
        if (c == chunks - 1) {
#pragma unroll
            for (int off = L / 2; off > 0; off >>= 1)
                acc += __shfl_xor(acc, off);
            if (row < n && r == 0)
                y[row] = acc;
            acc = 0.0f;
        }
        cur = nxt;
        grp = grp2;
        c = c2;
    }
}

template <int L, int U>
static hipError_t launch_q4p_l(const uint8_t *w, const uint8_t *xq, float *y, int64_t n, int nb, hipStream_t s)
{
    constexpr int R = 64 / L;
    const int64_t groups = (n + R - 1) / R;
    int64_t grid = (groups + kGemvThreads / 64 - 1) / (kGemvThreads / 64);
    if (grid > 0x7fffffff)
        grid = 0x7fffffff;
    hipLaunchKernelGGL((q4_0_packed_gemv_kernel<L, U>), dim3((unsigned)grid), dim3(kGemvThreads),
                       q4_gemv_lds_bytes(nb), s, w, xq, y, n, nb);
    return hipGetLastError();
}

hipError_t launch_q4_0_packed_gemv(const uint8_t *w, const uint8_t *xq, float *y, int64_t n, int64_t k,
                                   hipStream_t s)
{
    const int nb = (int)(k / 32);
    // the direct GEMV's lane counts, with a lane's units of two blocks as
    // two blocks
    if (n <= 16384) {
        if (nb > 128)
            return launch_q4p_l<64, 8>(w, xq, y, n, nb, s);
        if (nb > 64)
            return launch_q4p_l<32, 4>(w, xq, y, n, nb, s);
        if (nb > 32)
            return launch_q4p_l<16, 4>(w, xq, y, n, nb, s);
        return launch_q4p_l<8, 4>(w, xq, y, n, nb, s);
    }
    if (nb > 256)
        return launch_q4p_l<64, 8>(w, xq, y, n, nb, s);
    if (nb > 128)
        return launch_q4p_l<32, 8>(w, xq, y, n, nb, s);
    if (nb > 64)
        return launch_q4p_l<16, 8>(w, xq, y, n, nb, s);
    return launch_q4p_l<8, 8>(w, xq, y, n, nb, s);
}

size_t q4_0_packed_bytes(int64_t n, int64_t k) { return (size_t)(n * q4p_row_bytes((int)(k / 32))); }

// One 16-byte piece of the packed layout per thread: piece p < nb of a row
// is block p's nibbles, piece nb + t the scales of blocks 8t .. 8t + 7.
__global__ __launch_bounds__(256) void q4_0_pack_decode_kernel(const uint8_t *__restrict__ w, uint8_t *__restrict__ wp,
                                                               int64_t n, int nb)
{
    const int per_row = nb + (nb + 7) / 8;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n * per_row)
        return;
    const int64_t row = i / per_row;
    const int p = (int)(i % per_row);
    uint32_t out[4] = {0u, 0u, 0u, 0u};
    if (p < nb) {
        const uint8_t *src = w + (row * nb + p) * 18 + 2;
#pragma unroll
        for (int e = 0; e < 16; e++)
            out[e >> 2] |= (uint32_t)src[e] << (8 * (e & 3));
    } else {
#pragma unroll
        for (int b = 0; b < 8; b++) {
            const int blk = 8 * (p - nb) + b;
            if (blk < nb) {
                const uint8_t *src = w + (row * nb + blk) * 18;
                out[b >> 1] |= ((uint32_t)src[0] | ((uint32_t)src[1] << 8)) << (16 * (b & 1));
            }
        }
    }
    reinterpret_cast<u32x4 *>(wp)[i] = u32x4{out[0], out[1], out[2], out[3]};
}

hipError_t launch_q4_0_pack_decode(const uint8_t *w, uint8_t *wp, int64_t n, int64_t k, hipStream_t s)
{
    const int nb = (int)(k / 32);
    const int64_t pieces = n * (nb + (nb + 7) / 8);
    const int64_t grid = (pieces + 255) / 256;
    if (grid > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(q4_0_pack_decode_kernel, dim3((unsigned)grid), dim3(256), 0, s, w, wp, n, nb);
    return hipGetLastError();
}

// ------------------------------------------------------------------ Q8_0 weights
// Decode GEMV with the weights quantized to Q8_0 blocks as well (Fucina
// reference "Backends", 9.7: a Q8_0-quantized right-hand side against the
// per-call Q8_0 activation): for each row j and block b
//     sumi = sum_t q_w * q_x            exact int32 (no offset: codes are signed)
//     y_j += f32(d_w) * f32(d_x) * sumi f32
// Same structure as the Q4_0 kernel above: the activation staged once per
// workgroup in LDS, L lanes per row, a lane's unit a PAIR of 34-byte blocks
// (68 bytes = 17 dwords, dword aligned when the row's block count is even:
// four dwordx4 loads and one dword load, every byte used) or, for an odd
// block count, one block through a 9-dword window.

template <int U>
struct Q8wRaw {
    uint32_t w[U][17];
};

__device__ __forceinline__ void load_q8w_pair(const uint8_t *p, uint32_t w[17])
{
#pragma unroll
    for (int c = 0; c < 4; c++) {
        const u32x4 v = load4_a4(p + 16 * c);
#pragma unroll
        for (int e = 0; e < 4; e++)
            w[4 * c + e] = v[e];
    }
    w[16] = *reinterpret_cast<const uint32_t *>(p + 64);
}

// One Q8_0 block at byte offset o (o % 4 is 0 or 2) of `base`: the nine
// dwords from o - (o & 3), except that for o % 4 == 0 the ninth is replaced by
// the block's last two bytes (the dword would reach past the block, and past
// the buffer for its last block).
__device__ __forceinline__ void load_q8w_single(const uint8_t *base, int64_t o, uint32_t w[17])
{
    const uint8_t *p = base + (o & ~(int64_t)3);
    const u32x4 a = load4_a4(p), b = load4_a4(p + 16);
#pragma unroll
    for (int e = 0; e < 4; e++) {
        w[e] = a[e];
        w[4 + e] = b[e];
    }
    w[8] = (o & 3) ? *reinterpret_cast<const uint32_t *>(p + 32)
                   : (uint32_t)*reinterpret_cast<const uint16_t *>(base + o + 32);
}

__device__ __forceinline__ float q8w_block_dot(uint32_t dbits, const uint32_t qs[8], const ActLds &a, int b)
{
    const u32x4 xlo = a.qs[2 * b], xhi = a.qs[2 * b + 1];
    int s = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        s = sdot4(qs[i], xlo[i], s);
        s = sdot4(qs[4 + i], xhi[i], s);
    }
    return half_bits_to_float(dbits) * a.dx[b] * (float)s;
}

template <int L, int U, bool PAIR>
__device__ __forceinline__ void q8w_load(const uint8_t *__restrict__ w, int64_t row, int64_t n, int64_t row_bytes,
                                         int nu, int ubase, int r, Q8wRaw<U> &raw)
{
#pragma unroll
    for (int i = 0; i < U; i++) {
        // out-of-range units load the first unit of row 0 (masked later), so
        // the loads stay unconditional
        int u = ubase + r + i * L;
        const bool ok = row < n && u < nu;
        const int64_t rr = ok ? row : 0;
        u = ok ? u : 0;
        if (PAIR)
            load_q8w_pair(w + rr * row_bytes + (int64_t)u * 68, raw.w[i]);
        else
            load_q8w_single(w, rr * row_bytes + (int64_t)u * 34, raw.w[i]);
    }
}

template <int L, int U, bool PAIR>
__device__ __forceinline__ float q8w_compute(const Q8wRaw<U> &raw, int64_t row, int64_t n, int64_t row_bytes, int nu,
                                             int ubase, int r, const ActLds &act)
{
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < U; i++) {
        const int u = ubase + r + i * L;
        if (row < n && u < nu) {
            const uint32_t *w = raw.w[i];
            uint32_t q[8];
            if (PAIR) {
#pragma unroll
                for (int e = 0; e < 8; e++)
                    q[e] = funnel(w[e + 1], w[e], 16); // block A: bytes 2..33
                acc += q8w_block_dot(w[0] & 0xffffu, q, act, 2 * u);
                acc += q8w_block_dot(w[8] >> 16, w + 9, act, 2 * u + 1); // block B: d at 34, codes from 36
            } else {
                const bool odd = ((row * row_bytes + (int64_t)u * 34) & 3) != 0;
#pragma unroll
                for (int e = 0; e < 8; e++)
                    q[e] = odd ? w[e + 1] : funnel(w[e + 1], w[e], 16);
                acc += q8w_block_dot(odd ? (w[0] >> 16) : (w[0] & 0xffffu), q, act, u);
            }
        }
    }
    return acc;
}

// Persistent over work items exactly as q4_0_q8_0_gemv_kernel (same staging,
// same ordering of the activation and weight loads).
template <int L, int U, bool PAIR>
__global__ __launch_bounds__(kGemvThreads) void q8_0_q8_0_gemv_kernel(const uint8_t *__restrict__ w,
                                                                      const uint8_t *xq, float *__restrict__ y,
                                                                      int64_t n, int nb)
{
    extern __shared__ u32x4 smem[];
    constexpr int R = 64 / L;
    constexpr int WAVES = kGemvThreads / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane / L, r = lane % L;
    const int nu = PAIR ? nb / 2 : nb;
    const int chunk_units = U * L;
    const int chunks = (nu + chunk_units - 1) / chunk_units;
    const int64_t row_bytes = (int64_t)nb * 34;
    const int64_t n_groups = (n + R - 1) / R;
    const int64_t stride = (int64_t)gridDim.x * WAVES;

    ActRaw araw;
    stage_q8_load(xq, nb, araw);
    asm volatile("" ::: "memory");

    int64_t grp = (int64_t)blockIdx.x * WAVES + wave;
    int c = 0;
    Q8wRaw<U> cur;
    q8w_load<L, U, PAIR>(w, grp * R + g, n, row_bytes, nu, 0, r, cur);

    const ActLds act = stage_q8_finish(xq, nb, araw, smem);

    float acc = 0.0f;
    while (grp < n_groups) {
        int64_t grp2 = grp;
        int c2 = c + 1;
        if (c2 == chunks) {
            c2 = 0;
            grp2 += stride;
        }
        Q8wRaw<U> nxt;
        if (grp2 < n_groups)
            q8w_load<L, U, PAIR>(w, grp2 * R + g, n, row_bytes, nu, c2 * chunk_units, r, nxt);
        const int64_t row = grp * R + g;
        acc += q8w_compute<L, U, PAIR>(cur, row, n, row_bytes, nu, c * chunk_units, r, act);
        if (c == chunks - 1) {
#pragma unroll
            for (int off = L / 2; off > 0; off >>= 1)
                acc += __shfl_xor(acc, off);
            if (row < n && r == 0)
                y[row] = acc;
            acc = 0.0f;
        }
        cur = nxt;
        grp = grp2;
        c = c2;
    }
}

template <int L, int U, bool PAIR>
static hipError_t launch_q8w_l(const uint8_t *w, const uint8_t *xq, float *y, int64_t n, int nb, hipStream_t s)
{
    constexpr int R = 64 / L;
    const int64_t groups = (n + R - 1) / R;
    int64_t grid = (groups + kGemvThreads / 64 - 1) / (kGemvThreads / 64);
    if (grid > 0x7fffffff)
        grid = 0x7fffffff;
    hipLaunchKernelGGL((q8_0_q8_0_gemv_kernel<L, U, PAIR>), dim3((unsigned)grid), dim3(kGemvThreads),
                       q4_gemv_lds_bytes(nb), s, w, xq, y, n, nb);
    return hipGetLastError();
}

// Lanes per row: enough for one pass over the row at two units per lane
// (a 68-byte unit is about twice a Q4_0 pair, so two units per lane carry the
// bytes that four Q4_0 units do), 64 lanes for longer rows.
template <bool PAIR>
static hipError_t launch_q8w_pair(const uint8_t *w, const uint8_t *xq, float *y, int64_t n, int nb, hipStream_t s)
{
    const int nu = PAIR ? nb / 2 : nb;
    if (nu > 64)
        return launch_q8w_l<64, 2, PAIR>(w, xq, y, n, nb, s);
    if (nu > 32)
        return launch_q8w_l<32, 2, PAIR>(w, xq, y, n, nb, s);
    if (nu > 16)
        return launch_q8w_l<16, 2, PAIR>(w, xq, y, n, nb, s);
    return launch_q8w_l<8, 2, PAIR>(w, xq, y, n, nb, s);
}

hipError_t launch_q8_0_q8_0_gemv(const uint8_t *w, const uint8_t *xq, float *y, int64_t n, int64_t k, hipStream_t s)
{
    const int nb = (int)(k / 32);
    if (nb % 2 == 0)
        return launch_q8w_pair<true>(w, xq, y, n, nb, s);
    return launch_q8w_pair<false>(w, xq, y, n, nb, s);
}

// ------------------------------------------------------------------ small m
// Y[i][j] for 1 <= m <= 8 activation rows (speculative or batched decode):
// every weight unit is loaded once and dotted with all M rows.  Per row and
// block the arithmetic is the same exact int32 sum and f32 scaling as the
// m = 1 kernel.  16 lanes share a group of kGmRW weight rows: a lane holds the
// same unit (pair of blocks) of each of the group's rows, so one LDS read of an
// activation block feeds kGmRW block dots (LDS reads per dot fall by that
// factor: at m = 8 they, not the weight bytes, bound a one-row-per-lane
// layout).  The activations are staged into LDS one k-chunk (32 blocks) at a
// time, so LDS holds M x 32 blocks whatever k is, once per workgroup of 64
// weight rows; the next chunk's activation bytes and weight units are loaded
// into registers while the current chunk is computed.  The activations come
// either as Q8_0 blocks or as f32 rows, quantized here exactly as
// quantize_q8_0_kernel does (amax, d = amax / 127 in f32, codes rounded half
// away from zero, d stored as binary16), so the f32 entry is the Q8_0
// quantization and the GEMV in one launch.
// Three layouts: RW = 4 rows x U = 1 unit per lane for large n (64 weight
// rows per workgroup), RW = 2 x 1 for mid-sized n at m > 2 (32 rows), and
// RW = 1 row x U = 4 units for smaller n, where taller workgroups would be
// too few to fill the chip.
constexpr int kGmL = 16;       // lanes per row group
constexpr int kGmThreads = 256;

template <int M, int U, bool PAIR>
struct GmLds {
    static constexpr int CB = kGmL * U * (PAIR ? 2 : 1); // blocks per chunk
    u32x4 qs[M][CB][2]; // codes 0..15, 16..31
    float dx[M][CB];
    int c8[M][CB];      // -8 * sum of the block's codes
};

// Raw activation bytes of one chunk, loaded without being looked at.
template <int M, int U, bool PAIR, bool F32>
struct GmRaw {
    static constexpr int CB = GmLds<M, U, PAIR>::CB;
    // Q8_0: one block per task (row-major over M x CB), its nine-dword window
    // and last two bytes; f32: eight lanes per block, four floats each
    static constexpr int TASKS = F32 ? M * CB * 8 : M * CB;
    static constexpr int T = (TASKS + kGmThreads - 1) / kGmThreads;
    uint32_t v[T][F32 ? 4 : 10];
};

template <int M, int U, bool PAIR, bool F32>
__device__ __forceinline__ void gm_act_load(const void *xin, int64_t m, int nb, int chunk,
                                            GmRaw<M, U, PAIR, F32> &raw)
{
    constexpr int CB = GmLds<M, U, PAIR>::CB, TASKS = GmRaw<M, U, PAIR, F32>::TASKS;
#pragma unroll
    for (int t = 0; t < GmRaw<M, U, PAIR, F32>::T; t++) {
        const int task = threadIdx.x + t * kGmThreads;
        if constexpr (F32) {
            const int blk = task >> 3, sub = task & 7;
            const int r = blk / CB, b = chunk * CB + blk % CB;
            const bool ok = task < TASKS && r < m && b < nb;
            const float *x = static_cast<const float *>(xin);
            const u32x4 v = *reinterpret_cast<const u32x4 *>(x + (ok ? ((int64_t)r * nb + b) * 32 + 4 * sub : 0));
#pragma unroll
            for (int e = 0; e < 4; e++)
                raw.v[t][e] = v[e];
        } else {
            const int r = task / CB, b = chunk * CB + task % CB;
            const bool ok = task < TASKS && r < m && b < nb;
            const int64_t g = ok ? (int64_t)r * nb + b : 0; // flat block index
            const uint8_t *xq = static_cast<const uint8_t *>(xin);
            const uint32_t *p = reinterpret_cast<const uint32_t *>(xq);
            const int64_t a = (g * 34 - 2 * (g & 1)) / 4;         // window start (dword)
            const int64_t max_dw = (m * (int64_t)nb * 34) / 4 - 1; // last whole dword of the buffer
#pragma unroll
            for (int e = 0; e < 8; e++)
                raw.v[t][e] = p[a + e];
            raw.v[t][8] = p[a + 8 <= max_dw ? a + 8 : max_dw];
            raw.v[t][9] = *reinterpret_cast<const uint16_t *>(xq + g * 34 + 32);
        }
    }
}

template <int M, int U, bool PAIR, bool F32>
__device__ __forceinline__ void gm_act_store(const GmRaw<M, U, PAIR, F32> &raw, int64_t m, int nb, int chunk,
                                             GmLds<M, U, PAIR> &s)
{
    constexpr int CB = GmLds<M, U, PAIR>::CB, TASKS = GmRaw<M, U, PAIR, F32>::TASKS;
#pragma unroll
    for (int t = 0; t < GmRaw<M, U, PAIR, F32>::T; t++) {
        const int task = threadIdx.x + t * kGmThreads;
        if constexpr (F32) {
            // every lane computes (the shuffles need all of them); tasks past
            // the chunk only skip their stores
            const int blk = task >> 3, sub = task & 7;
            const int r = blk / CB, bl = blk % CB;
            const bool ok = task < TASKS && r < m && chunk * CB + bl < nb;
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; e++)
                v[e] = ok ? __builtin_bit_cast(float, raw.v[t][e]) : 0.0f;
            float a = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
            a = fmaxf(a, __shfl_xor(a, 1));
            a = fmaxf(a, __shfl_xor(a, 2));
            a = fmaxf(a, __shfl_xor(a, 4));
            const float d = a / 127.0f;
            uint32_t q = 0u;
#pragma unroll
            for (int e = 0; e < 4; e++)
                q |= ((uint32_t)quant_code(v[e], d) & 0xffu) << (8 * e);
            int sx = sdot4(q, 0x01010101u, 0);
            sx += __shfl_xor(sx, 1);
            sx += __shfl_xor(sx, 2);
            sx += __shfl_xor(sx, 4);
            if (task < TASKS) {
                reinterpret_cast<uint32_t *>(&s.qs[r][bl][0])[sub] = q; // codes 4 sub .. 4 sub + 3
                if (sub == 0) {
                    s.dx[r][bl] = half_bits_to_float(float_to_half_bits(d));
                    s.c8[r][bl] = -8 * sx;
                }
            }
        } else {
            if (task >= TASKS)
                continue;
            const int r = task / CB, bl = task % CB, b = chunk * CB + bl;
            const bool ok = r < m && b < nb;
            const int64_t g = ok ? (int64_t)r * nb + b : 0;
            uint32_t w9[9];
#pragma unroll
            for (int e = 0; e < 9; e++)
                w9[e] = raw.v[t][e];
            if (!(g & 1))
                w9[8] = raw.v[t][9];
            uint32_t d, q[8];
            decode_q8_window(w9, (g & 1) != 0, d, q);
            int sx = 0;
#pragma unroll
            for (int e = 0; e < 8; e++)
                sx = sdot4(q[e], 0x01010101u, sx);
            s.qs[r][bl][0] = ok ? u32x4{q[0], q[1], q[2], q[3]} : u32x4{0u, 0u, 0u, 0u};
            s.qs[r][bl][1] = ok ? u32x4{q[4], q[5], q[6], q[7]} : u32x4{0u, 0u, 0u, 0u};
            s.dx[r][bl] = ok ? half_bits_to_float(d) : 0.0f;
            s.c8[r][bl] = ok ? -8 * sx : 0;
        }
    }
}

// This lane's units of the chunk (U of them, L apart) in each of the group's
// RW rows, dotted with the M staged activation rows.
template <int M, int RW, int U, bool PAIR>
__device__ __forceinline__ void gm_compute(const GemvRaw<U> raw[RW], int64_t row0, int64_t n, int64_t row_bytes,
                                           int nu, int ubase, int r, const GmLds<M, U, PAIR> &s, float acc[RW][M])
{
#pragma unroll
    for (int i = 0; i < U; i++) {
        const int u = ubase + r + i * kGmL;
        if (u >= nu)
            continue;
        Q4Unit unit[RW];
#pragma unroll
        for (int q = 0; q < RW; q++) {
            if (PAIR)
                decode_q4_pair(raw[q].w[i], unit[q]);
            else
                decode_q4_single(raw[q].w[i], (((row0 + q) * row_bytes + (int64_t)u * 18) & 3) != 0, unit[q]);
        }
#pragma unroll
        for (int h = 0; h < (PAIR ? 2 : 1); h++) {
            const int bl = (PAIR ? 2 * (r + i * kGmL) : r + i * kGmL) + h; // block within the chunk
            uint32_t lo[RW][4], hi[RW][4];
            float dw[RW];
#pragma unroll
            for (int q = 0; q < RW; q++) {
                // rows past n (the last group) contribute nothing and are not stored
                dw[q] = row0 + q < n ? half_bits_to_float(unit[q].d[h]) : 0.0f;
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    lo[q][e] = unit[q].qs[h][e] & 0x0f0f0f0fu;
                    hi[q][e] = (unit[q].qs[h][e] >> 4) & 0x0f0f0f0fu;
                }
            }
#pragma unroll
            for (int a = 0; a < M; a++) {
                const u32x4 xlo = s.qs[a][bl][0], xhi = s.qs[a][bl][1];
                const int c8 = s.c8[a][bl];
                const float dx = s.dx[a][bl];
#pragma unroll
                for (int q = 0; q < RW; q++) {
                    int sum = c8;
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        sum = sdot4(lo[q][e], xlo[e], sum);
                        sum = sdot4(hi[q][e], xhi[e], sum);
                    }
                    acc[q][a] += dw[q] * dx * (float)sum;
                }
            }
        }
    }
}

template <int M, int RW, int U, bool PAIR, bool F32>
__global__ __launch_bounds__(kGmThreads) void q4_0_gemv_m_kernel(const uint8_t *__restrict__ w, const void *xin,
                                                                  float *__restrict__ y, int64_t m, int64_t n, int nb)
{
    __shared__ GmLds<M, U, PAIR> s;
    constexpr int CB = GmLds<M, U, PAIR>::CB;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane / kGmL, r = lane % kGmL;
    const int nu = PAIR ? nb / 2 : nb;
    const int chunks = (nb + CB - 1) / CB;
    const int64_t row_bytes = (int64_t)nb * 18;
    // rows row0 .. row0 + RW - 1 (some may be >= n: loaded as row 0, masked)
    const int64_t row0 = (((int64_t)blockIdx.x * (kGmThreads / 64) + wave) * (64 / kGmL) + g) * RW;

    float acc[RW][M];
#pragma unroll
    for (int q = 0; q < RW; q++)
#pragma unroll
        for (int a = 0; a < M; a++)
            acc[q][a] = 0.0f;
    // Activation loads of a chunk go out before its weight loads: loads
    // retire in order, so the staging waits only for its own bytes.
    GmRaw<M, U, PAIR, F32> act;
    gm_act_load<M, U, PAIR, F32>(xin, m, nb, 0, act);
    GemvRaw<U> cur[RW], nxt[RW];
#pragma unroll
    for (int q = 0; q < RW; q++)
        gemv_load<kGmL, U, PAIR>(w, row0 + q, n, row_bytes, nu, 0, r, cur[q]);
    for (int c = 0; c < chunks; c++) {
        if (c > 0)
            __syncthreads(); // every wave is done with the previous chunk
        gm_act_store<M, U, PAIR, F32>(act, m, nb, c, s);
        __syncthreads();
        if (c + 1 < chunks) {
            gm_act_load<M, U, PAIR, F32>(xin, m, nb, c + 1, act);
#pragma unroll
            for (int q = 0; q < RW; q++)
                gemv_load<kGmL, U, PAIR>(w, row0 + q, n, row_bytes, nu, (c + 1) * U * kGmL, r, nxt[q]);
        }
        gm_compute<M, RW, U, PAIR>(cur, row0, n, row_bytes, nu, c * U * kGmL, r, s, acc);
#pragma unroll
        for (int q = 0; q < RW; q++)
            cur[q] = nxt[q];
    }
#pragma unroll
    for (int q = 0; q < RW; q++)
#pragma unroll
        for (int a = 0; a < M; a++) {
            float v = acc[q][a];
#pragma unroll
            for (int off = kGmL / 2; off > 0; off >>= 1)
                v += __shfl_xor(v, off);
            if (r == 0 && row0 + q < n && a < m)
                y[(int64_t)a * n + row0 + q] = v;
        }
}

template <int RW, int U, bool F32>
static hipError_t launch_gm_l(const uint8_t *w, const void *xin, float *y, int64_t m, int64_t n, int nb,
                              hipStream_t s)
{
    constexpr int R = 64 / kGmL * RW; // weight rows per wave
    const int64_t groups = (n + R - 1) / R;
    const int64_t grid = (groups + kGmThreads / 64 - 1) / (kGmThreads / 64);
    if (grid > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    const dim3 gd((unsigned)grid), bd(kGmThreads);
#define QLL_GM(MM)                                                                                                    \
    do {                                                                                                              \
        if (nb % 2 == 0)                                                                                              \
            hipLaunchKernelGGL((q4_0_gemv_m_kernel<MM, RW, U, true, F32>), gd, bd, 0, s, w, xin, y, m, n, nb);        \
        else                                                                                                          \
            hipLaunchKernelGGL((q4_0_gemv_m_kernel<MM, RW, U, false, F32>), gd, bd, 0, s, w, xin, y, m, n, nb);       \
    } while (0)
    if (m <= 1)
        QLL_GM(1);
    else if (m <= 2)
        QLL_GM(2);
    else if (m <= 4)
        QLL_GM(4);
    else
        QLL_GM(8);
#undef QLL_GM
    return hipGetLastError();
}

// 64-row workgroups (4 rows per lane group) once they number at least 512,
// or 128 with f32 activations, whose in-launch quantization each workgroup
// repeats (measured: at n = 14336 the f32 entry runs 1.3 to 2.6 times faster
// with 64-row workgroups, at n = 4096 1.4 to 1.6 times slower).
template <bool F32>
static hipError_t launch_gm(const uint8_t *w, const void *xin, float *y, int64_t m, int64_t n, int64_t k,
                            hipStream_t s)
{
    const int nb = (int)(k / 32);
    if (n >= (F32 ? 128 : 512) * 64)
        return launch_gm_l<4, 1, F32>(w, xin, y, m, n, nb, s);
    // two rows per lane once the LDS reads bound (m > 2) and the matrix is
    // tall enough to keep workgroups for them (4096 -> 14336 at m = 8: 17.6
    // against 26.0 us; m = 4: 12.4 against 14.5; at n = 4096 the grid gets
    // too small: 16.2 against 12.9 us)
    if (!F32 && m > 2 && n >= 8192)
        return launch_gm_l<2, 1, F32>(w, xin, y, m, n, nb, s);
    return launch_gm_l<1, 4, F32>(w, xin, y, m, n, nb, s);
}

hipError_t launch_q4_0_q8_0_gemv_m(const uint8_t *w, const uint8_t *xq, float *y, int64_t m, int64_t n, int64_t k,
                                   hipStream_t s)
{
    if (m > kMaxMMfma || (m == 1 && k <= kMaxKQ4Gemv)) {
        // groups of at most 32 activation rows (a last group of one row: the
        // GEMV); each group's outputs are its own rows of y
        if (m == 1)
            return launch_q4_0_q8_0_gemv(w, xq, y, n, k, s);
        for (int64_t a0 = 0; a0 < m; a0 += kMaxMMfma) {
            const int64_t mm = m - a0 < kMaxMMfma ? m - a0 : kMaxMMfma;
            const hipError_t e = launch_q4_0_q8_0_gemv_m(w, xq + a0 * (k / 32) * 34, y + a0 * n, mm, n, k, s);
            if (e != hipSuccess)
                return e;
        }
        return hipSuccess;
    }
    // the matrix-core kernel, except at m = 2 on tall matrices and m <= 4 on
    // very tall ones, where the weight stream bounds both and this kernel's
    // lighter staging wins (4096 -> 14336 at m = 2: 9.9 against 11.0 us;
    // 4096 -> 128256 at m = 2 / 4: 57 / 67.5 against 65 / 71.6 us)
    const bool gemv_style = (m == 2 && n >= 8192) || (m <= 4 && n >= 32768);
    if (m >= 2 && k >= kMinKMfma && k < kMaxKMfma && !gemv_style)
        return launch_q4_0_q8_0_small_m_mfma(w, xq, y, m, n, k, s);
    // rows of fewer than eight blocks (or very long rows at m <= 8): the
    // kernel above by groups of at most eight activation rows
    for (int64_t a0 = 0; a0 < m; a0 += kMaxMSmall) {
        const int64_t mm = m - a0 < kMaxMSmall ? m - a0 : kMaxMSmall;
        const hipError_t e = launch_gm<false>(w, xq + a0 * (k / 32) * 34, y + a0 * n, mm, n, k, s);
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

// The single launch wins only where the weights take one pass of the
// resident workgroups and the row is short: every workgroup then quantizes
// the row once, in the shadow of its first weight loads (4096 x 4096 at
// m = 1: 6.1 against 6.7 us for the two launches).  Elsewhere the repeated
// quantization costs more than a second launch (4096 -> 14336 at m = 1:
// 11.2 against 10.4 us; 14336 -> 4096: 18 against 11.7; every shape at
// m = 8, where each workgroup would quantize eight rows: 38 to 178 against
// 13 to 112 us), so given a workspace the rows are quantized once by the
// quantize kernel and the Q8_0 decode kernels run on them.
size_t q4_0_gemv_f32_workspace(int64_t m, int64_t n, int64_t k)
{
    if (m == 1 && k <= 4096 && n * k <= ((int64_t)1 << 24))
        return 0;
    return ((size_t)(m * (k / 32) * 34) + 255) & ~(size_t)255;
}

hipError_t launch_q4_0_q8_0_gemv_f32(const uint8_t *w, const float *x, float *y, int64_t m, int64_t n, int64_t k,
                                     uint8_t *ws, hipStream_t s)
{
    if (ws) {
        hipError_t e = launch_quantize_q8_0(x, ws, m * (k / 32), s);
        if (e != hipSuccess)
            return e;
        if (m == 1 && k <= kMaxKQ4Gemv)
            return launch_q4_0_q8_0_gemv(w, ws, y, n, k, s);
        return launch_q4_0_q8_0_gemv_m(w, ws, y, m, n, k, s);
    }
    // m = 1: the GEMV kernel, quantizing the row while it stages it (the
    // whole row fits in LDS up to kMaxKQ4Gemv; longer rows stage by chunks)
    if (m == 1 && k <= kMaxKQ4Gemv) {
        const int nb = (int)(k / 32);
        if (nb % 2 == 0)
            return launch_pair<true, true>(w, x, y, n, nb, s);
        return launch_pair<false, true>(w, x, y, n, nb, s);
    }
    return launch_gm<true>(w, x, y, m, n, k, s);
}

} // namespace qll
