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
__device__ __forceinline__ ActLds stage_q8_row(const uint8_t *__restrict__ xq, int nb, void *smem)
{
    u32x4 *s_qs = reinterpret_cast<u32x4 *>(smem);
    float *s_dx = reinterpret_cast<float *>(s_qs + 2 * nb);
    int *s_c8 = reinterpret_cast<int *>(s_dx + nb);
    for (int b = threadIdx.x; b < nb; b += blockDim.x) {
        uint32_t d, q[8];
        load_q8_0_block(xq, (int64_t)b * 34, d, q);
        int sx = 0;
#pragma unroll
        for (int i = 0; i < 8; i++)
            sx = sdot4(q[i], 0x01010101u, sx);
        s_qs[2 * b] = u32x4{q[0], q[1], q[2], q[3]};
        s_qs[2 * b + 1] = u32x4{q[4], q[5], q[6], q[7]};
        s_dx[b] = half_bits_to_float(d);
        s_c8[b] = -8 * sx;
    }
    __syncthreads();
    return ActLds{s_qs, s_dx, s_c8};
}

constexpr int kGemvThreads = 256;
constexpr int kGemvUnroll = 4;

template <int L, bool PAIR>
__global__ __launch_bounds__(kGemvThreads) void q4_0_q8_0_gemv_kernel(const uint8_t *__restrict__ w,
                                                                      const uint8_t *__restrict__ xq,
                                                                      float *__restrict__ y, int64_t n, int nb)
{
    extern __shared__ u32x4 smem[];
    const ActLds act = stage_q8_row(xq, nb, smem);

    constexpr int R = 64 / L; // rows per wave
    constexpr int WAVES = kGemvThreads / 64;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane / L, r = lane % L;
    const int nu = PAIR ? nb / 2 : nb;
    const int64_t row_bytes = (int64_t)nb * 18;
    const int64_t stride = (int64_t)gridDim.x * WAVES * R;

    for (int64_t row0 = ((int64_t)blockIdx.x * WAVES + wave) * R; row0 < n; row0 += stride) {
        const int64_t row = row0 + g;
        float acc = 0.0f;
        if (row < n) {
            const uint8_t *wr = w + row * row_bytes;
            for (int u0 = r; u0 < nu; u0 += kGemvUnroll * L) {
                Q4Unit unit[kGemvUnroll];
#pragma unroll
                for (int i = 0; i < kGemvUnroll; i++) {
                    const int u = u0 + i * L;
                    if (u < nu) {
                        if (PAIR) {
                            uint32_t raw[9];
                            load_q4_pair(wr + (int64_t)u * 36, raw);
                            decode_q4_pair(raw, unit[i]);
                        } else {
                            uint32_t raw[5];
                            const int64_t o = row * row_bytes + (int64_t)u * 18;
                            load_q4_single(w, o, raw);
                            decode_q4_single(raw, (o & 3) != 0, unit[i]);
                        }
                    }
                }
#pragma unroll
                for (int i = 0; i < kGemvUnroll; i++) {
                    const int u = u0 + i * L;
                    if (u < nu) {
                        if (PAIR) {
                            acc += q4_block_dot(unit[i].d[0], unit[i].qs[0], act, 2 * u);
                            acc += q4_block_dot(unit[i].d[1], unit[i].qs[1], act, 2 * u + 1);
                        } else {
                            acc += q4_block_dot(unit[i].d[0], unit[i].qs[0], act, u);
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int off = L / 2; off > 0; off >>= 1)
            acc += __shfl_xor(acc, off);
        if (row < n && r == 0)
            y[row] = acc;
    }
}

size_t q4_gemv_lds_bytes(int nb) { return (size_t)nb * 40; }

template <int L, bool PAIR>
static hipError_t launch_l(const uint8_t *w, const uint8_t *xq, float *y, int64_t n, int nb, hipStream_t s)
{
    constexpr int R = 64 / L;
    const int64_t waves = (n + R - 1) / R;
    int64_t grid = (waves + kGemvThreads / 64 - 1) / (kGemvThreads / 64);
    if (grid > 8192)
        grid = 8192;
    hipLaunchKernelGGL((q4_0_q8_0_gemv_kernel<L, PAIR>), dim3((unsigned)grid), dim3(kGemvThreads),
                       q4_gemv_lds_bytes(nb), s, w, xq, y, n, nb);
    return hipGetLastError();
}

template <bool PAIR>
static hipError_t launch_pair(const uint8_t *w, const uint8_t *xq, float *y, int64_t n, int nb, hipStream_t s)
{
    const int nu = PAIR ? nb / 2 : nb;
    // about four units per lane per row; 8..64 lanes per row
    if (nu >= 256)
        return launch_l<64, PAIR>(w, xq, y, n, nb, s);
    if (nu >= 128)
        return launch_l<32, PAIR>(w, xq, y, n, nb, s);
    if (nu >= 64)
        return launch_l<16, PAIR>(w, xq, y, n, nb, s);
    return launch_l<8, PAIR>(w, xq, y, n, nb, s);
}

hipError_t launch_q4_0_q8_0_gemv(const uint8_t *w, const uint8_t *xq, float *y, int64_t n, int64_t k,
                                 hipStream_t s)
{
    const int nb = (int)(k / 32);
    if (nb % 2 == 0)
        return launch_pair<true>(w, xq, y, n, nb, s);
    return launch_pair<false>(w, xq, y, n, nb, s);
}

} // namespace qll
