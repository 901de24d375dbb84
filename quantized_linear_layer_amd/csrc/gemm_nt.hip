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
};

template <int WFMT, int L, int U>
__device__ __forceinline__ void nt_load(const uint8_t *wr, int64_t nv, int64_t c0, int r, NtRaw<WFMT, U> &raw)
{
#pragma unroll
    for (int i = 0; i < U; i++) {
        int64_t v = c0 + r + (int64_t)i * L;
        v = v < nv ? v : 0; // past the row: reload vector 0 (masked in nt_dot)
        raw.w[i] = *reinterpret_cast<const u32x4 *>(wr + v * 16);
    }
}

template <int WFMT, int L, int U>
__device__ __forceinline__ float nt_dot(const float *__restrict__ x, int64_t nv, int64_t c0, int r,
                                        const NtRaw<WFMT, U> &raw)
{
    constexpr int V = NtW<WFMT>::V;
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < U; i++) {
        const int64_t v = c0 + r + (int64_t)i * L;
        if (v < nv) {
            const float *xv = x + v * V;
#pragma unroll
            for (int q = 0; q < V / 4; q++) {
                const float4 xs = *reinterpret_cast<const float4 *>(xv + 4 * q);
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
        nt_load<WFMT, L, U>(wr, nv, 0, r, cur);
        for (int64_t c0 = 0; c0 < nv; c0 += step) {
            if (c0 + step < nv)
                nt_load<WFMT, L, U>(wr, nv, c0 + step, r, nxt);
            acc += nt_dot<WFMT, L, U>(x, nv, c0, r, cur);
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
