// Format encoders and activation quantizers.
//
//  * Q4_0 packing: 32 four-bit codes and an fp16 scale per block; element t of
//    a block is the low nibble of byte t (t < 16) or the high nibble of byte
//    t - 16 (llama.cpp visual guide lesson 31 "CPU backend", "How the
//    quantized dot product works": the unpack masks the low 4 bits, then
//    shifts for the high 4).
//  * Ternary packing: 16 two-bit codes (weight + 1) per uint32, code s at
//    bits 2s (Loom "Plan 9 SIMD Forward", "BitNet ternary MAD kernel").
//  * Q8_0 activation quantization per 32-block (Fucina reference "Backends",
//    9.7: the f32 activation rows are quantized per call).
//  * Per-row int8 activation quantization with scale 127 / max|x| (Loom, the
//    same section).
// The quantizers are bit-exact with the oracle: IEEE f32 division and
// multiplication, round half away from zero, binary16 round to nearest even.
#include "common.h"

namespace qll {

// One thread per Q4_0 block: 32 code bytes + one scale -> 18 bytes.
__global__ __launch_bounds__(256) void pack_q4_0_kernel(const uint8_t *__restrict__ codes,
                                                        const uint16_t *__restrict__ d_bits,
                                                        uint8_t *__restrict__ w, int64_t nblocks)
{
    int64_t gb = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (gb >= nblocks)
        return;
    // codes of block gb are bytes [32*gb, 32*gb + 32): row-major [n][k] with
    // k % 32 == 0 makes the blocks contiguous in this flat order.
    const u32x4 *c = reinterpret_cast<const u32x4 *>(codes + gb * 32);
    u32x4 lo = c[0], hi = c[1];
    uint16_t *out = reinterpret_cast<uint16_t *>(w + gb * 18); // 2-byte aligned
    out[0] = d_bits[gb];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        uint32_t v = (lo[i] & 0x0f0f0f0fu) | ((hi[i] & 0x0f0f0f0fu) << 4);
        out[1 + 2 * i] = (uint16_t)(v & 0xffffu);
        out[2 + 2 * i] = (uint16_t)(v >> 16);
    }
}

// One thread per ternary word: 16 code bytes -> one uint32.
__global__ __launch_bounds__(256) void pack_ternary_kernel(const uint8_t *__restrict__ codes,
                                                           uint32_t *__restrict__ w, int64_t nwords)
{
    int64_t gw = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (gw >= nwords)
        return;
    u32x4 c = *reinterpret_cast<const u32x4 *>(codes + gw * 16);
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int b = 0; b < 4; b++)
            word |= ((c[i] >> (8 * b)) & 3u) << (2 * (4 * i + b));
    w[gw] = word;
}

hipError_t launch_pack_q4_0(const uint8_t *codes, const uint16_t *d_bits, uint8_t *w, int64_t n, int64_t k,
                            hipStream_t s)
{
    int64_t nblocks = n * (k / 32);
    int64_t grid = (nblocks + 255) / 256;
    hipLaunchKernelGGL(pack_q4_0_kernel, dim3((unsigned)grid), dim3(256), 0, s, codes, d_bits, w, nblocks);
    return hipGetLastError();
}

hipError_t launch_pack_ternary(const uint8_t *codes, uint32_t *w, int64_t n, int64_t k, hipStream_t s)
{
    int64_t nwords = n * (k / 16);
    int64_t grid = (nwords + 255) / 256;
    hipLaunchKernelGGL(pack_ternary_kernel, dim3((unsigned)grid), dim3(256), 0, s, codes, w, nwords);
    return hipGetLastError();
}

// ------------------------------------------------------------------ Q8_0

// Flat over all m*k/32 blocks (rows of x are whole blocks).  Eight lanes own a
// block, four floats each; a workgroup of TH lanes owns TH / 8 blocks,
// assembles their bytes in LDS and writes them with dword stores.  Up to
// 2048 blocks (a decode row) one-wave workgroups spread the row over more
// CUs (k = 4096: 2.13 -> 2.00 us); larger inputs use 256 lanes.
template <int TH>
__global__ __launch_bounds__(TH) void quantize_q8_0_kernel(const float *__restrict__ x, uint8_t *__restrict__ xq,
                                                            int64_t nblocks)
{
    constexpr int BPW = TH / 8;
    __shared__ uint32_t s_out[BPW * 34 / 4];
    uint8_t *sb = reinterpret_cast<uint8_t *>(s_out);
    const int t = threadIdx.x, bl = t >> 3, sub = t & 7;
    const int64_t blk0 = (int64_t)blockIdx.x * BPW;
    const int64_t gb = blk0 + bl;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (gb < nblocks)
        v = reinterpret_cast<const float4 *>(x)[gb * 8 + sub];
    float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    a = fmaxf(a, __shfl_xor(a, 1));
    a = fmaxf(a, __shfl_xor(a, 2));
    a = fmaxf(a, __shfl_xor(a, 4));
    const float d = a / 127.0f;
    const int q0 = quant_code(v.x, d), q1 = quant_code(v.y, d), q2 = quant_code(v.z, d), q3 = quant_code(v.w, d);
    uint16_t *dst16 = reinterpret_cast<uint16_t *>(sb + bl * 34 + 2 + 4 * sub);
    dst16[0] = (uint16_t)((q0 & 0xff) | ((q1 & 0xff) << 8));
    dst16[1] = (uint16_t)((q2 & 0xff) | ((q3 & 0xff) << 8));
    if (sub == 0)
        *reinterpret_cast<uint16_t *>(sb + bl * 34) = float_to_half_bits(d);
    __syncthreads();
    int64_t left = nblocks - blk0;
    const int cnt = left < BPW ? (int)left : BPW;
    const int bytes = cnt * 34;
    uint8_t *dst = xq + blk0 * 34; // 34 BPW * blockIdx.x: dword aligned (BPW even)
    for (int i = t; i < bytes / 4; i += TH)
        reinterpret_cast<uint32_t *>(dst)[i] = s_out[i];
    if ((bytes & 3) != 0 && t == 0)
        *reinterpret_cast<uint16_t *>(dst + bytes - 2) = *reinterpret_cast<const uint16_t *>(sb + bytes - 2);
}

hipError_t launch_quantize_q8_0(const float *x, uint8_t *xq, int64_t nblocks, hipStream_t s)
{
    if (nblocks <= 2048) {
        hipLaunchKernelGGL(quantize_q8_0_kernel<64>, dim3((unsigned)((nblocks + 7) / 8)), dim3(64), 0, s, x, xq, nblocks);
        return hipGetLastError();
    }
    int64_t grid = (nblocks + 31) / 32;
    hipLaunchKernelGGL(quantize_q8_0_kernel<256>, dim3((unsigned)grid), dim3(256), 0, s, x, xq, nblocks);
    return hipGetLastError();
}

// ------------------------------------------------------------------ int8 rows

__device__ __forceinline__ int quant_i8(float x, float s)
{
    if (s == 0.0f)
        return 0;
    float r = roundf(x * s); // f32 product, ties away from zero
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int)r;
}

template <typename T, typename Op>
__device__ __forceinline__ T block_reduce_256(T v, Op op, T *scratch)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        v = op(v, __shfl_xor(v, off));
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0)
        scratch[wave] = v;
    __syncthreads();
    T r = op(op(scratch[0], scratch[1]), op(scratch[2], scratch[3]));
    __syncthreads();
    return r;
}

// One workgroup per row.  VEC = 4 when k % 4 == 0 (float4 loads, 4-byte
// stores), else 1.  Rows of at most 4096 elements (VEC = 4) stay in
// registers between the amax pass and the quantization pass, so the row is
// read from memory once (2560 elements: 3.12 -> 2.79 us).
template <int VEC>
__global__ __launch_bounds__(256) void quantize_i8_rows_kernel(const float *__restrict__ x, int8_t *__restrict__ xq,
                                                               float *__restrict__ act_scale,
                                                               int32_t *__restrict__ act_sum, int64_t k)
{
    __shared__ float s_f[4];
    __shared__ int s_i[4];
    const int64_t row = blockIdx.x;
    const float *xr = x + row * k;
    int8_t *qr = xq + row * k;
    const int64_t nv = k / VEC;
    float a = 0.0f;
    constexpr int HR = 4; // float4 pieces per thread kept in registers between the two passes
    float4 held[HR];
    const bool hold = VEC == 4 && nv <= 256 * HR; // uniform
    if (hold) {
#pragma unroll
        for (int j = 0; j < HR; j++) {
            const int64_t i = threadIdx.x + 256 * j;
            held[j] = i < nv ? reinterpret_cast<const float4 *>(xr)[i] : make_float4(0.f, 0.f, 0.f, 0.f);
            a = fmaxf(a, fmaxf(fmaxf(fabsf(held[j].x), fabsf(held[j].y)), fmaxf(fabsf(held[j].z), fabsf(held[j].w))));
        }
    } else {
    for (int64_t i = threadIdx.x; i < nv; i += 256) {
        if (VEC == 4) {
            float4 v = reinterpret_cast<const float4 *>(xr)[i];
            a = fmaxf(a, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
        } else {
            a = fmaxf(a, fabsf(xr[i]));
        }
    }
    }
    const float amax = block_reduce_256(a, [](float p, float q) { return fmaxf(p, q); }, s_f);
    float sc = (amax == 0.0f) ? 0.0f : 127.0f / amax; // IEEE division
    if (!__builtin_isfinite(sc))
        sc = 0.0f;
    int sum = 0;
    if (hold) {
#pragma unroll
        for (int j = 0; j < HR; j++) {
            const int64_t i = threadIdx.x + 256 * j;
            if (i < nv) {
                const float4 v = held[j];
                int q0 = quant_i8(v.x, sc), q1 = quant_i8(v.y, sc), q2 = quant_i8(v.z, sc), q3 = quant_i8(v.w, sc);
                sum += q0 + q1 + q2 + q3;
                reinterpret_cast<uint32_t *>(qr)[i] =
                    (uint32_t)(q0 & 0xff) | ((uint32_t)(q1 & 0xff) << 8) | ((uint32_t)(q2 & 0xff) << 16) |
                    ((uint32_t)(q3 & 0xff) << 24);
            }
        }
    } else
    for (int64_t i = threadIdx.x; i < nv; i += 256) {
        if (VEC == 4) {
            float4 v = reinterpret_cast<const float4 *>(xr)[i];
            int q0 = quant_i8(v.x, sc), q1 = quant_i8(v.y, sc), q2 = quant_i8(v.z, sc), q3 = quant_i8(v.w, sc);
            sum += q0 + q1 + q2 + q3;
            reinterpret_cast<uint32_t *>(qr)[i] =
                (uint32_t)(q0 & 0xff) | ((uint32_t)(q1 & 0xff) << 8) | ((uint32_t)(q2 & 0xff) << 16) |
                ((uint32_t)(q3 & 0xff) << 24);
        } else {
            int q = quant_i8(xr[i], sc);
            sum += q;
            qr[i] = (int8_t)q;
        }
    }
    sum = block_reduce_256(sum, [](int p, int q) { return p + q; }, s_i);
    if (threadIdx.x == 0) {
        act_scale[row] = sc;
        act_sum[row] = sum;
    }
}

hipError_t launch_quantize_i8_rows(const float *x, int8_t *xq, float *act_scale, int32_t *act_sum, int64_t m,
                                   int64_t k, hipStream_t s)
{
    if (k % 4 == 0)
        hipLaunchKernelGGL(quantize_i8_rows_kernel<4>, dim3((unsigned)m), dim3(256), 0, s, x, xq, act_scale,
                           act_sum, k);
    else
        hipLaunchKernelGGL(quantize_i8_rows_kernel<1>, dim3((unsigned)m), dim3(256), 0, s, x, xq, act_scale,
                           act_sum, k);
    return hipGetLastError();
}

} // namespace qll
