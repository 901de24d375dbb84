// Internal header of libqll.so: device helpers shared by the kernels and the
// launcher declarations called by the C-ABI layer (abi.hip).  Kernels below
// the ABI are unchecked: the ABI validates shapes, pointers and alignment
// once, then launches (the kernel contract of Fucina course "Chapter 06 --
// Going fast on CPUs", 6.3).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qll {

// 16-byte vector of dwords that only promises 4-byte alignment: global
// dwordx4 loads need no more on gfx950, and the 18- and 34-byte block formats
// only give dword alignment for pairs of blocks.
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float half_bits_to_float(uint32_t bits)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits & 0xffffu));
}

// f32 -> binary16 bits, round to nearest even (v_cvt_f16_f32 in the default
// rounding mode).
__device__ __forceinline__ uint16_t float_to_half_bits(float f)
{
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// Low 32 bits of ({hi, lo} >> s).
__device__ __forceinline__ uint32_t funnel(uint32_t hi, uint32_t lo, uint32_t s)
{
    return __builtin_amdgcn_alignbit(hi, lo, s);
}

// Signed 4x8-bit dot product accumulated into c (v_dot4_i32_i8).
__device__ __forceinline__ int32_t sdot4(uint32_t a, uint32_t b, int32_t c)
{
    return __builtin_amdgcn_sdot4((int32_t)a, (int32_t)b, c, false);
}

__device__ __forceinline__ u32x4 load4_a4(const uint8_t *p)
{
    return *reinterpret_cast<const u32x4_a4 *>(p);
}

// Q8_0 code of x for the block scale d (IEEE f32 division, ties away from
// zero, clamped to +-127; d = 0 gives 0).
__device__ __forceinline__ int quant_code(float x, float d)
{
    if (d == 0.0f)
        return 0;
    float r = roundf(x / d);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int)r;
}

// Q8_0 block at byte offset o of `base` (o % 4 is 0 or 2) -> binary16 d bits
// and the 32 int8 codes as 8 dwords.  Reads only bytes of this block and, when
// o % 4 == 2, the two bytes before it (inside the same buffer, since o >= 34).
__device__ __forceinline__ void load_q8_0_block(const uint8_t *base, int64_t o, uint32_t &d, uint32_t q[8])
{
    if ((o & 3) == 0) {
        const uint32_t *p = reinterpret_cast<const uint32_t *>(base + o);
        uint32_t w[8];
#pragma unroll
        for (int i = 0; i < 8; i++)
            w[i] = p[i];
        uint32_t tail = *reinterpret_cast<const uint16_t *>(base + o + 32);
        d = w[0] & 0xffffu;
#pragma unroll
        for (int i = 0; i < 7; i++)
            q[i] = funnel(w[i + 1], w[i], 16);
        q[7] = funnel(tail, w[7], 16);
    } else {
        const uint32_t *p = reinterpret_cast<const uint32_t *>(base + o - 2);
        uint32_t w0 = p[0];
        d = w0 >> 16;
#pragma unroll
        for (int i = 0; i < 8; i++)
            q[i] = p[i + 1];
    }
}

// ------------------------------------------------------------ launchers
// Each returns a hipError_t of the launch; arguments are already validated.

hipError_t launch_pack_q4_0(const uint8_t *codes, const uint16_t *d_bits, uint8_t *w, int64_t n, int64_t k,
                            hipStream_t s);
hipError_t launch_pack_ternary(const uint8_t *codes, uint32_t *w, int64_t n, int64_t k, hipStream_t s);
hipError_t launch_quantize_q8_0(const float *x, uint8_t *xq, int64_t nblocks, hipStream_t s);
hipError_t launch_quantize_i8_rows(const float *x, int8_t *xq, float *act_scale, int32_t *act_sum, int64_t m,
                                   int64_t k, hipStream_t s);
hipError_t launch_q4_0_q8_0_gemv(const uint8_t *w, const uint8_t *xq, float *y, int64_t n, int64_t k,
                                 hipStream_t s);
// y[i] = sum of parts[s * count + i] over the splits s, in split order (the
// split-k GEMMs' second launch).
hipError_t launch_sum_splits(const float *parts, float *y, int64_t count, int splits, hipStream_t s);
hipError_t launch_q4_0_q8_0_gemm(const uint8_t *w, const uint8_t *xq, float *y, int64_t m, int64_t n, int64_t k,
                                 void *ws, hipStream_t s);
// Small-m decode: Q8_0 activations at 1 <= m <= 64 (groups of at most 32
// rows above 32; m <= kMaxMSmall when k >= kMaxKMfma), or, in the
// quantize-fused entry, f32 activations quantized to Q8_0 inside the launch
// (1 <= m <= kMaxMSmall).
constexpr int64_t kMaxMSmall = 8;
hipError_t launch_q4_0_q8_0_gemv_m(const uint8_t *w, const uint8_t *xq, float *y, int64_t m, int64_t n, int64_t k,
                                   hipStream_t s);
// Small m on the int8 matrix core (1 <= m <= kMaxMMfma, kMinKMfma <= k <
// kMaxKMfma: a stage is eight blocks, and 32 activation rows are addressed
// with 32-bit offsets): Q8_0 activations, no workspace.
constexpr int64_t kMaxMMfma = 32;
constexpr int64_t kMinKMfma = 256, kMaxKMfma = (int64_t)1 << 24;

// Whether the Q4_0 x Q8_0 GEMM entry runs the small-m kernels (no
// workspace) rather than the 128-row GEMM: m <= 8 at any k; otherwise
// k < kMaxKMfma and m <= 64, above 32 as groups of at most 32 activation
// rows (each group re-reads the weights, which beats the GEMM's padding of m
// to 128 rows up to there: at m = 64, 4096 -> 14336 33 against 44 us,
// 4096 -> 128256 206 against 234 us; at m = 96 the GEMM wins).
inline bool q4_small_m_path(int64_t m, int64_t n, int64_t k)
{
    (void)n;
    return m <= kMaxMSmall || (k < kMaxKMfma && m <= 64);
}
hipError_t launch_q4_0_q8_0_small_m_mfma(const uint8_t *w, const uint8_t *xq, float *y, int64_t m, int64_t n,
                                         int64_t k, hipStream_t s);
// With ws (at least q4_0_gemv_f32_workspace bytes, nonzero), the rows are
// quantized into ws by the quantize kernel and the Q8_0 decode kernel runs
// on them; with ws == nullptr, one launch quantizes inside each workgroup.
hipError_t launch_q4_0_q8_0_gemv_f32(const uint8_t *w, const float *x, float *y, int64_t m, int64_t n, int64_t k,
                                     uint8_t *ws, hipStream_t s);
size_t q4_0_gemv_f32_workspace(int64_t m, int64_t n, int64_t k);
size_t q4_0_q8_0_gemm_workspace(int64_t m, int64_t n, int64_t k);
// Decode GEMV with Q8_0 weights.
hipError_t launch_q8_0_q8_0_gemv(const uint8_t *w, const uint8_t *xq, float *y, int64_t n, int64_t k, hipStream_t s);
// Transposed-B (W stored [n][k]) f32 GEMV and GEMM with f32, bf16 or f16
// weights (the values of the ABI's QLL_DTYPE_*).
enum { QLL_W_F32 = 0, QLL_W_BF16 = 1, QLL_W_F16 = 2 };
hipError_t launch_gemv_nt(const float *x, const void *w, int wfmt, float *y, int64_t n, int64_t k, hipStream_t s);
hipError_t launch_sgemm_nt(const float *a, const void *w, int wfmt, float *c, int64_t m, int64_t n, int64_t k,
                           hipStream_t s);
bool gemm_nt_bf16_core_shape(int64_t m, int64_t k);
size_t gemm_nt_workspace(int wfmt, int64_t m, int64_t n, int64_t k);
hipError_t launch_gemm_nt_bf16_mfma(const float *x, const void *w, int wfmt, float *y, int64_t m, int64_t n,
                                    int64_t k, void *ws, hipStream_t s, bool b_kn = false);
// Load-time repack of Q4_0 weights and the GEMM on them (6-bit matrix-core path).
size_t q4_0_repacked_bytes(int64_t n, int64_t k);
// Decode-packed Q4_0 weights (groups of eight blocks: nibbles, then scales).
size_t q4_0_packed_bytes(int64_t n, int64_t k);
hipError_t launch_q4_0_pack_decode(const uint8_t *w, uint8_t *wp, int64_t n, int64_t k, hipStream_t s);
hipError_t launch_q4_0_packed_gemv(const uint8_t *w, const uint8_t *xq, float *y, int64_t n, int64_t k,
                                   hipStream_t s);
hipError_t launch_q4_0_repack(const uint8_t *w, uint8_t *wp, int64_t n, int64_t k, hipStream_t s);
size_t q4_0_packed_gemm_workspace(int64_t m, int64_t n, int64_t k);
hipError_t launch_q4_0_packed_gemm(const uint8_t *wp, const uint8_t *xq, float *y, int64_t m, int64_t n, int64_t k,
                                   void *ws, hipStream_t s);
size_t q8_0_repacked_bytes(int64_t n, int64_t k);
hipError_t launch_q8_0_repack(const uint8_t *w, uint8_t *wp, int64_t n, int64_t k, hipStream_t s);
hipError_t launch_q8_0_packed_gemm(const uint8_t *wp, const uint8_t *xq, float *y, int64_t m, int64_t n, int64_t k,
                                   void *ws, hipStream_t s);
hipError_t launch_sgemv(const float *x, const float *b, float *c, int64_t n, int64_t k, float *ws, hipStream_t s);
size_t sgemv_workspace(int64_t n, int64_t k);
hipError_t launch_sgemm(const float *a, const float *b, float *c, int64_t m, int64_t n, int64_t k, hipStream_t s);
hipError_t launch_ternary_gemv(const uint32_t *w, float w_scale, const int8_t *xq, const float *act_scale,
                               const int32_t *act_sum, float *y, int64_t n, int64_t k, hipStream_t s);
hipError_t launch_ternary_gemm(const uint32_t *w, float w_scale, const int8_t *xq, const float *act_scale,
                               const int32_t *act_sum, float *y, int64_t m, int64_t n, int64_t k, hipStream_t s);

// Largest k the LDS-staged decode kernels accept (the activation of one row
// is kept whole in LDS).
constexpr int64_t kMaxKQ4Gemv = 49152;
constexpr int64_t kMaxKTernaryGemv = 65536;

} // namespace qll
