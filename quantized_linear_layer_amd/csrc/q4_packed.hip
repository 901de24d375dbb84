// Q4_0 x Q8_0 prefill GEMM on load-time repacked weights, Y[m][n] = X . W^T,
// with the per-block arithmetic of llama.cpp visual guide lesson 31 "CPU
// backend" ("How the quantized dot product works") for every (i, j):
//     P[i,j,b] = sum_t (q_w[j,b,t] - 8) * q_x[i,b,t]     exact integer
//     Y[i,j]  += f32(d_w[j,b]) * f32(d_x[i,b]) * P[i,j,b]
// The weights are rewritten once, at load time, into the operand form of the
// matrix core (the packed right-hand side of Fucina reference "Backends",
// 9.7: a layout chosen for the kernel, built once and reused by every call).
//
// Matrix-core route: gfx950's block-scaled MFMA on 6-bit floats,
// v_mfma_scale_f32_32x32x64_f8f6f4 with both operands in e3m2 (sign, 3-bit
// exponent with bias 3, 2-bit mantissa), whose values include every integer
// in [-8, 8].  A weight w = q_w - 8 is one such value.  An activation code
// q_x in [-127, 127] is split as q_x = 16 h + l with l in [-8, 7] and h in
// [-8, 8], both exact.  One MFMA with K = 64 then takes a whole 32-element
// block: K 0..31 carry h against w with the E8M0 block scale 2^4, K 32..63
// carry l against the same w with scale 1, so
//     D = sum_t 16 h_t w_t + sum_t l_t w_t = P
// with every product and partial sum an integer far below 2^24: P is the
// exact block sum.  This MFMA issues at the rate of the f16 32x32x16 one but
// covers four times its K, so a block sum costs half of what two f16 K = 16
// steps do, and with unbiased operands no bias term is needed.  The scale
// tile S = 2 d_x d_w (exact) comes from v_mfma_f32_32x32x8_f16 as in the
// direct-layout GEMM, and the vector ALU does acc += S * P.
//
// Packed weight layout, for 128-row tiles t (rows n padded with zeros) and
// blocks b, chunk c = t * nb + b:
//   codes: 3072 bytes at 3072 c: plane 0 = code dwords 0..3 of row r at
//          16 r, plane 1 = code dwords 4..5 of row r at 2048 + 8 r; the 32
//          codes of a row are element t at bits 6 t of its six dwords, in the
//          block's element order (t < 16: low nibble of qs[t], else the high
//          nibble of qs[t - 16]);
//   d_w:   binary16 bits of row r at byte 2 (128 c + r) after the codes.
// The prepared activations (per call, in the workspace) use the same tiling
// over 128-row tiles of X: 6144 bytes per chunk (h codes as planes 0 and 1,
// then l codes as planes 0 and 1) and 128 binary16 d_x per chunk.
#include "common.h"

namespace qll {

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
#define QLL_LDS __attribute__((address_space(3)))

constexpr int PBM = 128, PBN = 128, PKB = 2, PNBUF = 3;
constexpr int kPThreads = 256;
constexpr int kPWChunk = 3072; // codes of 128 weight rows x one block
constexpr int kPXChunk = 6144; // h and l codes of 128 activation rows x one block
constexpr int kPSChunk = 256;  // binary16 scales of 128 rows x one block
constexpr uint32_t kE8M0One = 127, kE8M0Sixteen = 131;

// e3m2 code of an integer v in [-8, 8]: magnitudes 0..8 -> 0, 1.0 x 2^0,
// 1.0 x 2^1, 1.5 x 2^1, 1.0 x 2^2, 1.25 x 2^2, 1.5 x 2^2, 1.75 x 2^2,
// 1.0 x 2^3; the sign is bit 5.
__device__ __forceinline__ uint32_t e3m2_code(int v)
{
    const uint32_t a = (uint32_t)(v < 0 ? -v : v);
    const uint32_t mag = a >= 8 ? 24u : (uint32_t)((0x1716151412100C00ull >> (8 * a)) & 0xffu);
    return mag | (v < 0 ? 32u : 0u);
}

// 16 six-bit codes -> three dwords, code e at bits 6 e.
__device__ __forceinline__ void pack16_6bit(const uint32_t c[16], uint32_t out[3])
{
    uint64_t lo = 0;
    uint32_t hi = 0;
#pragma unroll
    for (int e = 0; e < 16; e++) {
        const int bit = 6 * e;
        if (bit + 6 <= 64) {
            lo |= (uint64_t)c[e] << bit;
        } else if (bit >= 64) {
            hi |= c[e] << (bit - 64);
        } else {
            lo |= (uint64_t)c[e] << bit;
            hi |= c[e] >> (64 - bit);
        }
    }
    out[0] = (uint32_t)lo;
    out[1] = (uint32_t)(lo >> 32);
    out[2] = hi;
}

// Writes one row's 32 codes (element order) as the two planes of a chunk.
__device__ __forceinline__ void store_planes(uint8_t *chunk, int r, const uint32_t c[32])
{
    uint32_t d[6];
    pack16_6bit(c, d);
    pack16_6bit(c + 16, d + 3);
    *reinterpret_cast<u32x4 *>(chunk + 16 * r) = u32x4{d[0], d[1], d[2], d[3]};
    *reinterpret_cast<u32x2 *>(chunk + 2048 + 8 * r) = u32x2{d[4], d[5]};
}

// ------------------------------------------------------------------ repack

// One thread per (tile row r, chunk c), r fastest so the plane stores of a
// wave are contiguous.  Rows at or past n get zero codes and d_w = 0.
__global__ __launch_bounds__(256) void q4p_repack_kernel(const uint8_t *__restrict__ w, uint8_t *__restrict__ codes,
                                                         uint16_t *__restrict__ dws, int64_t n, int nb, int64_t total)
{
    const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (g >= total)
        return;
    const int r = (int)(g & 127);
    const int64_t c = g >> 7;
    const int64_t t = c / nb;
    const int b = (int)(c % nb);
    const int64_t row = t * PBN + r;
    uint32_t code[32];
    uint16_t d = 0;
    if (row < n) {
        const uint8_t *blk = w + (row * nb + b) * 18;
        d = (uint16_t)(blk[0] | (blk[1] << 8));
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const int byte = blk[2 + i];
            code[i] = e3m2_code((byte & 15) - 8);
            code[16 + i] = e3m2_code((byte >> 4) - 8);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 32; i++)
            code[i] = 0u;
    }
    store_planes(codes + c * kPWChunk, r, code);
    dws[c * PBN + r] = d;
}

size_t q4_0_repacked_bytes(int64_t n, int64_t k)
{
    const int64_t nt = (n + PBN - 1) / PBN;
    return (size_t)nt * (size_t)(k / 32) * (kPWChunk + kPSChunk);
}

hipError_t launch_q4_0_repack(const uint8_t *w, uint8_t *wp, int64_t n, int64_t k, hipStream_t s)
{
    const int nb = (int)(k / 32);
    const int64_t nt = (n + PBN - 1) / PBN;
    const int64_t total = nt * nb * PBN;
    uint16_t *dws = reinterpret_cast<uint16_t *>(wp + (size_t)nt * nb * kPWChunk);
    const int64_t grid = (total + 255) / 256;
    if (grid > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(q4p_repack_kernel, dim3((unsigned)grid), dim3(256), 0, s, w, wp, dws, n, nb, total);
    return hipGetLastError();
}

// ------------------------------------------------------------------ activations

struct Q4pPrep {
    uint8_t *x;   // [mp / 128][nbp] chunks of kPXChunk bytes
    uint16_t *dx; // [mp / 128][nbp][128]
    int64_t mp, nbp;
};

// One thread per (row r of a 128-row tile, chunk (tile, block)), r fastest.
// The Q8_0 block (34 bytes) is read whole; rows >= m and blocks >= nb are
// written as zeros (zero codes, d_x = 0).
__global__ __launch_bounds__(256) void q4p_prep_kernel(const uint8_t *__restrict__ xq, Q4pPrep p, int64_t m, int nb,
                                                       int64_t total)
{
    const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (g >= total)
        return;
    const int r = (int)(g & 127);
    const int64_t c = g >> 7;
    const int64_t mt = c / p.nbp;
    const int64_t b = c % p.nbp;
    const int64_t row = mt * PBM + r;
    uint32_t hc[32], lc[32];
    uint16_t d = 0;
    if (row < m && b < nb) {
        const uint8_t *blk = xq + (row * nb + b) * 34;
        d = (uint16_t)(blk[0] | (blk[1] << 8));
#pragma unroll
        for (int e = 0; e < 32; e++) {
            const int q = (int)(int8_t)blk[2 + e];
            const int l = ((q + 8) & 15) - 8; // in [-8, 7]
            const int h = (q - l) >> 4;       // exact: q - l is a multiple of 16
            hc[e] = e3m2_code(h);
            lc[e] = e3m2_code(l);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 32; e++) {
            hc[e] = 0u;
            lc[e] = 0u;
        }
    }
    uint8_t *chunk = p.x + c * kPXChunk;
    store_planes(chunk, r, hc);
    store_planes(chunk + 3072, r, lc);
    p.dx[c * PBM + r] = d;
}

// ------------------------------------------------------------------ GEMM

// Weight formats of the packed GEMM: Q4_0 (one six-dword code group per row
// and block: w = q - 8) or Q8_0 (two: w = 16 h + l, the split the
// activations get).
template <bool Q8W>
struct PFmt {
    static constexpr int kWChunk = Q8W ? 2 * kPWChunk : kPWChunk; // weight code bytes per chunk
    static constexpr int kDma = Q8W ? 7 : 5;                      // global -> LDS loads per wave and stage
};

template <bool Q8W>
struct Q4pLds {
    uint8_t xs[PKB][kPXChunk]; // h planes then l planes of each block
    uint8_t wq[PKB][PFmt<Q8W>::kWChunk];
    uint16_t dx[PKB][PBM];
    uint16_t dw[PKB][PBN];
};

// One wave-wide global -> LDS load of 16 bytes per lane: lane l reads
// base + off and the wave writes LDS at lds + 16 l.  Inline assembly keeps
// these loads out of the compiler's wait bookkeeping.
__device__ __forceinline__ void q4p_dma16(const void *base, uint32_t off, const QLL_LDS void *lds)
{
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base),
                 "s"((uint32_t)(uintptr_t)lds)
                 : "memory", "m0");
}

// Row-tile and column-tile bases of the stage loads, set once per workgroup.
struct Q4pSrc {
    const uint8_t *x;  // activation chunks of the row tile
    const uint8_t *dx; // d_x chunks of the row tile
    const uint8_t *w;  // weight code chunks of the column tile
    const uint8_t *dw; // d_w chunks of the column tile
};

// One wave's loads of a stage.  The wave index is a template argument so
// that every region, block and part number below is a constant; only the
// block offsets (32-bit: the largest is nb chunks of at most 6 KB) and the
// clamp at nb - 1 remain per stage.
template <bool Q8W, int WAVE>
__device__ __forceinline__ void q4p_load_wave(const Q4pSrc &src, int nb, int b, Q4pLds<Q8W> &s)
{
    constexpr int WC = PFmt<Q8W>::kWChunk;
    const int lane = threadIdx.x & 63;
    const uint32_t lo = 16u * (uint32_t)lane;
    const uint8_t *xb = src.x + (uint32_t)b * (uint32_t)kPXChunk;
    const QLL_LDS char *xs = (const QLL_LDS char *)&s.xs[0][0];
    const QLL_LDS char *wq = (const QLL_LDS char *)&s.wq[0][0];
    const auto wblock = [&](int kb) { return (uint32_t)(b + kb < nb ? b + kb : nb - 1); };
#pragma unroll
    for (int j = 0; j < 3; j++) {
        constexpr int r0 = 3 * WAVE;
        q4p_dma16(xb + (r0 + j) * 1024, lo, xs + (r0 + j) * 1024);
    }
    if (Q8W) {
#pragma unroll
        for (int j = 0; j < 3; j++) {
            const int region = 3 * WAVE + j, kb = region / 6, part = region % 6;
            q4p_dma16(src.w + wblock(kb) * (uint32_t)WC + part * 1024, lo, wq + kb * WC + part * 1024);
        }
        if (lane < 16) {
            if (WAVE < 2)
                q4p_dma16(src.dx + (uint32_t)(b + WAVE) * (uint32_t)kPSChunk, lo, (const QLL_LDS void *)&s.dx[WAVE][0]);
            else
                q4p_dma16(src.dw + wblock(WAVE - 2) * (uint32_t)kPSChunk, lo,
                          (const QLL_LDS void *)&s.dw[WAVE - 2][0]);
        }
    } else {
        constexpr int nw = WAVE < 2 ? 2 : 1;
#pragma unroll
        for (int j = 0; j < nw; j++) {
            const int region = WAVE < 2 ? 2 * WAVE + j : 2 + WAVE;
            const int kb = region / 3, part = region % 3;
            q4p_dma16(src.w + wblock(kb) * (uint32_t)WC + part * 1024, lo, wq + kb * WC + part * 1024);
        }
        if (WAVE == 2 && lane < 32) {
            q4p_dma16(src.dx + (uint32_t)b * (uint32_t)kPSChunk, lo, (const QLL_LDS void *)&s.dx[0][0]);
        } else if (WAVE == 3 && lane < 32) {
            const int bb = b + (lane >> 4) < nb ? b + (lane >> 4) : nb - 1;
            q4p_dma16(src.dw, (uint32_t)bb * kPSChunk + 16u * (uint32_t)(lane & 15),
                      (const QLL_LDS void *)&s.dw[0][0]);
        }
    }
}

// The loads of the stage holding blocks b and b + 1.  Q4_0 weights, five
// per wave:
//   * activations: the two blocks' chunks are adjacent (12 KB), three 1 KB
//     loads per wave;
//   * weight codes: the two chunks (6 KB) as six 1 KB loads, two each for
//     waves 0 and 1, one each for waves 2 and 3; a block at or past nb
//     loads block nb - 1 (its activations are zero, so it adds nothing);
//   * wave 2, lanes 0..31: the d_x of both blocks (512 adjacent bytes);
//     wave 3, lanes 0..31: d_w of both blocks (clamped as above).
// Q8_0 weights, seven per wave: activations as above, the weight codes
// (12 KB) as three 1 KB loads per wave, and d_x (waves 0, 1) and d_w
// (waves 2, 3) one block per wave on lanes 0..15.
template <bool Q8W>
__device__ __forceinline__ void q4p_load_stage(const Q4pSrc &src, int nb, int b, int wave, Q4pLds<Q8W> &s)
{
    switch (wave) {
    case 0: q4p_load_wave<Q8W, 0>(src, nb, b, s); break;
    case 1: q4p_load_wave<Q8W, 1>(src, nb, b, s); break;
    case 2: q4p_load_wave<Q8W, 2>(src, nb, b, s); break;
    default: q4p_load_wave<Q8W, 3>(src, nb, b, s); break;
    }
}

template <typename T>
__device__ __forceinline__ T q4p_lds(const QLL_LDS char *base, uint32_t off)
{
    return *reinterpret_cast<const QLL_LDS T *>(base + off);
}

// Per-lane LDS byte offsets from the start of a stage buffer; reads add only
// immediates (block, tile) to them.
struct Q4pLaneOff {
    uint32_t x0, x1[2]; // this lane's activation planes (h for lanes 0..31, l for 32..63), tile rows 0 and 1
    uint32_t w0, w1[2]; // weight planes, tile columns 0 and 1, block 0
    uint32_t dx, dw;
};

template <bool Q8W>
__device__ __forceinline__ Q4pLaneOff q4p_lane_offsets(int wm, int wn, int lane)
{
    typedef Q4pLds<Q8W> Lds;
    const int lr = lane & 31, lh = lane >> 5;
    Q4pLaneOff o;
    o.x0 = (uint32_t)(offsetof(Lds, xs) + lh * 3072 + 16 * (wm + lr));
    o.w0 = (uint32_t)(offsetof(Lds, wq) + 16 * (wn + lr));
    o.dx = (uint32_t)(offsetof(Lds, dx) + 2 * (wm + lr));
    o.dw = (uint32_t)(offsetof(Lds, dw) + 2 * (wn + lr));
#pragma unroll
    for (int i = 0; i < 2; i++) {
        o.x1[i] = (uint32_t)(offsetof(Lds, xs) + lh * 3072 + 2048 + 8 * (wm + 32 * i + lr));
        o.w1[i] = (uint32_t)(offsetof(Lds, wq) + 2048 + 8 * (wn + 32 * i + lr));
    }
    // Opaque to the compiler, so that the two 8-byte reads of a block (tiles
    // 0 and 1, different base registers) are not merged into one read of
    // four registers, which would then have to be copied into the two
    // six-register MFMA operands.
    asm volatile("" : "+v"(o.x0), "+v"(o.x1[0]), "+v"(o.x1[1]), "+v"(o.w0), "+v"(o.w1[0]), "+v"(o.w1[1]),
                 "+v"(o.dx), "+v"(o.dw));
    return o;
}

// Operand fragments of the wave's 64 x 64 tile (2 x 2 tiles of 32 x 32) for
// one block.  Lane l holds row (column) l % 32 of its tile and K half l / 32:
// the h codes (A, scale 2^4) or l codes (A, scale 1) of its row, and the
// same 32 weight codes (B) in both halves.  The scale tile takes
// {d_x, 0, 0, 0} and {d_w, 0, 0, 0} in both lane halves, so S = 2 d_x d_w
// exactly; the outputs are halved at the end.
struct Q4pA {
    i32x8 x;   // activation codes of tile row i
    f16x4 s;   // {d_x, 0, 0, 0}
};
template <bool Q8W>
struct Q4pB {
    i32x8 m, l; // weight codes of tile column j (Q8_0 weights: h and l groups; Q4_0: m only)
    f16x4 s;    // {d_w, 0, 0, 0}
};

__device__ __forceinline__ void q4p_read_a(const QLL_LDS char *base, const Q4pLaneOff &o, int kb, int i, Q4pA &a)
{
    const u32x4 x0 = q4p_lds<u32x4>(base, o.x0 + kb * kPXChunk + 512 * i);
    const u32x2 x1 = q4p_lds<u32x2>(base, o.x1[i] + kb * kPXChunk);
    a.x = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], 0, 0};
    const uint32_t d = q4p_lds<uint16_t>(base, o.dx + kb * 2 * PBM + 64 * i);
    a.s = __builtin_bit_cast(f16x4, u32x2{d, 0u});
}

template <bool Q8W>
__device__ __forceinline__ void q4p_read_b(const QLL_LDS char *base, const Q4pLaneOff &o, int kb, int j,
                                           Q4pB<Q8W> &b)
{
    constexpr int WC = PFmt<Q8W>::kWChunk;
    const u32x4 w0 = q4p_lds<u32x4>(base, o.w0 + kb * WC + 512 * j);
    const u32x2 w1 = q4p_lds<u32x2>(base, o.w1[j] + kb * WC);
    b.m = i32x8{(int)w0[0], (int)w0[1], (int)w0[2], (int)w0[3], (int)w1[0], (int)w1[1], 0, 0};
    if (Q8W) { // the l half of the weight codes, 3072 bytes further
        const u32x4 v0 = q4p_lds<u32x4>(base, o.w0 + kb * WC + 3072 + 512 * j);
        const u32x2 v1 = q4p_lds<u32x2>(base, o.w1[j] + kb * WC + 3072);
        b.l = i32x8{(int)v0[0], (int)v0[1], (int)v0[2], (int)v0[3], (int)v1[0], (int)v1[1], 0, 0};
    }
    const uint32_t d = q4p_lds<uint16_t>(base, o.dw + kb * 2 * PBN + 64 * j);
    b.s = __builtin_bit_cast(f16x4, u32x2{d, 0u});
}

// The block sum P and the scale tile S of one 32 x 32 tile.
template <bool Q8W>
__device__ __forceinline__ void q4p_mfma(const Q4pA &a, const Q4pB<Q8W> &b, uint32_t scale_a, f32x16 &p, f32x16 &sc)
{
    if (Q8W) { // sum 16 h_w (16 h_x + l_x) + l_w (16 h_x + l_x)
        p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a.x, b.m, f32x16{}, 3, 3, 0, scale_a, 0, kE8M0Sixteen);
        p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a.x, b.l, p, 3, 3, 0, scale_a, 0, kE8M0One);
    } else {
        p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a.x, b.m, f32x16{}, 3, 3, 0, scale_a, 0, kE8M0One);
    }
    sc = __builtin_amdgcn_mfma_f32_32x32x8f16(a.s, b.s, f32x16{}, 0, 0, 0);
}

// Consecutive workgroup ids go to the 8 XCDs in turn; each XCD walks a
// contiguous run of (weight tile, all row tiles), so the row tiles that share
// a weight tile meet it in that XCD's L2.
__device__ __forceinline__ void q4p_tile(int64_t mt_count, int64_t nt_count, int64_t &m_tile, int64_t &n_tile)
{
    const int64_t total = mt_count * nt_count;
    const int64_t id = blockIdx.x;
    int64_t logical = id;
    if (total % 8 == 0)
        logical = (id % 8) * (total / 8) + id / 8;
    n_tile = logical / mt_count;
    m_tile = logical % mt_count;
}

// Wait until at most N vector-memory loads of this wave are outstanding and
// its LDS operations are done, then meet the workgroup.
template <int N>
__device__ __forceinline__ void q4p_sync()
{
    static_assert(N < 16, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(N | (0x7 << 4)); // vmcnt(N) expcnt(7) lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// One stage, computed from buffer CUR: steps t = 0..7 take block t / 4,
// tile (i, j) = ((t / 2) % 2, t % 2), whose fragments are A[i], B[j].  Each
// step issues its MFMAs, then the reads that refill the fragments just
// finished with (A[0] after step 1 of a block, B[0] after step 2, A[1] and
// B[1] after step 3) with those of the next block, two or three steps
// before their use, then the scale fmas of the step before it; the
// scheduling fences keep that order, so the vector ALU works on step t - 1
// while the matrix core works on step t.  After step 4 each wave waits for
// its loads of the next stage and the workgroup meets: every wave has then
// read this buffer whole (block 1 is in registers) and the next one is
// complete, so the loads of the stage three ahead go into this buffer at
// once, and steps 5..7 read the next stage's block 0.
template <bool Q8W, int CUR>
__device__ __forceinline__ void q4p_stage(Q4pLds<Q8W> *lds, const Q4pLaneOff &lo, uint32_t scale_a,
                                          f32x16 (&acc)[2][2], Q4pA (&A)[2], Q4pB<Q8W> (&B)[2], const Q4pSrc &src,
                                          int nb, int b_load, int swave)
{
    constexpr int DMA = PFmt<Q8W>::kDma;
    const QLL_LDS char *cur = (const QLL_LDS char *)&lds[CUR];
    const QLL_LDS char *nxt = (const QLL_LDS char *)&lds[(CUR + 1) % PNBUF];
    f32x16 p[2], sc[2];
#pragma unroll
    for (int t = 0; t <= 4 * PKB; t++) {
        if (t < 4 * PKB)
            q4p_mfma<Q8W>(A[(t >> 1) & 1], B[t & 1], scale_a, p[t & 1], sc[t & 1]);
        __builtin_amdgcn_sched_barrier(0);
        if (t == 4) {
            q4p_sync<DMA>();
            q4p_load_stage<Q8W>(src, nb, b_load, swave, lds[CUR]);
        }
        if (t < 4 * PKB) {
            const QLL_LDS char *rb = t < 4 ? cur : nxt;
            const int rkb = t < 4 ? 1 : 0;
            if ((t & 3) == 1)
                q4p_read_a(rb, lo, rkb, 0, A[0]);
            if ((t & 3) == 2)
                q4p_read_b<Q8W>(rb, lo, rkb, 0, B[0]);
            if ((t & 3) == 3) {
                q4p_read_a(rb, lo, rkb, 1, A[1]);
                q4p_read_b<Q8W>(rb, lo, rkb, 1, B[1]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (t > 0) {
            const int u = t - 1, ui = (u >> 1) & 1, uj = u & 1;
#pragma unroll
            for (int v = 0; v < 16; v++)
                acc[ui][uj][v] = fmaf(sc[u & 1][v], p[u & 1][v], acc[ui][uj][v]);
            // keeps these fmas in this step: the loads' branches split the
            // stage into blocks, and the compiler would otherwise sink each
            // fma to the next use of its accumulator
            asm volatile("" : "+v"(acc[ui][uj]));
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <bool Q8W>
__global__ __launch_bounds__(kPThreads) void packed_gemm_kernel(const uint8_t *__restrict__ wcodes,
                                                                const uint16_t *__restrict__ dws, Q4pPrep prep,
                                                                float *__restrict__ y, int64_t m, int64_t n, int nb,
                                                                int per_split)
{
    constexpr int DMA = PFmt<Q8W>::kDma;
    __shared__ Q4pLds<Q8W> lds[PNBUF];
    int64_t m_tile, n_tile;
    q4p_tile(prep.mp / PBM, (n + PBN - 1) / PBN, m_tile, n_tile);
    const int64_t m0 = m_tile * PBM, n0 = n_tile * PBN;
    const int b_begin = blockIdx.y * per_split;
    y += (int64_t)blockIdx.y * m * n;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
            acc[i][j] = f32x16{};

    const int nstages = per_split / PKB;
    const Q4pLaneOff lo = q4p_lane_offsets<Q8W>(wm, wn, lane);
    const uint32_t scale_a = lane < 32 ? kE8M0Sixteen : kE8M0One;

    // Three stage buffers, stage st computed from buffer st % 3 (the loop
    // runs three stages per trip, so every LDS address is a lane offset plus
    // an immediate).  The loads run three stages ahead; stages past the
    // range load padding (zero activations, clamped weights) and are never
    // computed.  Wave roles in the loads are uniform per wave, so the wave
    // index goes through a scalar register.
    Q4pSrc src;
    src.x = prep.x + m_tile * prep.nbp * kPXChunk;
    src.dx = reinterpret_cast<const uint8_t *>(prep.dx) + m_tile * prep.nbp * kPSChunk;
    src.w = wcodes + n_tile * nb * (int64_t)PFmt<Q8W>::kWChunk;
    src.dw = reinterpret_cast<const uint8_t *>(dws) + n_tile * nb * (int64_t)kPSChunk;
    const int swave = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
    for (int s0 = 0; s0 < PNBUF; s0++)
        q4p_load_stage<Q8W>(src, nb, b_begin + s0 * PKB, swave, lds[s0]);
    q4p_sync<DMA * (PNBUF - 1)>();
    Q4pA A[2];
    Q4pB<Q8W> B[2];
#pragma unroll
    for (int i = 0; i < 2; i++) {
        q4p_read_a((const QLL_LDS char *)&lds[0], lo, 0, i, A[i]);
        q4p_read_b<Q8W>((const QLL_LDS char *)&lds[0], lo, 0, i, B[i]);
    }
    int st = 0;
    for (; st + PNBUF <= nstages; st += PNBUF) {
        q4p_stage<Q8W, 0>(lds, lo, scale_a, acc, A, B, src, nb, b_begin + (st + 3) * PKB, swave);
        q4p_stage<Q8W, 1>(lds, lo, scale_a, acc, A, B, src, nb, b_begin + (st + 4) * PKB, swave);
        q4p_stage<Q8W, 2>(lds, lo, scale_a, acc, A, B, src, nb, b_begin + (st + 5) * PKB, swave);
    }
    if (st < nstages)
        q4p_stage<Q8W, 0>(lds, lo, scale_a, acc, A, B, src, nb, b_begin + (st + 3) * PKB, swave);
    if (st + 1 < nstages)
        q4p_stage<Q8W, 1>(lds, lo, scale_a, acc, A, B, src, nb, b_begin + (st + 4) * PKB, swave);
    // no load may still be writing this workgroup's LDS when it ends
    __builtin_amdgcn_s_waitcnt(0x7 << 4); // vmcnt(0) expcnt(7) lgkmcnt(0)

#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int v = 0; v < 16; v++) {
                const int64_t row = m0 + wm + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                const int64_t col = n0 + wn + 32 * j + (lane & 31);
                if (row < m && col < n)
                    y[row * n + col] = 0.5f * acc[i][j][v]; // the scale tiles are 2 d_x d_w
            }
}


// Split k when the output tiles alone leave workgroup slots empty (two
// workgroups fit per CU); each split keeps at least 16 blocks and a multiple
// of 2 PKB of them.  Workspace: split partials (if any), prepared
// activations, d_x.
struct Q4pPlan {
    int splits, per_split;
    int64_t mp, nbp;
    size_t x_off, dx_off, total;
};

static Q4pPlan q4p_plan(int64_t m, int64_t n, int64_t k)
{
    Q4pPlan p;
    const int64_t nb = k / 32;
    p.mp = (m + PBM - 1) / PBM * PBM;
    const int64_t tiles = ((n + PBN - 1) / PBN) * (p.mp / PBM);
    int64_t s = 512 / tiles;
    if (s > nb / 16)
        s = nb / 16;
    if (s > 8)
        s = 8;
    if (s < 2)
        s = 1;
    const int64_t q = 2 * PKB;
    int64_t per = (nb + s - 1) / s;
    per = (per + q - 1) / q * q;
    s = (nb + per - 1) / per;
    p.splits = (int)s;
    p.per_split = (int)per;
    // the last split's range plus the stages the pipeline loads past it
    p.nbp = per * s + PNBUF * PKB;
    auto up = [](size_t v) { return (v + 255) / 256 * 256; };
    const size_t parts = s > 1 ? up((size_t)s * (size_t)(m * n) * sizeof(float)) : 0;
    const size_t chunks = (size_t)(p.mp / PBM) * (size_t)p.nbp;
    p.x_off = parts;
    p.dx_off = p.x_off + up(chunks * kPXChunk);
    p.total = p.dx_off + up(chunks * kPSChunk);
    return p;
}

size_t q4_0_packed_gemm_workspace(int64_t m, int64_t n, int64_t k)
{
    return q4p_plan(m, n, k).total;
}

template <bool Q8W>
static hipError_t launch_packed_gemm(const uint8_t *wp, const uint8_t *xq, float *y, int64_t m, int64_t n, int64_t k,
                                     void *ws, hipStream_t s)
{
    const Q4pPlan plan = q4p_plan(m, n, k);
    uint8_t *base = static_cast<uint8_t *>(ws);
    Q4pPrep prep;
    prep.x = base + plan.x_off;
    prep.dx = reinterpret_cast<uint16_t *>(base + plan.dx_off);
    prep.mp = plan.mp;
    prep.nbp = plan.nbp;
    const int nb = (int)(k / 32);
    const int64_t prep_threads = plan.mp * plan.nbp;
    hipLaunchKernelGGL(q4p_prep_kernel, dim3((unsigned)((prep_threads + 255) / 256)), dim3(256), 0, s, xq, prep, m,
                       nb, prep_threads);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int64_t nt = (n + PBN - 1) / PBN;
    const uint16_t *dws = reinterpret_cast<const uint16_t *>(wp + (size_t)nt * nb * PFmt<Q8W>::kWChunk);
    const int64_t tiles = nt * (plan.mp / PBM);
    float *out = plan.splits > 1 ? reinterpret_cast<float *>(base) : y;
    hipLaunchKernelGGL(packed_gemm_kernel<Q8W>, dim3((unsigned)tiles, (unsigned)plan.splits), dim3(kPThreads), 0, s,
                       wp, dws, prep, out, m, n, nb, plan.per_split);
    e = hipGetLastError();
    if (e != hipSuccess || plan.splits == 1)
        return e;
    return launch_sum_splits(out, y, m * n, plan.splits, s);
}

hipError_t launch_q4_0_packed_gemm(const uint8_t *wp, const uint8_t *xq, float *y, int64_t m, int64_t n, int64_t k,
                                   void *ws, hipStream_t s)
{
    return launch_packed_gemm<false>(wp, xq, y, m, n, k, ws, s);
}

// ------------------------------------------------------------------ Q8_0 weights

// Q8_0 weights W[n][k/32] repacked exactly as the prepass prepares activation
// rows: the same chunks over 128-row tiles (h and l code groups of each
// row, 6144 bytes per chunk), then d_w, 128 binary16 per chunk.
size_t q8_0_repacked_bytes(int64_t n, int64_t k)
{
    const int64_t nt = (n + PBN - 1) / PBN;
    return (size_t)nt * (size_t)(k / 32) * (2 * kPWChunk + kPSChunk);
}

hipError_t launch_q8_0_repack(const uint8_t *w, uint8_t *wp, int64_t n, int64_t k, hipStream_t s)
{
    const int nb = (int)(k / 32);
    const int64_t nt = (n + PBN - 1) / PBN;
    Q4pPrep p;
    p.x = wp;
    p.dx = reinterpret_cast<uint16_t *>(wp + (size_t)nt * nb * (2 * kPWChunk));
    p.mp = nt * PBN;
    p.nbp = nb;
    const int64_t total = p.mp * nb;
    const int64_t grid = (total + 255) / 256;
    if (grid > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(q4p_prep_kernel, dim3((unsigned)grid), dim3(256), 0, s, w, p, n, nb, total);
    return hipGetLastError();
}

hipError_t launch_q8_0_packed_gemm(const uint8_t *wp, const uint8_t *xq, float *y, int64_t m, int64_t n, int64_t k,
                                   void *ws, hipStream_t s)
{
    return launch_packed_gemm<true>(wp, xq, y, m, n, k, ws, s);
}

} // namespace qll
