"""Parity of the Q4_0 x Q8_0 path on the GPU against the oracle: packing and
Q8_0 quantization bit-exact, block sums bit-exact through the unit-scale and
power-of-two cases, float outputs within 1e-4 * sum_b |term_b|."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from gpu_util import assert_within, host, pack_q4_0, q4_gemm, q4_gemv, quantize_q8_0

pytestmark = pytest.mark.gpu
TOL = 1e-4


def rand_case(seed, m, n, k):
    rng = np.random.default_rng(seed)
    codes, d_bits = synth.q4_0_weights(rng, n, k)
    x = synth.normal_f32(rng, (m, k))
    return codes, d_bits, x


@pytest.mark.parametrize("n,k", [(1, 32), (3, 96), (7, 320), (64, 512), (5, 4096), (33, 14336)])
def test_pack_q4_0_bit_exact(qll_gpu, n, k):
    codes, d_bits, _ = rand_case(n * 7 + k, 1, n, k)
    w = pack_q4_0(codes, d_bits)
    assert np.array_equal(host(w), O.pack_q4_0(codes, d_bits).reshape(-1))


@pytest.mark.parametrize("m,k", [(1, 32), (1, 96), (3, 352), (17, 4096), (1, 14336), (33, 64)])
def test_quantize_q8_0_bit_exact(qll_gpu, m, k):
    rng = np.random.default_rng(m * 100 + k)
    x = synth.normal_f32(rng, (m, k))
    x[0, :32] = 0.0                                    # a zero block
    if k >= 64:
        x[0, 32:64] *= np.float32(1e-6)                # a block with a subnormal fp16 scale
    if k >= 96:
        x[0, 64:96] = np.array([127.0, 0.5, -0.5, 2.5, -2.5, 126.5, -126.5] + [1.5] * 25, np.float32)
    xq = quantize_q8_0(x)
    assert np.array_equal(host(xq), O.quantize_q8_0(x).reshape(-1))


def test_quantize_q8_0_f32_quotient_ties(qll_gpu):
    # Inputs whose IEEE f32 quotient x/d rounds onto k + 1/2 while the exact
    # quotient lies below it: only a kernel that divides in f32 and rounds
    # half away from zero gives the oracle's codes.
    import pins
    sets = pins._f32_tie_crossings(np.random.default_rng(25), 64, quotient=True)
    x = np.zeros((2, 32 * 32), np.float32)
    for b, (amax, xs) in enumerate(sets):
        row, col = divmod(b, 32)
        x[row, 32 * col] = -amax if b % 3 == 0 else amax
        x[row, 32 * col + 1:32 * col + 32] = xs
    assert np.array_equal(host(quantize_q8_0(x)), O.quantize_q8_0(x).reshape(-1))


def test_quantize_q8_0_prefill_size(qll_gpu):
    x = synth.q4_prefill_x(0)
    assert np.array_equal(host(quantize_q8_0(x)), O.quantize_q8_0(x).reshape(-1))


def _gemv_check(codes, d_bits, x, what):
    n, k = codes.shape
    w = pack_q4_0(codes, d_bits)
    xq = quantize_q8_0(x)
    y = host(q4_gemv(w, xq, n, k))
    y_ref, mag = O.q4_0_q8_0(O.pack_q4_0(codes, d_bits), O.quantize_q8_0(x), 1, n, k)
    assert_within(y, y_ref[0], mag[0], TOL, what)
    return y, y_ref[0]


def test_gemv_small_layer(qll_gpu):
    codes, d_bits, x = synth.q4_small()
    _gemv_check(codes, d_bits, x, "Q4_0 GEMV 512x512")


@pytest.mark.parametrize("n", [1, 3, 7, 8, 15, 16, 17, 31, 64, 128, 257])
@pytest.mark.parametrize("k", [32, 64, 96, 256, 512, 1024, 4096, 8192, 16384])
def test_gemv_adversarial_shapes(qll_gpu, n, k):
    codes, d_bits, x = rand_case(n * 31 + k, 1, n, k)
    _gemv_check(codes, d_bits, x, f"GEMV n={n} k={k}")


@pytest.mark.parametrize("n,k", [(5, 49152), (9, 28672), (3, 16416)])
def test_gemv_largest_k(qll_gpu, n, k):
    # k = 49152 is the largest the entry accepts (60 KiB of staged activation
    # in LDS); 16416 (513 blocks) is the first k past the two blocks per thread
    # that the staging holds in registers
    codes, d_bits, x = rand_case(n * 31 + k, 1, n, k)
    _gemv_check(codes, d_bits, x, f"GEMV n={n} k={k}")


@pytest.mark.parametrize("s", range(4))
def test_gemv_8b_shapes_full(qll_gpu, s):
    codes, d_bits, x = synth.q4_decode(s)
    _gemv_check(codes, d_bits, x, f"GEMV 8B shape {synth.SHAPES_8B[s]}")


def _unit_scale_x(rng, m, k):
    # integer-valued activations with a +-127 in every block: d = 127/127 = 1
    x = rng.integers(-127, 128, (m, k)).astype(np.float32)
    x[:, ::32] = 127.0
    return x


@pytest.mark.parametrize("n,k", [(40, 512), (17, 4096), (9, 14336), (5, 96)])
def test_gemv_unit_scales_bit_exact(qll_gpu, n, k):
    # dw = dx = 1: y is the integer sum of the block sums, |y| < 2^24, so any
    # f32 summation order gives it exactly.
    rng = np.random.default_rng(n + k)
    codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
    d_bits = np.full((n, k // 32), 0x3c00, np.uint16)
    x = _unit_scale_x(rng, 1, k)
    y, _ = _gemv_check(codes, d_bits, x, "unit scales")
    want = x.astype(np.int64) @ (codes.astype(np.int64) - 8).T
    assert np.array_equal(y.astype(np.float64), want[0].astype(np.float64))


def test_gemv_power_of_two_scales_bit_exact(qll_gpu):
    rng = np.random.default_rng(3)
    n, k = 33, 4096
    codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
    d_bits = np.full((n, k // 32), 0x2000, np.uint16)  # 2^-7
    x = _unit_scale_x(rng, 1, k) * np.float32(2.0 ** -3) * np.float32(127.0 / 127.0)
    y, y_ref = _gemv_check(codes, d_bits, x, "power-of-two scales")
    assert np.array_equal(y.astype(np.float64), y_ref)


def test_gemv_one_hot(qll_gpu):
    # x = 0 except x_p = 127: y_j = dw[j, p/32] * (code[j, p] - 8) * 127 exactly
    rng = np.random.default_rng(4)
    n, k = 64, 512
    codes, d_bits = synth.q4_0_weights(rng, n, k)
    w = pack_q4_0(codes, d_bits)
    dw = d_bits.view(np.float16).astype(np.float64)
    for p in list(range(32)) + [33, 200, 511]:
        x = np.zeros((1, k), np.float32)
        x[0, p] = 127.0
        y = host(q4_gemv(w, quantize_q8_0(x), n, k))
        want = dw[:, p // 32] * (codes[:, p].astype(np.float64) - 8.0) * 127.0
        assert np.array_equal(y.astype(np.float64), want), p


def test_gemv_zero_cases(qll_gpu):
    rng = np.random.default_rng(6)
    n, k = 20, 256
    codes, d_bits = synth.q4_0_weights(rng, n, k)
    y = host(q4_gemv(pack_q4_0(codes, d_bits), quantize_q8_0(np.zeros((1, k), np.float32)), n, k))
    assert np.all(y == 0)
    x = synth.normal_f32(rng, (1, k))
    y = host(q4_gemv(pack_q4_0(np.full((n, k), 8, np.uint8), d_bits), quantize_q8_0(x), n, k))
    assert np.all(y == 0)


def test_gemv_deterministic(qll_gpu):
    codes, d_bits, x = synth.q4_decode(0)
    n, k = codes.shape
    w = pack_q4_0(codes, d_bits)
    xq = quantize_q8_0(x)
    y1 = host(q4_gemv(w, xq, n, k))
    y2 = host(q4_gemv(w, xq, n, k))
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


def _gemm_check(codes, d_bits, x, what):
    n, k = codes.shape
    m = x.shape[0]
    w = pack_q4_0(codes, d_bits)
    xq = quantize_q8_0(x)
    y = host(q4_gemm(w, xq, m, n, k)).reshape(m, n)
    y_ref, mag = O.q4_0_q8_0(O.pack_q4_0(codes, d_bits), O.quantize_q8_0(x), m, n, k)
    assert_within(y, y_ref, mag, TOL, what)
    return y, y_ref, w, xq


# (128, 256, 3232): 101 blocks split six ways -- the last split holds one real
# block and 19 of padding; (257, 131, 608): odd block count, three row tiles
# with a one-row tail, weight buffer length 2 mod 4 (131 x 19 blocks)
@pytest.mark.parametrize("m,n,k", [(2, 1, 32), (3, 7, 96), (17, 64, 512), (130, 129, 320), (128, 128, 4096),
                                   (200, 300, 64), (64, 33, 14336), (128, 256, 3232), (257, 131, 608),
                                   # split k with m * n odd (the split sum's scalar path) and even
                                   (65, 33, 14336), (129, 131, 4096), (66, 34, 8192),
                                   # 9 <= m <= 32: the small-m kernels
                                   (9, 257, 4096), (32, 1000, 1024), (31, 128, 96), (20, 33, 14336), (12, 129, 32)])
def test_gemm_shapes(qll_gpu, m, n, k):
    codes, d_bits, x = rand_case(m * 1000 + n + k, m, n, k)
    _gemm_check(codes, d_bits, x, f"GEMM m={m} n={n} k={k}")


def test_gemm_unit_scales_bit_exact(qll_gpu):
    rng = np.random.default_rng(8)
    m, n, k = 70, 150, 1024
    codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
    d_bits = np.full((n, k // 32), 0x3c00, np.uint16)
    x = _unit_scale_x(rng, m, k)
    y, _, _, _ = _gemm_check(codes, d_bits, x, "GEMM unit scales")
    want = x.astype(np.int64) @ (codes.astype(np.int64) - 8).T
    assert np.array_equal(y.astype(np.float64), want.astype(np.float64))


def test_gemm_small_tile_unit_scales_bit_exact(qll_gpu):
    # the small-m band (9 <= m <= 32) on integer-valued outputs
    rng = np.random.default_rng(18)
    m, n, k = 20, 300, 2048
    codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
    d_bits = np.full((n, k // 32), 0x3c00, np.uint16)
    x = _unit_scale_x(rng, m, k)
    y, _, _, _ = _gemm_check(codes, d_bits, x, "GEMM m=20 unit scales")
    want = x.astype(np.int64) @ (codes.astype(np.int64) - 8).T
    assert np.array_equal(y.astype(np.float64), want.astype(np.float64))


@pytest.mark.parametrize("s,m", [(0, 16), (1, 9), (2, 32)])
def test_gemm_small_tile_8b_shapes_full(qll_gpu, s, m):
    # the small-m band (9 <= m <= 32) at an 8B-class layer's full size,
    # every output checked: the shape's weights with the first m rows of its
    # prefill input
    codes, d_bits, _ = synth.q4_decode(s)
    x = synth.q4_prefill_x(s, m=m)
    _gemm_check(codes, d_bits, x, f"GEMM m={m} 8B shape {synth.SHAPES_8B[s]}")


def test_gemm_rows_match_gemv(qll_gpu):
    codes, d_bits, x = rand_case(9, 24, 96, 512)
    y, y_ref, w, xq = _gemm_check(codes, d_bits, x, "GEMM")
    n, k = codes.shape
    for i in (0, 5, 23):
        xqi = quantize_q8_0(x[i:i + 1])
        yi = host(q4_gemv(w, xqi, n, k))
        _, mag = O.q4_0_q8_0(O.pack_q4_0(codes, d_bits), O.quantize_q8_0(x[i:i + 1]), 1, n, k)
        assert np.all(np.abs(yi - y[i]) <= 2 * TOL * mag[0])


@pytest.mark.parametrize("s", range(4))
def test_gemm_prefill_8b_shapes_full(qll_gpu, s):
    # full prefill size (m = 512), every output against the oracle
    import full_refs
    codes, d_bits, x, y_ref, mag = full_refs.q4_prefill(s)
    n, k = codes.shape
    m = x.shape[0]
    w = pack_q4_0(codes, d_bits)
    xq = quantize_q8_0(x)
    y = host(q4_gemm(w, xq, m, n, k)).reshape(m, n)
    assert_within(y, y_ref, mag, TOL, f"prefill shape {synth.SHAPES_8B[s]}")
    del w, xq
    torch.cuda.empty_cache()
