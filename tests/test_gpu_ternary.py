"""Parity of the BitNet ternary path on the GPU against the oracle: packing
and int8 row quantization bit-exact, code sums bit-exact through the
unit-scale case, outputs within 1e-4 * sum_t |(c - 1) q| * w_scale / act_scale."""
import numpy as np
import pytest

import oracle as O
import synth
from gpu_util import assert_within, dev, host, pack_ternary, quantize_i8_rows, ternary

pytestmark = pytest.mark.gpu
TOL = 1e-4


@pytest.mark.parametrize("n,k", [(1, 16), (3, 48), (7, 160), (64, 2560), (6912, 2560)])
def test_pack_bit_exact(qll_gpu, n, k):
    codes = synth.ternary_codes(np.random.default_rng(n + k), n, k)
    w = pack_ternary(codes)
    assert np.array_equal(host(w).view(np.uint32), O.pack_ternary(codes).reshape(-1))


@pytest.mark.parametrize("m,k", [(1, 16), (3, 2560), (64, 2560), (5, 30), (2, 1027),
                                 (2, 4096), (2, 4100)])  # rows held in registers up to 4096, not at 4100
def test_quantize_i8_rows_bit_exact(qll_gpu, m, k):
    rng = np.random.default_rng(m * 13 + k)
    x = synth.normal_f32(rng, (m, k))
    if m >= 3:
        x[1] = 0.0
        x[2, :8] = [127.0, 0.5, -0.5, 2.5, -2.5, 126.5, -126.5, 1.5]
        x[2, 8:] = np.clip(x[2, 8:], -100, 100)
    q, s, t = quantize_i8_rows(x)
    q_ref, s_ref, t_ref = O.quantize_i8_rows(x)
    assert np.array_equal(host(q).reshape(m, k), q_ref)
    assert np.array_equal(host(s).view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(host(t), t_ref)


def test_quantize_i8_rows_f32_product_ties(qll_gpu):
    # Rows whose f32 product x * (127/amax) rounds onto k + 1/2 while the exact
    # product lies below it (f32 product, then half away from zero).
    import pins
    sets = pins._f32_tie_crossings(np.random.default_rng(26), 16, quotient=False)
    x = np.zeros((len(sets), 2560), np.float32)
    for i, (amax, xs) in enumerate(sets):
        x[i, 7 * i] = -amax if i % 2 else amax
        x[i, 100:100 + 31] = xs
        x[i, 2000:2031] = xs[::-1]
    q, s, t = quantize_i8_rows(x)
    q_ref, s_ref, t_ref = O.quantize_i8_rows(x)
    assert np.array_equal(host(q).reshape(x.shape), q_ref)
    assert np.array_equal(host(s).view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(host(t), t_ref)


def _check(codes, w_scale, x, what):
    n, k = codes.shape
    m = x.shape[0]
    w = pack_ternary(codes)
    q, s, t = quantize_i8_rows(x)
    y = host(ternary(w, w_scale, q, s, t, m, n, k)).reshape(m, n)
    q_ref, s_ref, t_ref = O.quantize_i8_rows(x)
    y_ref, mag = O.ternary(O.pack_ternary(codes), w_scale, q_ref, s_ref, t_ref, n, k)
    assert_within(y, y_ref, mag, TOL, what)
    return y


@pytest.mark.parametrize("m", [1, 64])
def test_bitnet_layer_full(qll_gpu, m):
    codes, w_scale, x = synth.ternary_layer()
    _check(codes, w_scale, x[:m], f"ternary 2560->6912 m={m}")


@pytest.mark.parametrize("m,n,k", [(1, 1, 16), (1, 7, 48), (1, 33, 160), (1, 257, 1024), (2, 5, 16), (3, 17, 48),
                                   (17, 31, 160), (65, 40, 2560), (130, 70, 1024), (64, 16, 64),
                                   (5, 70, 14336), (33, 9, 4112),  # long k: several register buffers per wave
                                   (2, 33, 1088), (16, 32, 2048), (40, 100, 192), (100, 3, 4160),  # partial last chunks
                                   # m = 1, k % 64 == 0: several chunks per row, a partial chunk, and
                                   # activations beyond the pieces a thread stages from registers (k > 16384)
                                   (1, 37, 16384), (1, 19, 65536), (1, 5, 4160), (1, 70, 6208), (1, 130, 192),
                                   # m > 1, k % 64 == 0: the GEMM's k split over 1..6 waves (by grid size
                                   # and chunk count), several chunks per wave, ragged tiles
                                   (1030, 2050, 1088), (7, 130, 3072), (33, 65, 6208),
                                   # k % 128 == 0, k <= 3072, at most 256 tiles: the eight-wave burst
                                   # kernel, with waves left without steps (k = 128, 384, 1280, 2688),
                                   # second parts shorter than the first (1280, 1920, 2560) or as long
                                   # (3072), ragged tiles, and a grid of exactly 256 tiles; k = 6912
                                   # beside it goes to the k-split kernel
                                   (3, 70, 128), (40, 65, 384), (2, 64, 1280), (33, 100, 2560), (9, 200, 2688),
                                   (20, 90, 1920), (64, 2560, 6912), (50, 8190, 256)])
def test_shapes(qll_gpu, m, n, k):
    rng = np.random.default_rng(m * 100 + n * 7 + k)
    codes = synth.ternary_codes(rng, n, k)
    x = synth.normal_f32(rng, (m, k))
    _check(codes, np.float32(0.037), x, f"ternary m={m} n={n} k={k}")


@pytest.mark.parametrize("m", [1, 9])
def test_unit_scale_bit_exact(qll_gpu, m):
    rng = np.random.default_rng(11)
    n, k = 300, 2560
    codes = synth.ternary_codes(rng, n, k)
    x = rng.integers(-127, 128, (m, k)).astype(np.float32)
    x[:, 5] = 127.0
    y = _check(codes, np.float32(1.0), x, "unit scale")
    want = x.astype(np.int64) @ (codes.astype(np.int64) - 1).T
    assert np.array_equal(y.astype(np.float64), want.astype(np.float64))


def test_one_hot_and_zero_rows(qll_gpu):
    rng = np.random.default_rng(12)
    n, k = 40, 64
    codes = synth.ternary_codes(rng, n, k)
    w = pack_ternary(codes)
    for p in list(range(16)) + [16, 31, 63]:
        x = np.zeros((2, k), np.float32)
        x[0, p] = 127.0  # row 1 stays zero
        q, s, t = quantize_i8_rows(x)
        y = host(ternary(w, np.float32(1.0), q, s, t, 2, n, k)).reshape(2, n)
        assert np.array_equal(y[0].astype(np.float64), 127.0 * (codes[:, p].astype(np.float64) - 1.0)), p
        assert np.all(y[1] == 0)
        y1 = host(ternary(w, np.float32(1.0), q, s, t, 1, n, k))
        assert np.array_equal(y1, y[0])
