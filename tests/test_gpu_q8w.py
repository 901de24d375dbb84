"""Parity of the Q8_0-weight path (weights and activations both Q8_0 blocks)
against the oracle: the decode GEMV on the Q8_0 bytes, the load-time repack
(decoded in numpy from the e3m2 definition: 16 h + l must give back every
code), and the prefill GEMM on repacked weights.  Float outputs within
1e-4 * sum_b |term_b|; unit-scale cases bit-exact (the outputs are integers
below 2^24); weight codes over the whole int8 range, -128 included."""
import numpy as np
import pytest
import torch

import oracle as O
import quantized_linear_layer_amd as qll
import synth
from gpu_util import assert_within, dev, empty, host, quantize_q8_0
from pins import np_pack_q8_0
from test_gpu_q4_repacked import e3m2_value

pytestmark = pytest.mark.gpu
TOL = 1e-4


def upload_q8w(codes, d_bits):
    # block_q8_0 bytes laid out by the tests' own numpy packer (the oracle only checks)
    return dev(np_pack_q8_0(codes, d_bits).reshape(-1))


def gemv(w, xq, n, k):
    y = empty(n, torch.float32)
    qll.qll_q8_0_q8_0_gemv(w, xq, y, n, k)
    return y


def repack(w, n, k):
    wp = empty(qll.qll_q8_0_repacked_bytes(n, k))
    qll.qll_q8_0_repack(w, wp, n, k)
    return wp


def gemm(wp, xq, m, n, k):
    y = empty(m * n, torch.float32)
    ws = empty(qll.qll_workspace_bytes(qll.QLL_OP_Q8_0_REPACKED_GEMM, m, n, k))
    qll.qll_q8_0_repacked_q8_0_gemm(wp, xq, y, m, n, k, ws=ws)
    return y


def _case(seed, m, n, k):
    rng = np.random.default_rng(seed)
    codes, d_bits = synth.q8_0_weights(rng, n, k)
    codes[rng.random((n, k)) < 0.01] = -128
    return codes, d_bits, synth.normal_f32(rng, (m, k))


@pytest.mark.parametrize("n", [1, 3, 7, 17, 64, 129, 257])
@pytest.mark.parametrize("k", [32, 64, 96, 512, 4096, 8224, 14336])
def test_gemv_shapes(qll_gpu, n, k):
    codes, d_bits, x = _case(n * 100 + k, 1, n, k)
    y = host(gemv(upload_q8w(codes, d_bits), quantize_q8_0(x), n, k))
    y_ref, mag = O.q8_0_q8_0(O.pack_q8_0(codes, d_bits), O.quantize_q8_0(x), 1, n, k)
    assert_within(y, y_ref[0], mag[0], TOL, f"Q8_0 GEMV n={n} k={k}")


@pytest.mark.parametrize("n,k", [(5, 49152), (4, 28704)])
def test_gemv_largest_k(qll_gpu, n, k):
    codes, d_bits, x = _case(n * 100 + k, 1, n, k)
    y = host(gemv(upload_q8w(codes, d_bits), quantize_q8_0(x), n, k))
    y_ref, mag = O.q8_0_q8_0(O.pack_q8_0(codes, d_bits), O.quantize_q8_0(x), 1, n, k)
    assert_within(y, y_ref[0], mag[0], TOL, f"Q8_0 GEMV n={n} k={k}")


@pytest.mark.parametrize("s", range(4))
def test_gemv_8b_shapes_full(qll_gpu, s):
    codes, d_bits, x = synth.q8w_decode(s)
    n, k = codes.shape
    y = host(gemv(upload_q8w(codes, d_bits), quantize_q8_0(x), n, k))
    y_ref, mag = O.q8_0_q8_0(O.pack_q8_0(codes, d_bits), O.quantize_q8_0(x), 1, n, k)
    assert_within(y, y_ref[0], mag[0], TOL, f"Q8_0 GEMV {synth.SHAPES_8B[s]}")


def _unit_x(rng, m, k):
    x = rng.integers(-126, 127, (m, k)).astype(np.float32)
    x[rng.random((m, k)) < 0.25] += np.float32(0.5)
    x[:, ::32] = np.where(rng.random((m, k // 32)) < 0.5, 127.0, -127.0)
    return x


def _int_want(x, codes):
    q = np.asarray(O.quantize_q8_0(x), np.uint8).reshape(x.shape[0], -1, 34)
    assert np.all(q[:, :, :2].view(np.uint16) == 0x3c00)
    qx = q[:, :, 2:].view(np.int8).reshape(x.shape).astype(np.int64)
    return qx @ codes.astype(np.int64).T


@pytest.mark.parametrize("m,n,k", [(1, 40, 512), (1, 9, 14336), (1, 5, 96), (70, 150, 1024), (129, 33, 4096),
                                   (3, 9, 96)])
def test_unit_scales_bit_exact(qll_gpu, m, n, k):
    rng = np.random.default_rng(m + n + k)
    codes = rng.integers(-128, 128, (n, k)).astype(np.int8)
    codes[0, :64] = -128
    d_bits = np.full((n, k // 32), 0x3c00, np.uint16)
    x = _unit_x(rng, m, k)
    want = _int_want(x, codes).astype(np.float64)
    w = upload_q8w(codes, d_bits)
    xq = quantize_q8_0(x)
    if m == 1:
        assert np.array_equal(host(gemv(w, xq, n, k)).astype(np.float64), want[0])
    y = host(gemm(repack(w, n, k), xq, m, n, k)).reshape(m, n)
    assert np.array_equal(y.astype(np.float64), want)


@pytest.mark.parametrize("n,k", [(1, 32), (5, 96), (129, 320), (300, 4096)])
def test_repack_decodes_to_codes(qll_gpu, n, k):
    rng = np.random.default_rng(n * 3 + k)
    codes, d_bits = synth.q8_0_weights(rng, n, k)
    codes[0, :32] = -128
    wp = host(repack(upload_q8w(codes, d_bits), n, k))
    nb, nt = k // 32, (n + 127) // 128
    assert wp.size == nt * nb * 6400
    raw = wp[:nt * nb * 6144].reshape(nt, nb, 2, 3072)

    def planes(part):
        p0 = part[:, :, :2048].reshape(nt, nb, 128, 16)
        p1 = part[:, :, 2048:].reshape(nt, nb, 128, 8)
        bits = np.unpackbits(np.concatenate([p0, p1], axis=3), axis=3, bitorder="little")
        code = (bits.reshape(nt, nb, 128, 32, 6) * (1 << np.arange(6))).sum(axis=4)
        return e3m2_value(code).transpose(0, 2, 1, 3).reshape(nt * 128, k)

    h, l = planes(raw[:, :, 0]), planes(raw[:, :, 1])
    assert np.all(np.abs(h) <= 8) and np.all((l >= -8) & (l <= 7))
    assert np.array_equal(16 * h[:n] + l[:n], codes.astype(np.float64))
    assert np.all(h[n:] == 0) and np.all(l[n:] == 0)
    d = wp[nt * nb * 6144:].view(np.uint16).reshape(nt, nb, 128).transpose(0, 2, 1).reshape(nt * 128, nb)
    assert np.array_equal(d[:n], d_bits) and np.all(d[n:] == 0)


@pytest.mark.parametrize("m,n,k", [(1, 7, 32), (2, 1, 32), (3, 7, 96), (17, 64, 512), (130, 129, 320),
                                   (128, 128, 4096), (200, 300, 64), (64, 33, 14336), (128, 256, 3232),
                                   (257, 131, 608)])
def test_gemm_shapes(qll_gpu, m, n, k):
    codes, d_bits, x = _case(m * 1000 + n + k + 5, m, n, k)
    y = host(gemm(repack(upload_q8w(codes, d_bits), n, k), quantize_q8_0(x), m, n, k)).reshape(m, n)
    y_ref, mag = O.q8_0_q8_0(O.pack_q8_0(codes, d_bits), O.quantize_q8_0(x), m, n, k)
    assert_within(y, y_ref, mag, TOL, f"Q8_0 GEMM m={m} n={n} k={k}")


def test_gemm_one_hot(qll_gpu):
    m, n, k = 32, 20, 320
    rng = np.random.default_rng(5)
    codes = rng.integers(-128, 128, (n, k)).astype(np.int8)
    d_bits = np.full((n, k // 32), 0x3c00, np.uint16)
    x = np.zeros((m, k), np.float32)
    pos = rng.integers(0, k, m)
    x[np.arange(m), pos] = 127.0
    y = host(gemm(repack(upload_q8w(codes, d_bits), n, k), quantize_q8_0(x), m, n, k)).reshape(m, n)
    assert np.array_equal(y.astype(np.float64), 127.0 * codes[:, pos].T.astype(np.float64))


@pytest.mark.parametrize("s", range(4))
def test_gemm_prefill_8b_shapes_full(qll_gpu, s):
    # full prefill size (m = 512), every output against the oracle
    import full_refs
    wq, x, y_ref, mag = full_refs.q8w_prefill(s)
    m, k = x.shape
    n = wq.shape[0]
    wp = repack(dev(wq.reshape(-1)), n, k)
    y = host(gemm(wp, quantize_q8_0(x), m, n, k)).reshape(m, n)
    assert_within(y, y_ref, mag, TOL, f"Q8_0 prefill {synth.SHAPES_8B[s]}")
    del wp
    torch.cuda.empty_cache()
