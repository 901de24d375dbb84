"""The decode-packed Q4_0 layout (per row: a plane of the blocks' 16 nibble
bytes, then a plane of their binary16 scales padded to 16 bytes) and the
decode GEMV on it.  The layout is read
back in numpy, byte for byte, against the codes and scales it was packed
from; the GEMV is checked against the oracle's Q4_0 x Q8_0 product of the
original weights (1e-4 * sum_b |term_b|), bit-exact where every partial sum
is an integer below 2^24."""
import numpy as np
import pytest
import torch

import oracle as O
import quantized_linear_layer_amd as qll
import synth
from gpu_util import assert_within, dev, empty, host, pack_q4_0, quantize_q8_0

pytestmark = pytest.mark.gpu
TOL = 1e-4


def decode_pack(w, n, k):
    wp = empty(qll.qll_q4_0_decode_packed_bytes(n, k))
    qll.qll_q4_0_decode_pack(w, wp, n, k)
    return wp


def packed_gemv(wp, xq, n, k):
    y = empty(n, torch.float32)
    qll.qll_q4_0_decode_packed_q8_0_gemv(wp, xq, y, n, k)
    return y


def unpack_layout(buf, n, k):
    """(codes [n][k], d_bits [n][k/32], scale-plane padding) read from the bytes."""
    nb = k // 32
    npad = -(-nb // 8) * 8
    rows = np.asarray(buf, np.uint8).reshape(n, 16 * nb + 2 * npad)
    qs = rows[:, :16 * nb].reshape(n, nb, 16)
    d = np.ascontiguousarray(rows[:, 16 * nb:]).view(np.uint16)
    # element e < 16: low nibble of byte e; e >= 16: high nibble of byte e - 16
    codes = np.concatenate([qs & 0x0F, qs >> 4], axis=2).reshape(n, k)
    return codes, d[:, :nb], d[:, nb:]


@pytest.mark.parametrize("n,k", [(1, 32), (3, 96), (5, 256), (7, 288), (17, 8224), (4, 4096)])
def test_layout_round_trip(qll_gpu, n, k):
    rng = np.random.default_rng(n * 31 + k)
    codes, d_bits = synth.q4_0_weights(rng, n, k)
    buf = host(decode_pack(pack_q4_0(codes, d_bits), n, k))
    assert buf.size == n * (16 * (k // 32) + 16 * -(-(k // 32) // 8))
    c2, d2, pad_d = unpack_layout(buf, n, k)
    assert np.array_equal(c2, codes)
    assert np.array_equal(d2, np.asarray(d_bits, np.uint16))
    assert np.all(pad_d == 0)


# one group, a partial group, several groups with a ragged last one, the
# lane counts 8 / 16 / 32 / 64 per row, the largest staged k
@pytest.mark.parametrize("n,k", [(300, 4096), (33, 14336), (7, 96), (129, 608), (64, 4160), (5, 32), (17, 8224),
                                 (3, 256), (70, 2048), (40, 49152), (1, 1024)])
def test_gemv(qll_gpu, n, k):
    rng = np.random.default_rng(n * 7 + k)
    codes, d_bits = synth.q4_0_weights(rng, n, k)
    x = synth.normal_f32(rng, (1, k))
    y = host(packed_gemv(decode_pack(pack_q4_0(codes, d_bits), n, k), quantize_q8_0(x), n, k))
    y_ref, mag = O.q4_0_q8_0(O.pack_q4_0(codes, d_bits), O.quantize_q8_0(x), 1, n, k)
    assert_within(y, y_ref[0], mag[0], TOL, f"decode-packed GEMV n={n} k={k}")


@pytest.mark.parametrize("n,k", [(40, 512), (9, 14336), (130, 4128)])
def test_unit_scales_bit_exact(qll_gpu, n, k):
    # dw = dx = 1: y is an integer below 2^24, exact in any summation order
    rng = np.random.default_rng(n + k)
    codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
    d_bits = np.full((n, k // 32), 0x3c00, np.uint16)
    x = rng.integers(-126, 127, (1, k)).astype(np.float32)
    x[:, ::32] = 127.0  # d = 1 in every activation block
    q = O.quantize_q8_0(x)
    raw = np.asarray(q, np.uint8).reshape(k // 32, 34)
    assert np.all(raw[:, :2].view(np.uint16) == 0x3c00)
    want = raw[:, 2:].view(np.int8).reshape(k).astype(np.int64) @ (codes.astype(np.int64) - 8).T
    y = host(packed_gemv(decode_pack(pack_q4_0(codes, d_bits), n, k), quantize_q8_0(x), n, k))
    assert np.array_equal(y.astype(np.float64), want.astype(np.float64))


@pytest.mark.parametrize("s", range(4))
def test_8b_shapes_every_output(qll_gpu, s):
    codes, d_bits, x = synth.q4_decode(s)
    n, k = codes.shape
    y = host(packed_gemv(decode_pack(pack_q4_0(codes, d_bits), n, k), quantize_q8_0(x), n, k))
    y_ref, mag = O.q4_0_q8_0(O.pack_q4_0(codes, d_bits), O.quantize_q8_0(x), 1, n, k)
    assert_within(y, y_ref[0], mag[0], TOL, f"decode-packed GEMV {synth.SHAPES_8B[s]}")
