"""Parity of the repacked-weight Q4_0 x Q8_0 prefill path.

The load-time repack (qll_q4_0_repack) is checked byte for byte by decoding
its output in numpy from the e3m2 definition (sign bit, 3-bit exponent with
bias 3, 2-bit mantissa; subnormals at exponent 0) and comparing with the raw
codes and scales.  The GEMM on repacked weights is checked against the oracle
(1e-4 * sum_b |term_b|), bit-exactly on unit scales, and bit for bit against
the direct-layout GEMM: both form the exact block sums and the exact scale
products and add them in the same block and split order, so their outputs
must be identical."""
import numpy as np
import pytest
import torch

import oracle as O
import quantized_linear_layer_amd as qll
import synth
from gpu_util import assert_within, dev, empty, host, pack_q4_0, q4_gemm, quantize_q8_0

pytestmark = pytest.mark.gpu
TOL = 1e-4


def e3m2_value(code):
    code = np.asarray(code, np.int64)
    s = (code >> 5) & 1
    e = (code >> 2) & 7
    mant = code & 3
    mag = np.where(e == 0, mant / 4.0 * 2.0 ** -2, (1.0 + mant / 4.0) * 2.0 ** (e - 3.0))
    return np.where(s == 1, -mag, mag)


def unpack_repacked(wp, n, k):
    """Decoded weights [nt*128][k] and scale bits [nt*128][k/32] of a repacked buffer."""
    nb, nt = k // 32, (n + 127) // 128
    raw = np.asarray(wp, np.uint8)
    codes = raw[:nt * nb * 3072].reshape(nt, nb, 3072)
    p0 = codes[:, :, :2048].reshape(nt, nb, 128, 16)
    p1 = codes[:, :, 2048:].reshape(nt, nb, 128, 8)
    six = np.concatenate([p0, p1], axis=3)                      # [nt][nb][128][24] bytes
    bits = np.unpackbits(six, axis=3, bitorder="little")        # [.., 192], bit i of the 192-bit row
    fields = bits.reshape(nt, nb, 128, 32, 6)
    code = (fields * (1 << np.arange(6))).sum(axis=4)          # element e at bits 6e..6e+5
    vals = e3m2_value(code)                                     # [nt][nb][128][32]
    w = vals.transpose(0, 2, 1, 3).reshape(nt * 128, nb * 32)
    d = raw[nt * nb * 3072:].view(np.uint16).reshape(nt, nb, 128).transpose(0, 2, 1).reshape(nt * 128, nb)
    return w, d


def repack(w, n, k):
    wp = empty(qll.qll_q4_0_repacked_bytes(n, k))
    qll.qll_q4_0_repack(w, wp, n, k)
    return wp


def packed_gemm(wp, xq, m, n, k):
    y = empty(m * n, torch.float32)
    ws = empty(qll.qll_workspace_bytes(qll.QLL_OP_Q4_0_REPACKED_GEMM, m, n, k))
    qll.qll_q4_0_repacked_q8_0_gemm(wp, xq, y, m, n, k, ws=ws)
    return y


def _case(seed, m, n, k):
    rng = np.random.default_rng(seed)
    codes, d_bits = synth.q4_0_weights(rng, n, k)
    return codes, d_bits, synth.normal_f32(rng, (m, k))


@pytest.mark.parametrize("n,k", [(1, 32), (5, 96), (128, 64), (129, 320), (300, 4096), (17, 14336)])
def test_repack_decodes_to_codes(qll_gpu, n, k):
    rng = np.random.default_rng(n + k)
    codes, d_bits = synth.q4_0_weights(rng, n, k)
    wp = host(repack(pack_q4_0(codes, d_bits), n, k))
    assert wp.size == qll.qll_q4_0_repacked_bytes(n, k) == ((n + 127) // 128) * (k // 32) * 3328
    w, d = unpack_repacked(wp, n, k)
    assert np.array_equal(w[:n], codes.astype(np.float64) - 8.0)
    assert np.array_equal(d[:n], np.asarray(d_bits, np.uint16))
    assert np.all(w[n:] == 0) and np.all(d[n:] == 0)


# ragged rows and columns, odd block counts, one-block and split-k shapes
# (64 x 33 x 14336 splits k; 128 x 256 x 3232 leaves one real block in the
# last split), m = 1 and small m (the repacked GEMM serves every m)
@pytest.mark.parametrize("m,n,k", [(1, 7, 32), (2, 1, 32), (3, 7, 96), (8, 40, 256), (17, 64, 512), (130, 129, 320),
                                   (128, 128, 4096), (200, 300, 64), (64, 33, 14336), (128, 256, 3232),
                                   (257, 131, 608), (65, 33, 14336)])
def test_repacked_gemm_shapes(qll_gpu, m, n, k):
    codes, d_bits, x = _case(m * 1000 + n + k, m, n, k)
    w = pack_q4_0(codes, d_bits)
    xq = quantize_q8_0(x)
    y = host(packed_gemm(repack(w, n, k), xq, m, n, k)).reshape(m, n)
    y_ref, mag = O.q4_0_q8_0(O.pack_q4_0(codes, d_bits), O.quantize_q8_0(x), m, n, k)
    assert_within(y, y_ref, mag, TOL, f"repacked GEMM m={m} n={n} k={k}")
    if qll.qll_workspace_bytes(qll.QLL_OP_Q4_0_Q8_0_GEMM, m, n, k) > 0:
        # the direct-layout GEMM kernel: same exact sums, same order (the
        # small-m kernels that run below m = 65 add the blocks in their own)
        y_direct = host(q4_gemm(w, xq, m, n, k)).reshape(m, n)
        assert np.array_equal(y.view(np.uint32), y_direct.view(np.uint32))


def _unit_scale_x(rng, m, k):
    # a +-127 in every block (d = 1 exactly), integers and exact ties elsewhere
    x = rng.integers(-126, 127, (m, k)).astype(np.float32)
    x[rng.random((m, k)) < 0.25] += np.float32(0.5)
    x[:, ::32] = np.where(rng.random((m, k // 32)) < 0.5, 127.0, -127.0)
    return x


@pytest.mark.parametrize("m,n,k", [(70, 150, 1024), (129, 33, 4096), (3, 9, 96)])
def test_repacked_unit_scales_bit_exact(qll_gpu, m, n, k):
    # d_w = d_x = 1: every output is an integer below 2^24, exact in any order;
    # the activation codes span the full [-127, 127] range of the h/l split
    rng = np.random.default_rng(m + n + k)
    codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
    d_bits = np.full((n, k // 32), 0x3c00, np.uint16)
    x = _unit_scale_x(rng, m, k)
    q = np.asarray(O.quantize_q8_0(x), np.uint8).reshape(m, k // 32, 34)
    assert np.all(q[:, :, :2].view(np.uint16) == 0x3c00)
    qx = q[:, :, 2:].view(np.int8).reshape(m, k).astype(np.int64)
    assert qx.min() == -127 and qx.max() == 127
    want = qx @ (codes.astype(np.int64) - 8).T
    y = host(packed_gemm(repack(pack_q4_0(codes, d_bits), n, k), quantize_q8_0(x), m, n, k)).reshape(m, n)
    assert np.array_equal(y.astype(np.float64), want.astype(np.float64))


def test_repacked_one_hot(qll_gpu):
    # a single nonzero activation per row picks one weight element: checks the
    # element order inside the 6-bit planes and the block indexing
    m, n, k = 32, 20, 320
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
    d_bits = np.full((n, k // 32), 0x3c00, np.uint16)
    x = np.zeros((m, k), np.float32)
    pos = rng.integers(0, k, m)
    x[np.arange(m), pos] = 127.0
    y = host(packed_gemm(repack(pack_q4_0(codes, d_bits), n, k), quantize_q8_0(x), m, n, k)).reshape(m, n)
    want = 127.0 * (codes[:, pos].T.astype(np.float64) - 8.0)
    assert np.array_equal(y.astype(np.float64), want)


@pytest.mark.parametrize("s", range(4))
def test_repacked_prefill_8b_shapes(qll_gpu, s):
    # full prefill size (m = 512): every output against the oracle, and
    # bit-equal to the direct-layout GEMM
    import full_refs
    codes, d_bits, x, y_ref, mag = full_refs.q4_prefill(s)
    n, k = codes.shape
    m = x.shape[0]
    w = pack_q4_0(codes, d_bits)
    xq = quantize_q8_0(x)
    wp = repack(w, n, k)
    y = host(packed_gemm(wp, xq, m, n, k)).reshape(m, n)
    assert_within(y, y_ref, mag, TOL, f"repacked prefill {synth.SHAPES_8B[s]}")
    y_direct = host(q4_gemm(w, xq, m, n, k)).reshape(m, n)
    assert np.array_equal(y.view(np.uint32), y_direct.view(np.uint32))
    del w, xq, wp
    torch.cuda.empty_cache()
