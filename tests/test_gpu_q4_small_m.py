"""Parity of the small-m decode kernels against the oracle: the Q4_0 x Q8_0
GEMM entry at 2 <= m <= 8 (weights loaded once for all rows) and the
quantize-fused entry (f32 activations quantized to Q8_0 inside the launch)
at 1 <= m <= 8, with and without its workspace.  Float outputs within
1e-4 * sum_b |term_b|; integer cases bit-exact.  The fused entry's
in-launch quantization is checked bit for bit through the results it must
reproduce: against the GEMM entry wherever both run the GEMV-style kernel
(m = 1, rows of fewer than eight blocks, m = 2 on tall matrices, m <= 4 on
very tall ones), and with
its workspace (quantize, then the GEMM entry's kernel) always."""
import numpy as np
import pytest
import torch

import oracle as O
import quantized_linear_layer_amd as qll
import synth
from gpu_util import assert_within, dev, empty, host, pack_q4_0, q4_gemm, quantize_q8_0

pytestmark = pytest.mark.gpu
TOL = 1e-4

# (n, k): one k-chunk, several chunks with a ragged last one, odd block
# counts (one block per unit instead of pairs), a single block
SHAPES = [(300, 4096), (33, 14336), (7, 96), (129, 608), (64, 4160), (5, 32), (17, 8224)]


def gemv_f32(w, x, m, n, k, route="single"):
    """The fused entry without a workspace ("single": one launch quantizing
    in every workgroup) or with one of the size it asks for ("ws": quantize
    once, then the Q8_0 decode kernel; the single launch where it asks for
    none)."""
    y = empty(m * n, torch.float32)
    ws = None
    if route == "ws":
        need = qll.qll_workspace_bytes(qll.QLL_OP_Q4_0_GEMV_F32, m, n, k)
        ws = empty(need) if need else None
    qll.qll_q4_0_q8_0_gemv_f32(w, dev(np.asarray(x, np.float32)), y, m, n, k, ws=ws)
    return y


def _case(seed, m, n, k):
    rng = np.random.default_rng(seed)
    codes, d_bits = synth.q4_0_weights(rng, n, k)
    x = synth.normal_f32(rng, (m, k))
    return codes, d_bits, x


def _gemv_style(m, n, k):
    # shapes on which the GEMM entry runs the GEMV-style kernel, as the
    # fused entry's single launch does (elsewhere it runs the int8
    # matrix-core kernel, whose f32 sums are added in another order)
    return m == 1 or k < 256 or (m == 2 and n >= 8192) or (m <= 4 and n >= 32768)


def _ref(codes, d_bits, x):
    n, k = codes.shape
    return O.q4_0_q8_0(O.pack_q4_0(codes, d_bits), O.quantize_q8_0(x), x.shape[0], n, k)


@pytest.mark.parametrize("m", [2, 3, 5, 8])
@pytest.mark.parametrize("n,k", SHAPES)
def test_small_m_gemm(qll_gpu, m, n, k):
    codes, d_bits, x = _case(m * 977 + n * 13 + k, m, n, k)
    y = host(q4_gemm(pack_q4_0(codes, d_bits), quantize_q8_0(x), m, n, k)).reshape(m, n)
    y_ref, mag = _ref(codes, d_bits, x)
    assert_within(y, y_ref, mag, TOL, f"small-m GEMM m={m} n={n} k={k}")


@pytest.mark.parametrize("route", ["single", "ws"])
@pytest.mark.parametrize("m", [1, 2, 4, 7, 8])
@pytest.mark.parametrize("n,k", SHAPES)
def test_fused_f32_gemv(qll_gpu, m, n, k, route):
    codes, d_bits, x = _case(m * 577 + n * 11 + k, m, n, k)
    w = pack_q4_0(codes, d_bits)
    y = host(gemv_f32(w, x, m, n, k, route)).reshape(m, n)
    y_ref, mag = _ref(codes, d_bits, x)
    assert_within(y, y_ref, mag, TOL, f"fused GEMV m={m} n={n} k={k}")
    # the same dot on Q8_0 input from qll_quantize_q8_0: identical arithmetic
    # after the staging, so any difference in the in-launch quantization
    # shows up as a bit difference
    if route == "ws" or _gemv_style(m, n, k):
        y2 = host(q4_gemm(w, quantize_q8_0(x), m, n, k)).reshape(m, n)
        assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))


@pytest.mark.parametrize("route", ["single", "ws"])
@pytest.mark.parametrize("n,k", [(5, 49152), (7, 49184), (3, 65536)])
def test_fused_f32_gemv_long_rows(qll_gpu, n, k, route):
    # m = 1 stages the whole row in LDS up to k = 49152 and by chunks beyond
    # (with a workspace: the GEMV up to 49152, the small-m kernel beyond)
    codes, d_bits, x = _case(n * 13 + k, 1, n, k)
    w = pack_q4_0(codes, d_bits)
    y = host(gemv_f32(w, x, 1, n, k, route)).reshape(1, n)
    y_ref, mag = _ref(codes, d_bits, x)
    assert_within(y, y_ref, mag, TOL, f"fused GEMV m=1 n={n} k={k} {route}")
    y2 = host(gemv_f32(w, x, 1, n, k, "single" if route == "ws" else "ws")).reshape(1, n)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))


def test_fused_workspace_short_or_absent(qll_gpu):
    # a workspace one byte short, or none, selects the single launch (the
    # same bits either way); a whole one quantizes first and runs the GEMM
    # entry's kernel (the same bits as quantize + GEMM)
    op = qll.QLL_OP_Q4_0_GEMV_F32
    m, n, k = 3, 70, 8192
    codes, d_bits, x = _case(4242, m, n, k)
    w = pack_q4_0(codes, d_bits)
    need = qll.qll_workspace_bytes(op, m, n, k)
    assert need >= m * (k // 32) * 34
    outs = []
    for ws in (None, empty(need - 1), empty(need)):
        y = empty(m * n, torch.float32)
        qll.qll_q4_0_q8_0_gemv_f32(w, dev(x), y, m, n, k, ws=ws)
        outs.append(host(y))
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    y2 = host(q4_gemm(w, quantize_q8_0(x), m, n, k))
    assert np.array_equal(outs[2].view(np.uint32), y2.view(np.uint32))
    y_ref, mag = _ref(codes, d_bits, x)
    for y in outs:
        assert_within(y.reshape(m, n), y_ref, mag, TOL, "fused GEMV, workspace short, absent or whole")


# n >= 32768 takes the 4-rows-per-lane-group layout: odd block counts (one
# block per unit), a ragged last row group, several k-chunks
@pytest.mark.parametrize("m", [1, 2, 5, 8])
@pytest.mark.parametrize("n,k", [(32771, 96), (40001, 4160), (32768, 1056)])
def test_large_n_layout(qll_gpu, m, n, k):
    codes, d_bits, x = _case(m * 31 + n + k, m, n, k)
    w = pack_q4_0(codes, d_bits)
    y = host(gemv_f32(w, x, m, n, k)).reshape(m, n)
    y_ref, mag = _ref(codes, d_bits, x)
    assert_within(y, y_ref, mag, TOL, f"fused large-n m={m} n={n} k={k}")
    y2 = host(q4_gemm(w, quantize_q8_0(x), m, n, k)).reshape(m, n)
    assert_within(y2, y_ref, mag, TOL, f"GEMM large-n m={m} n={n} k={k}")
    if _gemv_style(m, n, k):
        assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))


# 8192 <= n < 32768 at m > 2 takes the 2-rows-per-lane-group layout (rows of
# fewer than eight blocks, where the GEMM entry runs the GEMV-style kernel):
# odd block counts, a ragged last row group
@pytest.mark.parametrize("m", [3, 4, 8])
@pytest.mark.parametrize("n,k", [(8193, 96), (14337, 224), (9000, 160)])
def test_mid_n_layout(qll_gpu, m, n, k):
    codes, d_bits, x = _case(m * 17 + n + k, m, n, k)
    w = pack_q4_0(codes, d_bits)
    y = host(q4_gemm(w, quantize_q8_0(x), m, n, k)).reshape(m, n)
    y_ref, mag = _ref(codes, d_bits, x)
    assert_within(y, y_ref, mag, TOL, f"small-m mid-n m={m} n={n} k={k}")
    y2 = host(gemv_f32(w, x, m, n, k)).reshape(m, n)  # the fused entry's single launch (its own layout)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))


def _unit_scale_x(rng, m, k):
    # a +-127 in every block (d = 1 exactly), integers and exact ties elsewhere
    x = rng.integers(-126, 127, (m, k)).astype(np.float32)
    ties = rng.random((m, k)) < 0.25
    x[ties] += np.float32(0.5)  # ... .5 values round away from zero
    x[:, ::32] = np.where(rng.random((m, k // 32)) < 0.5, 127.0, -127.0)
    return x


@pytest.mark.parametrize("m,n,k", [(1, 40, 512), (3, 17, 96), (8, 9, 14336), (5, 33, 4128)])
def test_unit_scales_bit_exact(qll_gpu, m, n, k):
    # dw = dx = 1: y is an integer below 2^24, exact in any summation order;
    # the codes come from the oracle's quantizer (ties away from zero)
    rng = np.random.default_rng(m + n + k)
    codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
    d_bits = np.full((n, k // 32), 0x3c00, np.uint16)
    x = _unit_scale_x(rng, m, k)
    want = _int_reference(O.quantize_q8_0(x), codes, m, n, k)
    w = pack_q4_0(codes, d_bits)
    y_fused = host(gemv_f32(w, x, m, n, k)).reshape(m, n)
    assert np.array_equal(y_fused.astype(np.float64), want.astype(np.float64))
    if m >= 2:
        y = host(q4_gemm(w, quantize_q8_0(x), m, n, k)).reshape(m, n)
        assert np.array_equal(y.astype(np.float64), want.astype(np.float64))


def _int_reference(q, codes, m, n, k):
    # integer codes of the oracle's Q8_0 blocks (34 bytes: fp16 d, 32 int8)
    raw = np.asarray(q, np.uint8).reshape(m, k // 32, 34)
    assert np.all(raw[:, :, :2].view(np.uint16) == 0x3c00)  # d = 1 in every block
    qx = raw[:, :, 2:].view(np.int8).reshape(m, k).astype(np.int64)
    return qx @ (codes.astype(np.int64) - 8).T


def test_fused_zero_rows(qll_gpu):
    rng = np.random.default_rng(21)
    m, n, k = 4, 50, 1024
    codes, d_bits = synth.q4_0_weights(rng, n, k)
    x = synth.normal_f32(rng, (m, k))
    x[1] = 0.0
    x[3, 64:96] = 0.0  # one all-zero block: d = 0, codes 0
    w = pack_q4_0(codes, d_bits)
    y = host(gemv_f32(w, x, m, n, k)).reshape(m, n)
    assert np.all(y[1] == 0)
    y_ref, mag = _ref(codes, d_bits, x)
    assert_within(y, y_ref, mag, TOL, "fused with zero rows")


@pytest.mark.parametrize("s", range(4))
def test_8b_shapes_fused_m1_and_m8(qll_gpu, s):
    # full decode sizes: the fused entry at m = 1 (both routes) against the
    # oracle on every output; at m = 8 the small-m GEMM and the fused entry's
    # single launch on a sample of outputs, and its workspace route
    # (quantize, then the same kernel) bit for bit against the GEMM
    codes, d_bits, x1 = synth.q4_decode(s)
    n, k = codes.shape
    w = pack_q4_0(codes, d_bits)
    wq = O.pack_q4_0(codes, d_bits)
    y = host(gemv_f32(w, x1, 1, n, k))
    y_ref, mag = O.q4_0_q8_0(wq, O.quantize_q8_0(x1), 1, n, k)
    assert_within(y, y_ref[0], mag[0], TOL, f"fused m=1 {synth.SHAPES_8B[s]}")
    assert np.array_equal(y.view(np.uint32), host(gemv_f32(w, x1, 1, n, k, "ws")).view(np.uint32))
    x8 = synth.q4_prefill_x(s)[:8]
    y8 = host(q4_gemm(w, quantize_q8_0(x8), 8, n, k)).reshape(8, n)
    yws = host(gemv_f32(w, x8, 8, n, k, "ws")).reshape(8, n)
    assert np.array_equal(yws.view(np.uint32), y8.view(np.uint32))
    ysingle = host(gemv_f32(w, x8, 8, n, k, "single")).reshape(8, n)
    rng = np.random.default_rng(300 + s)
    ii = np.concatenate([[0, 7], rng.integers(0, 8, 2000)])
    jj = np.concatenate([[0, n - 1], rng.integers(0, n, 2000)])
    y_ref, mag = O.q4_0_q8_0_sampled(wq, O.quantize_q8_0(x8), 8, n, k, ii, jj)
    assert_within(y8[ii, jj], y_ref, mag, TOL, f"small-m m=8 {synth.SHAPES_8B[s]}")
    assert_within(ysingle[ii, jj], y_ref, mag, TOL, f"fused single launch m=8 {synth.SHAPES_8B[s]}")
