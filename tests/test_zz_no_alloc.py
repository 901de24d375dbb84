"""The allocation-free Q4_0 x Q8_0 GEMM entry (static device scratch) against
the workspace entry on the same inputs: the same kernels, so every output
must be bit-equal, and within 1e-4 * sum_b |term_b| of the oracle.  Two
calls in a row, the second on a smaller input (the scratch keeps the first
call's contents), then the small-m and the too-large cases."""
import numpy as np
import pytest
import torch

import oracle as O
import quantized_linear_layer_amd as qll
import synth
from gpu_util import assert_within, empty, host, pack_q4_0, q4_gemm, quantize_q8_0

pytestmark = pytest.mark.gpu
TOL = 1e-4


def _noalloc(w, xq, m, n, k):
    y = empty(m * n, torch.float32)
    qll.qll_q4_0_q8_0_gemm_noalloc(w, xq, y, m, n, k)
    return y


def _case(seed, m, n, k):
    rng = np.random.default_rng(seed)
    codes, d_bits = synth.q4_0_weights(rng, n, k)
    x = synth.normal_f32(rng, (m, k))
    return codes, d_bits, x


def _check(codes, d_bits, x, what):
    n, k = codes.shape
    m = x.shape[0]
    w = pack_q4_0(codes, d_bits)
    xq = quantize_q8_0(x)
    y = host(_noalloc(w, xq, m, n, k)).reshape(m, n)
    y_ws = host(q4_gemm(w, xq, m, n, k)).reshape(m, n)
    assert np.array_equal(y.view(np.uint32), y_ws.view(np.uint32)), f"{what}: differs from the workspace entry"
    y_ref, mag = O.q4_0_q8_0(O.pack_q4_0(codes, d_bits), O.quantize_q8_0(x), m, n, k)
    assert_within(y, y_ref, mag, TOL, what)


def test_two_calls_second_smaller(qll_gpu):
    # 512 x 4096 x 4096 splits k four ways (partials and prepared activations
    # fill most of the scratch); the second call's shapes are smaller and
    # ragged, so stale bytes from the first would show
    print("noalloc: 512x4096x4096 then 130x300x1056", flush=True)
    _check(*_case(1, 512, 4096, 4096), "noalloc 512x4096x4096")
    _check(*_case(2, 130, 300, 1056), "noalloc 130x300x1056 after a larger call")


def test_32_row_tiles_and_small_m(qll_gpu):
    print("noalloc: 20x257x4096, then m = 5 (no scratch)", flush=True)
    _check(*_case(3, 20, 257, 4096), "noalloc 20x257x4096")
    _check(*_case(4, 5, 64, 512), "noalloc m=5")


def test_8b_prefill_shape(qll_gpu):
    # the (14336 -> 4096) prefill layer, whose workspace is the largest of
    # the 8B-class shapes, every output against the oracle's full result
    import full_refs
    print("noalloc: 512x4096x14336", flush=True)
    codes, d_bits, x, y_ref, mag = full_refs.q4_prefill(1)
    n, k = codes.shape
    assert qll.qll_workspace_bytes(qll.QLL_OP_Q4_0_Q8_0_GEMM, 512, n, k) <= qll.QLL_NOALLOC_SCRATCH_BYTES
    w = pack_q4_0(codes, d_bits)
    xq = quantize_q8_0(x)
    y = host(_noalloc(w, xq, 512, n, k)).reshape(512, n)
    assert_within(y, y_ref, mag, TOL, "noalloc 512x4096x14336")
    assert np.array_equal(y.view(np.uint32), host(q4_gemm(w, xq, 512, n, k)).reshape(512, n).view(np.uint32))


def test_shape_beyond_the_scratch_is_refused(qll_gpu):
    m, n, k = 4096, 64, 14336
    assert qll.qll_workspace_bytes(qll.QLL_OP_Q4_0_Q8_0_GEMM, m, n, k) > qll.QLL_NOALLOC_SCRATCH_BYTES
    w = empty(n * (k // 32) * 18)
    xq = empty(m * (k // 32) * 34)
    y = empty(m * n, torch.float32)
    with pytest.raises(qll.QllError) as e:
        qll.qll_q4_0_q8_0_gemm_noalloc(w, xq, y, m, n, k)
    assert e.value.status == -7
