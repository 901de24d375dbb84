"""Parity of the f32 GEMM and GEMV on the GPU against the f64 oracle:
|C - C_ref| <= 1e-5 * sum_p |a_ip * b_pj|, plus exact closed-form cases."""
import numpy as np
import pytest

import oracle as O
import synth
import torch

import quantized_linear_layer_amd as qll
from gpu_util import assert_within, dev, empty, host, sgemm

pytestmark = pytest.mark.gpu
TOL = 1e-5


def sgemm_core(a_t, b_t, m, n, k):
    """m > 1 with a workspace: the bf16 matrix core, both operands split into
    three exact bf16 parts (B transposed on the way)."""
    c = empty(m * n, torch.float32)
    ws = empty(max(16, qll.qll_workspace_bytes(qll.QLL_OP_SGEMM_BF16, m, n, k)))
    qll.qll_sgemm(a_t, b_t, c, m, n, k, ws=ws)
    return c


def _check(a, b, what, core=False):
    m, k = a.shape
    n = b.shape[1]
    c = host((sgemm_core if core else sgemm)(dev(a), dev(b), m, n, k)).reshape(m, n)
    c_ref, mag = O.sgemm(a, b)
    assert_within(c, c_ref, mag, TOL, what)
    return c


@pytest.mark.parametrize("m,n,k", [(1, 1, 1), (2, 3, 5), (7, 11, 13), (33, 17, 23), (48, 192, 128), (130, 257, 300),
                                   (128, 128, 16), (129, 130, 17), (256, 64, 1000), (1, 7, 3), (1, 4096, 33),
                                   (1, 300, 4096), (1, 1000, 1000), (256, 384, 48), (384, 128, 1024)])
def test_shapes(qll_gpu, m, n, k):
    rng = np.random.default_rng(m * 7919 + n * 31 + k)
    a = synth.uniform_f32(rng, (m, k))
    b = synth.uniform_f32(rng, (k, n))
    _check(a, b, f"sgemm {m}x{n}x{k}")


def test_exact_cases(qll_gpu):
    rng = np.random.default_rng(2)
    a = synth.uniform_f32(rng, (70, 96))
    c = _check(a, np.eye(96, dtype=np.float32), "identity")
    assert np.array_equal(c, a)
    ai = rng.integers(-2, 3, (150, 200)).astype(np.float32)
    bi = rng.integers(-2, 3, (200, 90)).astype(np.float32)
    c = _check(ai, bi, "small integers")
    assert np.array_equal(c.astype(np.int64), ai.astype(np.int64) @ bi.astype(np.int64))
    c = _check(np.ones((1, 777), np.float32), np.ones((777, 65), np.float32), "ones gemv")
    assert np.all(c == 777.0)


def test_gemv_config_full(qll_gpu):
    a, b, x = synth.f32_gemm()
    c = _check(x, b, "f32 GEMV 4096x4096")
    c2 = host(sgemm(dev(x), dev(b), 1, 4096, 4096)).reshape(1, 4096)
    assert np.array_equal(c.view(np.uint32), c2.view(np.uint32)), "GEMV not deterministic"


def test_gemm_config_full(qll_gpu):
    # the f32 GEMM 4096^3 on the f32 matrix core, every output
    import full_refs
    a, b, c_ref, mag = full_refs.sgemm_4096()
    m, k = a.shape
    n = b.shape[1]
    c = host(sgemm(dev(a), dev(b), m, n, k)).reshape(m, n)
    assert_within(c, c_ref, mag, TOL, "f32 GEMM 4096^3")

def test_gemm_row_matches_gemv(qll_gpu):
    rng = np.random.default_rng(5)
    a = synth.uniform_f32(rng, (40, 512))
    b = synth.uniform_f32(rng, (512, 300))
    c = _check(a, b, "gemm")
    for i in (0, 17, 39):
        ci = host(sgemm(dev(a[i:i + 1]), dev(b), 1, 300, 512))
        _, mag = O.sgemm(a[i:i + 1], b)
        assert np.all(np.abs(ci - c[i]) <= 2 * TOL * mag[0])


@pytest.mark.parametrize("m,n,k", [(2, 3, 16), (48, 192, 128), (128, 128, 16), (130, 257, 304), (256, 384, 48),
                                   (384, 128, 1024), (70, 33, 4096), (129, 65, 80)])
def test_bf16_core_shapes(qll_gpu, m, n, k):
    rng = np.random.default_rng(m * 7919 + n * 31 + k + 5)
    a = synth.uniform_f32(rng, (m, k))
    b = synth.uniform_f32(rng, (k, n))
    _check(a, b, f"sgemm on the bf16 core {m}x{n}x{k}", core=True)


def test_bf16_core_exact_cases(qll_gpu):
    # A . I = A: the three parts of every a add up to a exactly; small
    # integers are exact in the first part and give exact sums
    rng = np.random.default_rng(12)
    a = synth.uniform_f32(rng, (70, 96)) * np.float32(1e3)
    c = _check(a, np.eye(96, dtype=np.float32), "identity", core=True)
    assert np.array_equal(c, a)
    ai = rng.integers(-2, 3, (150, 208)).astype(np.float32)
    bi = rng.integers(-2, 3, (208, 90)).astype(np.float32)
    c = _check(ai, bi, "small integers", core=True)
    assert np.array_equal(c.astype(np.int64), ai.astype(np.int64) @ bi.astype(np.int64))


def test_bf16_core_config_full(qll_gpu):
    # the same GEMM on the bf16 matrix core (operands split into three exact
    # bf16 parts), every output
    import full_refs
    a, b, c_ref, mag = full_refs.sgemm_4096()
    m, k = a.shape
    n = b.shape[1]
    c = host(sgemm_core(dev(a), dev(b), m, n, k)).reshape(m, n)
    assert_within(c, c_ref, mag, TOL, "f32 GEMM 4096^3 on the bf16 core")
    torch.cuda.empty_cache()


@pytest.mark.parametrize("core", [False, True])
def test_gemm_same_sign_4096(qll_gpu, core):
    # operands all of one sign (U(0, 1)): every partial sum grows with p, so
    # a rounding that always goes the same way (toward zero) adds up instead
    # of cancelling; 4096^3 runs without a K split, so each output is one
    # accumulation chain of k = 4096.  Whole rows and columns are checked.
    rng = np.random.default_rng(2024)
    a = synth.uniform_f32(rng, (4096, 4096), 0.0, 1.0)
    b = synth.uniform_f32(rng, (4096, 4096), 0.0, 1.0)
    c = host((sgemm_core if core else sgemm)(dev(a), dev(b), 4096, 4096, 4096)).reshape(4096, 4096)
    rows = np.array([0, 1, 777, 2048, 4095])
    cols = np.array([0, 63, 1000, 4095])
    ii = np.concatenate([np.repeat(rows, 4096), np.tile(np.arange(4096), len(cols))])
    jj = np.concatenate([np.tile(np.arange(4096), len(rows)), np.repeat(cols, 4096)])
    c_ref, mag = O.sgemm_sampled(a, b, ii, jj)
    err = assert_within(c[ii, jj], c_ref, mag, TOL, f"same-sign 4096^3 ({'bf16' if core else 'f32'} core)")
    print(f"same-sign 4096^3, {'bf16' if core else 'f32'} core: max |err|/mag = {err:.3g}")
    torch.cuda.empty_cache()
