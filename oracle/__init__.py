"""The CPU oracle of the quantized linear layer (ctypes wrapper over oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
bench's cpu_baseline leg, never by the product path.  It shares no code with
the HIP library.  Every function here only marshals numpy arrays; the
arithmetic is in oracle.c, where each routine cites the passage it follows:

* llama.cpp visual guide lesson 31 "CPU backend", "How the quantized dot
  product works" -- the Q4_0 x Q8_0 block dot and the block_q8_0 layout;
* Fucina course "Chapter 06 -- Going fast on CPUs", 6.4 -- the f32 GEMM
  referee, here accumulated in f64; 6.6 and "reduced precision" -- the
  transposed-B (NT) orientation with f32, bf16 or f16 weights widened exactly;
* Loom "Plan 9 SIMD Forward", "BitNet ternary MAD kernel" -- packed ternary
  weights, the ternary identity, per-row int8 activations;
* Fucina reference "Backends", 9.7 -- per-call Q8_0 activation quantization
  and Q8_0-quantized weights (the Q8_0 x Q8_0 block dot).

Every function is pinned by tests/test_oracle_*.py to something other than
itself (numpy brute force, closed forms, identities, exhaustive fp16).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB) or os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC):
            _build.build()
        _lib = load(_build.LIB)
    return _lib


_P = ctypes.c_void_p
_I = ctypes.c_int64


def load(path):
    """Load an oracle shared library and declare its signatures."""
    L = ctypes.CDLL(path)
    sig = {
        "orc_half_to_double_array": [_P, _P, _I],
        "orc_float_to_half_array": [_P, _P, _I],
        "orc_pack_q4_0": [_P, _P, _P, _I, _I],
        "orc_unpack_q4_0": [_P, _P, _P, _I, _I],
        "orc_quantize_q8_0": [_P, _P, _I, _I],
        "orc_unpack_q8_0": [_P, _P, _P, _I, _I],
        "orc_q4_0_q8_0": [_P, _P, _I, _I, _I, _P, _P],
        "orc_q4_0_q8_0_sampled": [_P, _P, _I, _I, _I, _P, _P, _I, _P, _P],
        "orc_q4_0_q8_0_block_sums": [_P, _P, _I, _I, _I, _P],
        "orc_pack_q8_0": [_P, _P, _P, _I, _I],
        "orc_q8_0_q8_0": [_P, _P, _I, _I, _I, _P, _P],
        "orc_q8_0_q8_0_sampled": [_P, _P, _I, _I, _I, _P, _P, _I, _P, _P],
        "orc_q8_0_q8_0_block_sums": [_P, _P, _I, _I, _I, _P],
        "orc_sgemm": [_P, _P, _I, _I, _I, _P, _P],
        "orc_sgemm_sampled": [_P, _P, _I, _I, _I, _P, _P, _I, _P, _P],
        "orc_gemm_nt": [_P, _P, ctypes.c_int, _I, _I, _I, _P, _P],
        "orc_gemm_nt_sampled": [_P, _P, ctypes.c_int, _I, _I, _I, _P, _P, _I, _P, _P],
        "orc_pack_ternary": [_P, _P, _I, _I],
        "orc_unpack_ternary": [_P, _P, _I, _I],
        "orc_quantize_i8_rows": [_P, _P, _P, _P, _I, _I],
        "orc_ternary": [_P, ctypes.c_float, _P, _P, _P, _I, _I, _I, _P, _P, _P],
        "orc_ternary_sampled": [_P, ctypes.c_float, _P, _P, _P, _I, _I, _I, _P, _P, _I, _P, _P],
        "orc_num_threads": [],
        "orc_set_num_threads": [ctypes.c_int],
    }
    for name, args in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    return L


class OracleError(RuntimeError):
    pass


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc, what):
    if rc != 0:
        raise OracleError(f"{what} failed with status {rc}")


def num_threads(L=None):
    return (L or lib()).orc_num_threads()


def set_num_threads(count, L=None):
    """Threads for the oracle's later calls (results are the same for any)."""
    L = L or lib()
    L.orc_set_num_threads.restype = None
    L.orc_set_num_threads(int(count))


# --------------------------------------------------------------------------- fp16

def half_to_double(bits, L=None):
    bits = _c(bits, np.uint16)
    out = np.empty(bits.shape, np.float64)
    (L or lib()).orc_half_to_double_array(_ptr(bits), _ptr(out), bits.size)
    return out


def float_to_half(x, L=None):
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    (L or lib()).orc_float_to_half_array(_ptr(x), _ptr(out), x.size)
    return out


# --------------------------------------------------------------------------- Q4_0 / Q8_0

def pack_q4_0(codes, d_bits, L=None):
    """codes uint8[n][k] (0..15), d_bits uint16[n][k/32] -> uint8[n][k/32*18]."""
    codes = _c(codes, np.uint8)
    d_bits = _c(d_bits, np.uint16)
    n, k = codes.shape
    w = np.empty((n, k // 32 * 18), np.uint8)
    _check((L or lib()).orc_pack_q4_0(_ptr(codes), _ptr(d_bits), _ptr(w), n, k), "pack_q4_0")
    return w


def unpack_q4_0(w, n, k, L=None):
    w = _c(w, np.uint8)
    codes = np.empty((n, k), np.uint8)
    d_bits = np.empty((n, k // 32), np.uint16)
    _check((L or lib()).orc_unpack_q4_0(_ptr(w), _ptr(codes), _ptr(d_bits), n, k), "unpack_q4_0")
    return codes, d_bits


def quantize_q8_0(x, L=None):
    """x float32[m][k] -> uint8[m][k/32*34] Q8_0 blocks."""
    x = _c(x, np.float32)
    if x.ndim == 1:
        x = x[None, :]
    m, k = x.shape
    xq = np.empty((m, k // 32 * 34), np.uint8)
    _check((L or lib()).orc_quantize_q8_0(_ptr(x), _ptr(xq), m, k), "quantize_q8_0")
    return xq


def unpack_q8_0(xq, m, k, L=None):
    xq = _c(xq, np.uint8)
    q = np.empty((m, k), np.int8)
    d_bits = np.empty((m, k // 32), np.uint16)
    _check((L or lib()).orc_unpack_q8_0(_ptr(xq), _ptr(q), _ptr(d_bits), m, k), "unpack_q8_0")
    return q, d_bits


def q4_0_q8_0(w, xq, m, n, k, L=None):
    """Y = X.W^T in f64, and mag = sum_b |term_b|, both float64[m][n]."""
    w = _c(w, np.uint8)
    xq = _c(xq, np.uint8)
    y = np.empty((m, n), np.float64)
    mag = np.empty((m, n), np.float64)
    _check((L or lib()).orc_q4_0_q8_0(_ptr(w), _ptr(xq), m, n, k, _ptr(y), _ptr(mag)), "q4_0_q8_0")
    return y, mag


def q4_0_q8_0_sampled(w, xq, m, n, k, ii, jj, L=None):
    w = _c(w, np.uint8)
    xq = _c(xq, np.uint8)
    ii = _c(ii, np.int64)
    jj = _c(jj, np.int64)
    y = np.empty(ii.size, np.float64)
    mag = np.empty(ii.size, np.float64)
    _check((L or lib()).orc_q4_0_q8_0_sampled(_ptr(w), _ptr(xq), m, n, k, _ptr(ii), _ptr(jj), ii.size,
                                              _ptr(y), _ptr(mag)), "q4_0_q8_0_sampled")
    return y, mag


def q4_0_q8_0_block_sums(w, xq, m, n, k, L=None):
    w = _c(w, np.uint8)
    xq = _c(xq, np.uint8)
    s = np.empty((m, n, k // 32), np.int32)
    _check((L or lib()).orc_q4_0_q8_0_block_sums(_ptr(w), _ptr(xq), m, n, k, _ptr(s)), "block_sums")
    return s


# --------------------------------------------------------------------------- Q8_0 weights

def pack_q8_0(q, d_bits, L=None):
    """q int8[n][k], d_bits uint16[n][k/32] -> uint8[n][k/32*34] Q8_0 blocks."""
    q = _c(q, np.int8)
    d_bits = _c(d_bits, np.uint16)
    n, k = q.shape
    w = np.empty((n, k // 32 * 34), np.uint8)
    _check((L or lib()).orc_pack_q8_0(_ptr(q), _ptr(d_bits), _ptr(w), n, k), "pack_q8_0")
    return w


def q8_0_q8_0(w, xq, m, n, k, L=None):
    """Y = X.W^T with Q8_0 weights and activations: f64 outputs and mag = sum_b |term_b|."""
    w = _c(w, np.uint8)
    xq = _c(xq, np.uint8)
    y = np.empty((m, n), np.float64)
    mag = np.empty((m, n), np.float64)
    _check((L or lib()).orc_q8_0_q8_0(_ptr(w), _ptr(xq), m, n, k, _ptr(y), _ptr(mag)), "q8_0_q8_0")
    return y, mag


def q8_0_q8_0_sampled(w, xq, m, n, k, ii, jj, L=None):
    w = _c(w, np.uint8)
    xq = _c(xq, np.uint8)
    ii = _c(ii, np.int64)
    jj = _c(jj, np.int64)
    y = np.empty(ii.size, np.float64)
    mag = np.empty(ii.size, np.float64)
    _check((L or lib()).orc_q8_0_q8_0_sampled(_ptr(w), _ptr(xq), m, n, k, _ptr(ii), _ptr(jj), ii.size,
                                              _ptr(y), _ptr(mag)), "q8_0_q8_0_sampled")
    return y, mag


def q8_0_q8_0_block_sums(w, xq, m, n, k, L=None):
    w = _c(w, np.uint8)
    xq = _c(xq, np.uint8)
    s = np.empty((m, n, k // 32), np.int32)
    _check((L or lib()).orc_q8_0_q8_0_block_sums(_ptr(w), _ptr(xq), m, n, k, _ptr(s)), "q8 block_sums")
    return s


# --------------------------------------------------------------------------- f32

def sgemm(a, b, L=None):
    a = _c(a, np.float32)
    b = _c(b, np.float32)
    m, k = a.shape
    k2, n = b.shape
    assert k == k2
    c = np.empty((m, n), np.float64)
    mag = np.empty((m, n), np.float64)
    _check((L or lib()).orc_sgemm(_ptr(a), _ptr(b), m, n, k, _ptr(c), _ptr(mag)), "sgemm")
    return c, mag


def sgemm_sampled(a, b, ii, jj, L=None):
    a = _c(a, np.float32)
    b = _c(b, np.float32)
    m, k = a.shape
    n = b.shape[1]
    ii = _c(ii, np.int64)
    jj = _c(jj, np.int64)
    c = np.empty(ii.size, np.float64)
    mag = np.empty(ii.size, np.float64)
    _check((L or lib()).orc_sgemm_sampled(_ptr(a), _ptr(b), m, n, k, _ptr(ii), _ptr(jj), ii.size,
                                          _ptr(c), _ptr(mag)), "sgemm_sampled")
    return c, mag


# --------------------------------------------------------------------------- NT (W stored [n][k])

W_DTYPES = {"f32": (0, np.float32), "bf16": (1, np.uint16), "f16": (2, np.uint16)}


def gemm_nt(a, w, wdtype, L=None):
    """C = A.W^T with W [n][k] of dtype 'f32' (float32), 'bf16' or 'f16' (uint16
    bit patterns); f64 C and mag = sum_p |a*w|."""
    code, npdt = W_DTYPES[wdtype]
    a = _c(a, np.float32)
    w = _c(w, npdt)
    m, k = a.shape
    n, k2 = w.shape
    assert k == k2
    c = np.empty((m, n), np.float64)
    mag = np.empty((m, n), np.float64)
    _check((L or lib()).orc_gemm_nt(_ptr(a), _ptr(w), code, m, n, k, _ptr(c), _ptr(mag)), "gemm_nt")
    return c, mag


def gemm_nt_sampled(a, w, wdtype, ii, jj, L=None):
    code, npdt = W_DTYPES[wdtype]
    a = _c(a, np.float32)
    w = _c(w, npdt)
    m, k = a.shape
    n = w.shape[0]
    ii = _c(ii, np.int64)
    jj = _c(jj, np.int64)
    c = np.empty(ii.size, np.float64)
    mag = np.empty(ii.size, np.float64)
    _check((L or lib()).orc_gemm_nt_sampled(_ptr(a), _ptr(w), code, m, n, k, _ptr(ii), _ptr(jj), ii.size,
                                            _ptr(c), _ptr(mag)), "gemm_nt_sampled")
    return c, mag


# --------------------------------------------------------------------------- ternary

def pack_ternary(codes, L=None):
    """codes uint8[n][k] (0..2) -> uint32[n][k/16]."""
    codes = _c(codes, np.uint8)
    n, k = codes.shape
    words = np.empty((n, k // 16), np.uint32)
    _check((L or lib()).orc_pack_ternary(_ptr(codes), _ptr(words), n, k), "pack_ternary")
    return words


def unpack_ternary(words, n, k, L=None):
    words = _c(words, np.uint32)
    codes = np.empty((n, k), np.uint8)
    _check((L or lib()).orc_unpack_ternary(_ptr(words), _ptr(codes), n, k), "unpack_ternary")
    return codes


def quantize_i8_rows(x, L=None):
    """x float32[m][k] -> (q int8[m][k], act_scale float32[m], act_sum int32[m])."""
    x = _c(x, np.float32)
    if x.ndim == 1:
        x = x[None, :]
    m, k = x.shape
    q = np.empty((m, k), np.int8)
    s = np.empty(m, np.float32)
    t = np.empty(m, np.int32)
    _check((L or lib()).orc_quantize_i8_rows(_ptr(x), _ptr(q), _ptr(s), _ptr(t), m, k), "quantize_i8_rows")
    return q, s, t


def ternary(words, w_scale, q, act_scale, act_sum, n, k, with_dots=False, L=None):
    words = _c(words, np.uint32)
    q = _c(q, np.int8)
    if q.ndim == 1:
        q = q[None, :]
    m = q.shape[0]
    act_scale = _c(act_scale, np.float32)
    act_sum = _c(act_sum, np.int32)
    y = np.empty((m, n), np.float64)
    mag = np.empty((m, n), np.float64)
    dots = np.empty((m, n), np.int32) if with_dots else None
    _check((L or lib()).orc_ternary(_ptr(words), float(w_scale), _ptr(q), _ptr(act_scale), _ptr(act_sum),
                                    m, n, k, _ptr(y), _ptr(mag), _ptr(dots)), "ternary")
    return (y, mag, dots) if with_dots else (y, mag)


def ternary_sampled(words, w_scale, q, act_scale, act_sum, n, k, ii, jj, L=None):
    words = _c(words, np.uint32)
    q = _c(q, np.int8)
    if q.ndim == 1:
        q = q[None, :]
    m = q.shape[0]
    act_scale = _c(act_scale, np.float32)
    act_sum = _c(act_sum, np.int32)
    ii = _c(ii, np.int64)
    jj = _c(jj, np.int64)
    y = np.empty(ii.size, np.float64)
    mag = np.empty(ii.size, np.float64)
    _check((L or lib()).orc_ternary_sampled(_ptr(words), float(w_scale), _ptr(q), _ptr(act_scale), _ptr(act_sum),
                                            m, n, k, _ptr(ii), _ptr(jj), ii.size, _ptr(y), _ptr(mag)),
           "ternary_sampled")
    return y, mag
