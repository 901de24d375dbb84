"""Helpers of the GPU parity tests: device allocation and one call per entry
point through the Python binding (which calls the C ABI), plus the tolerance
check.  Nothing here computes any part of the method."""
import numpy as np
import torch

import quantized_linear_layer_amd as qll

DEV = torch.device("cuda:0")


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def empty(nbytes_or_n, dtype=torch.uint8):
    return torch.empty(int(nbytes_or_n), dtype=dtype, device=DEV)


def pack_q4_0(codes, d_bits):
    n, k = codes.shape
    w = empty(n * (k // 32) * 18)
    qll.qll_pack_q4_0(dev(codes), dev(np.asarray(d_bits, np.uint16).view(np.int16)), w, n, k)
    return w


def quantize_q8_0(x):
    x = np.asarray(x, np.float32)
    m, k = x.shape
    xq = empty(m * (k // 32) * 34)
    qll.qll_quantize_q8_0(dev(x), xq, m, k)
    return xq


def q4_gemv(w, xq, n, k):
    y = empty(n, torch.float32)
    qll.qll_q4_0_q8_0_gemv(w, xq, y, n, k)
    return y


def q4_gemm(w, xq, m, n, k):
    y = empty(m * n, torch.float32)
    need = qll.qll_workspace_bytes(qll.QLL_OP_Q4_0_Q8_0_GEMM, m, n, k)
    ws = empty(need) if need else None
    qll.qll_q4_0_q8_0_gemm(w, xq, y, m, n, k, ws=ws)
    return y


def sgemm(a_t, b_t, m, n, k):
    c = empty(m * n, torch.float32)
    need = qll.qll_workspace_bytes(qll.QLL_OP_SGEMM, m, n, k)
    ws = empty(need) if need else None
    qll.qll_sgemm(a_t, b_t, c, m, n, k, ws=ws)
    return c


def quantize_i8_rows(x):
    x = np.asarray(x, np.float32)
    m, k = x.shape
    q = empty(m * k, torch.int8)
    s = empty(m, torch.float32)
    t = empty(m, torch.int32)
    qll.qll_quantize_i8_rows(dev(x), q, s, t, m, k)
    return q, s, t


def pack_ternary(codes):
    n, k = codes.shape
    w = empty(n * (k // 16), torch.int32)
    qll.qll_pack_ternary(dev(codes), w, n, k)
    return w


def ternary(w, w_scale, q, s, t, m, n, k):
    y = empty(m * n, torch.float32)
    if m == 1:
        qll.qll_ternary_gemv(w, w_scale, q, s, t, y, n, k)
    else:
        qll.qll_ternary_gemm(w, w_scale, q, s, t, y, m, n, k)
    return y


def assert_within(y, y_ref, mag, rel, what):
    """|y - y_ref| <= rel * mag elementwise (mag = 0 demands y == 0 exactly)."""
    y = np.asarray(y, np.float64).reshape(y_ref.shape)
    err = np.abs(y - y_ref)
    bad = ~(err <= rel * mag)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside {rel}*mag; first at {idx.tolist()}: "
                             f"got {y[tuple(idx[0])]!r} want {y_ref[tuple(idx[0])]!r} mag {mag[tuple(idx[0])]!r}")
    return float((err / np.where(mag > 0, mag, 1)).max()) if err.size else 0.0
