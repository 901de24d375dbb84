"""Python binding of libqll.so, the quantized linear layer for MI355X.

Argument marshalling only: every function has the name and the argument
order of the C entry point in include/qll.h, takes device tensors (PyTorch is
used for device memory and streams), checks that each tensor is a contiguous
CUDA tensor holding at least the bytes the call will touch, and passes raw
pointers plus torch's current stream.  All arithmetic runs in the HIP
kernels.  There is no fallback of any kind: if libqll.so is missing or does
not load, `load()` and every call raise.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqll.so")

QLL_OK = 0
QLL_OP_SGEMM = 1
QLL_OP_Q4_0_Q8_0_GEMM = 2
QLL_OP_TERNARY_GEMM = 3
QLL_OP_Q4_0_REPACKED_GEMM = 4
QLL_OP_Q8_0_REPACKED_GEMM = 5
QLL_OP_GEMM_NT_BF16 = 6
QLL_OP_GEMM_NT_F16 = 7
QLL_OP_GEMM_NT_F32 = 8
QLL_OP_SGEMM_BF16 = 9
QLL_OP_Q4_0_GEMV_F32 = 10
QLL_DTYPE_F32, QLL_DTYPE_BF16, QLL_DTYPE_F16 = 0, 1, 2

Q4_0_BLOCK_BYTES = 18
Q8_0_BLOCK_BYTES = 34

_lib = None


class QllError(RuntimeError):
    def __init__(self, fn, rc, msg):
        super().__init__(f"{fn}: {msg} (status {rc})")
        self.status = rc


def load(path=LIB_PATH):
    """Load libqll.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`")
    L = ctypes.CDLL(path)
    P, I, S, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    sig = {
        "qll_pack_q4_0": [P, P, P, I, I, P],
        "qll_pack_ternary": [P, P, I, I, P],
        "qll_quantize_q8_0": [P, P, I, I, P],
        "qll_q4_0_q8_0_gemv": [P, P, P, I, I, P],
        "qll_q4_0_q8_0_gemm": [P, P, P, I, I, I, P, S, P],
        "qll_q4_0_q8_0_gemv_f32": [P, P, P, I, I, I, P, S, P],
        "qll_q4_0_q8_0_gemm_noalloc": [P, P, P, I, I, I, P],
        "qll_q4_0_repack": [P, P, I, I, P],
        "qll_q4_0_decode_pack": [P, P, I, I, P],
        "qll_q4_0_decode_packed_q8_0_gemv": [P, P, P, I, I, P],
        "qll_q4_0_repacked_q8_0_gemm": [P, P, P, I, I, I, P, S, P],
        "qll_q8_0_q8_0_gemv": [P, P, P, I, I, P],
        "qll_q8_0_repack": [P, P, I, I, P],
        "qll_q8_0_repacked_q8_0_gemm": [P, P, P, I, I, I, P, S, P],
        "qll_sgemm": [P, P, P, I, I, I, P, S, P],
        "qll_gemm_nt": [P, P, ctypes.c_int, P, I, I, I, P, S, P],
        "qll_quantize_i8_rows": [P, P, P, P, I, I, P],
        "qll_ternary_gemv": [P, F, P, P, P, P, I, I, P],
        "qll_ternary_gemm": [P, F, P, P, P, P, I, I, I, P],
    }
    for name, args in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    L.qll_workspace_bytes.argtypes = [ctypes.c_int, I, I, I]
    L.qll_workspace_bytes.restype = ctypes.c_size_t
    L.qll_q4_0_repacked_bytes.argtypes = [I, I]
    L.qll_q4_0_repacked_bytes.restype = ctypes.c_size_t
    L.qll_q4_0_decode_packed_bytes.argtypes = [I, I]
    L.qll_q4_0_decode_packed_bytes.restype = ctypes.c_size_t
    L.qll_q8_0_repacked_bytes.argtypes = [I, I]
    L.qll_q8_0_repacked_bytes.restype = ctypes.c_size_t
    L.qll_status_string.argtypes = [ctypes.c_int]
    L.qll_status_string.restype = ctypes.c_char_p
    _lib = L
    return L


def qll_status_string(status):
    return load().qll_status_string(int(status)).decode()


def qll_workspace_bytes(op, m, n, k):
    return int(load().qll_workspace_bytes(int(op), int(m), int(n), int(k)))


def _ptr(t, nbytes, what):
    """Device pointer of `t` after checking it can hold `nbytes` bytes."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{what} must be a CUDA tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{what} holds {have} bytes, the call needs {nbytes}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _call(name, *args):
    rc = getattr(load(), name)(*args)
    if rc != QLL_OK:
        raise QllError(name, rc, qll_status_string(rc))


def _ws(ws, need):
    if need == 0:
        return None, 0
    if ws is None:
        raise ValueError(f"a workspace of {need} bytes is required")
    return _ptr(ws, need, "ws"), ws.numel() * ws.element_size()


# ----------------------------------------------------------------- packing

def qll_pack_q4_0(codes, d_bits, w, n, k, stream=None):
    _call("qll_pack_q4_0", _ptr(codes, n * k, "codes"), _ptr(d_bits, n * (k // 32) * 2, "d_bits"),
          _ptr(w, n * (k // 32) * Q4_0_BLOCK_BYTES, "w"), n, k, _stream(stream))


def qll_pack_ternary(codes, w, n, k, stream=None):
    _call("qll_pack_ternary", _ptr(codes, n * k, "codes"), _ptr(w, n * (k // 16) * 4, "w"), n, k, _stream(stream))


# ----------------------------------------------------------------- Q4_0 x Q8_0

def qll_quantize_q8_0(x, xq, m, k, stream=None):
    _call("qll_quantize_q8_0", _ptr(x, m * k * 4, "x"), _ptr(xq, m * (k // 32) * Q8_0_BLOCK_BYTES, "xq"), m, k,
          _stream(stream))


def qll_q4_0_q8_0_gemv(w, xq, y, n, k, stream=None):
    _call("qll_q4_0_q8_0_gemv", _ptr(w, n * (k // 32) * Q4_0_BLOCK_BYTES, "w"),
          _ptr(xq, (k // 32) * Q8_0_BLOCK_BYTES, "xq"), _ptr(y, n * 4, "y"), n, k, _stream(stream))


def qll_q4_0_q8_0_gemm(w, xq, y, m, n, k, ws=None, stream=None):
    need = qll_workspace_bytes(QLL_OP_Q4_0_Q8_0_GEMM, m, n, k)
    wsp, wsb = _ws(ws, need) if need != 2 ** 64 - 1 else (None, 0)
    _call("qll_q4_0_q8_0_gemm", _ptr(w, n * (k // 32) * Q4_0_BLOCK_BYTES, "w"),
          _ptr(xq, m * (k // 32) * Q8_0_BLOCK_BYTES, "xq"), _ptr(y, m * n * 4, "y"), m, n, k, wsp, wsb,
          _stream(stream))


QLL_NOALLOC_SCRATCH_BYTES = 64 << 20


def qll_q4_0_q8_0_gemm_noalloc(w, xq, y, m, n, k, stream=None):
    """qll_q4_0_q8_0_gemm with its workspace in the library's static device
    scratch (no allocation, no workspace argument); calls on one device must
    not overlap."""
    _call("qll_q4_0_q8_0_gemm_noalloc", _ptr(w, n * (k // 32) * Q4_0_BLOCK_BYTES, "w"),
          _ptr(xq, m * (k // 32) * Q8_0_BLOCK_BYTES, "xq"), _ptr(y, m * n * 4, "y"), m, n, k, _stream(stream))


def qll_q4_0_q8_0_gemv_f32(w, x, y, m, n, k, ws=None, stream=None):
    """Quantize-fused decode, 1 <= m <= 8: y[m][n] = Q8_0(x).W^T.  A workspace
    of at least qll_workspace_bytes(QLL_OP_Q4_0_GEMV_F32, ...) bytes (when
    that is nonzero) selects quantize-once-then-decode; none or a smaller
    one the single launch that quantizes in every workgroup."""
    wsp, wsb = (None, 0) if ws is None else (_ptr(ws, 0, "ws"), ws.numel() * ws.element_size())
    _call("qll_q4_0_q8_0_gemv_f32", _ptr(w, n * (k // 32) * Q4_0_BLOCK_BYTES, "w"), _ptr(x, m * k * 4, "x"),
          _ptr(y, m * n * 4, "y"), m, n, k, wsp, wsb, _stream(stream))


def qll_q4_0_decode_packed_bytes(n, k):
    return int(load().qll_q4_0_decode_packed_bytes(int(n), int(k)))


def qll_q4_0_decode_pack(w, wp, n, k, stream=None):
    """Load-time repack of Q4_0 blocks into the decode GEMV's aligned groups."""
    _call("qll_q4_0_decode_pack", _ptr(w, n * (k // 32) * Q4_0_BLOCK_BYTES, "w"),
          _ptr(wp, qll_q4_0_decode_packed_bytes(n, k), "wp"), n, k, _stream(stream))


def qll_q4_0_decode_packed_q8_0_gemv(wp, xq, y, n, k, stream=None):
    _call("qll_q4_0_decode_packed_q8_0_gemv", _ptr(wp, qll_q4_0_decode_packed_bytes(n, k), "wp"),
          _ptr(xq, (k // 32) * Q8_0_BLOCK_BYTES, "xq"), _ptr(y, n * 4, "y"), n, k, _stream(stream))


def qll_q4_0_repacked_bytes(n, k):
    return int(load().qll_q4_0_repacked_bytes(int(n), int(k)))


def qll_q4_0_repack(w, wp, n, k, stream=None):
    """Load-time repack of Q4_0 blocks into the matrix-core operand form."""
    need = qll_q4_0_repacked_bytes(n, k)
    _call("qll_q4_0_repack", _ptr(w, n * (k // 32) * Q4_0_BLOCK_BYTES, "w"),
          _ptr(wp, need if need != 2 ** 64 - 1 else 0, "wp"), n, k, _stream(stream))


def qll_q4_0_repacked_q8_0_gemm(wp, xq, y, m, n, k, ws=None, stream=None):
    need = qll_workspace_bytes(QLL_OP_Q4_0_REPACKED_GEMM, m, n, k)
    if need == 2 ** 64 - 1:
        wsp, wsb = None, 0
    else:
        wsp, wsb = _ws(ws, need)
    wp_need = qll_q4_0_repacked_bytes(n, k)
    _call("qll_q4_0_repacked_q8_0_gemm", _ptr(wp, wp_need if wp_need != 2 ** 64 - 1 else 0, "wp"),
          _ptr(xq, m * (k // 32) * Q8_0_BLOCK_BYTES, "xq"), _ptr(y, m * n * 4, "y"), m, n, k, wsp, wsb,
          _stream(stream))


# ----------------------------------------------------------------- Q8_0 weights

def qll_q8_0_q8_0_gemv(w, xq, y, n, k, stream=None):
    _call("qll_q8_0_q8_0_gemv", _ptr(w, n * (k // 32) * Q8_0_BLOCK_BYTES, "w"),
          _ptr(xq, (k // 32) * Q8_0_BLOCK_BYTES, "xq"), _ptr(y, n * 4, "y"), n, k, _stream(stream))


def qll_q8_0_repacked_bytes(n, k):
    return int(load().qll_q8_0_repacked_bytes(int(n), int(k)))


def qll_q8_0_repack(w, wp, n, k, stream=None):
    """Load-time repack of Q8_0 weight blocks into the matrix-core operand form."""
    need = qll_q8_0_repacked_bytes(n, k)
    _call("qll_q8_0_repack", _ptr(w, n * (k // 32) * Q8_0_BLOCK_BYTES, "w"),
          _ptr(wp, need if need != 2 ** 64 - 1 else 0, "wp"), n, k, _stream(stream))


def qll_q8_0_repacked_q8_0_gemm(wp, xq, y, m, n, k, ws=None, stream=None):
    need = qll_workspace_bytes(QLL_OP_Q8_0_REPACKED_GEMM, m, n, k)
    if need == 2 ** 64 - 1:
        wsp, wsb = None, 0
    else:
        wsp, wsb = _ws(ws, need)
    wp_need = qll_q8_0_repacked_bytes(n, k)
    _call("qll_q8_0_repacked_q8_0_gemm", _ptr(wp, wp_need if wp_need != 2 ** 64 - 1 else 0, "wp"),
          _ptr(xq, m * (k // 32) * Q8_0_BLOCK_BYTES, "xq"), _ptr(y, m * n * 4, "y"), m, n, k, wsp, wsb,
          _stream(stream))


# ----------------------------------------------------------------- f32

def qll_sgemm(a, b, c, m, n, k, ws=None, stream=None):
    """C = A.B; m == 1 needs a workspace (QLL_OP_SGEMM); at m > 1 a workspace
    of at least qll_workspace_bytes(QLL_OP_SGEMM_BF16, ...) bytes selects the
    bf16 matrix core, none or a smaller one the f32 one."""
    if m > 1 and ws is not None:  # the workspace's size selects the algorithm
        wsp, wsb = _ptr(ws, 0, "ws"), ws.numel() * ws.element_size()
    else:
        need = qll_workspace_bytes(QLL_OP_SGEMM, m, n, k)
        wsp, wsb = _ws(ws, need) if need != 2 ** 64 - 1 else (None, 0)
    _call("qll_sgemm", _ptr(a, m * k * 4, "a"), _ptr(b, k * n * 4, "b"), _ptr(c, m * n * 4, "c"), m, n, k, wsp, wsb,
          _stream(stream))


def qll_gemm_nt(x, w, w_dtype, y, m, n, k, ws=None, stream=None):
    """Y = X.W^T with W [n][k] of element type w_dtype (QLL_DTYPE_F32/BF16/F16);
    bf16 weights at m > 1 may need a workspace (qll_workspace_bytes with
    QLL_OP_GEMM_NT_BF16); f16 and f32 weights run on the bf16 matrix core when
    the workspace holds at least qll_workspace_bytes(QLL_OP_GEMM_NT_F16 / _F32,
    ...) bytes, on the f32 matrix core otherwise."""
    esize = 4 if w_dtype == QLL_DTYPE_F32 else 2
    if w_dtype == QLL_DTYPE_BF16:
        need = qll_workspace_bytes(QLL_OP_GEMM_NT_BF16, m, n, k)
    else:
        need = 0
    if w_dtype != QLL_DTYPE_BF16 and ws is not None:  # the workspace's size selects the algorithm
        wsp, wsb = _ptr(ws, 0, "ws"), ws.numel() * ws.element_size()
    else:
        wsp, wsb = _ws(ws, need) if need != 2 ** 64 - 1 else (None, 0)
    _call("qll_gemm_nt", _ptr(x, m * k * 4, "x"), _ptr(w, n * k * esize, "w"), int(w_dtype), _ptr(y, m * n * 4, "y"),
          m, n, k, wsp, wsb, _stream(stream))


# ----------------------------------------------------------------- ternary

def qll_quantize_i8_rows(x, xq, act_scale, act_sum, m, k, stream=None):
    _call("qll_quantize_i8_rows", _ptr(x, m * k * 4, "x"), _ptr(xq, m * k, "xq"), _ptr(act_scale, m * 4, "act_scale"),
          _ptr(act_sum, m * 4, "act_sum"), m, k, _stream(stream))


def qll_ternary_gemv(w, w_scale, xq, act_scale, act_sum, y, n, k, stream=None):
    _call("qll_ternary_gemv", _ptr(w, n * (k // 16) * 4, "w"), ctypes.c_float(float(w_scale)), _ptr(xq, k, "xq"),
          _ptr(act_scale, 4, "act_scale"), _ptr(act_sum, 4, "act_sum"), _ptr(y, n * 4, "y"), n, k, _stream(stream))


def qll_ternary_gemm(w, w_scale, xq, act_scale, act_sum, y, m, n, k, stream=None):
    _call("qll_ternary_gemm", _ptr(w, n * (k // 16) * 4, "w"), ctypes.c_float(float(w_scale)),
          _ptr(xq, m * k, "xq"), _ptr(act_scale, m * 4, "act_scale"), _ptr(act_sum, m * 4, "act_sum"),
          _ptr(y, m * n * 4, "y"), m, n, k, _stream(stream))
