"""The C-ABI library on the CPU: it loads, exports every entry point that
include/qll.h declares, and rejects bad arguments with the documented status
before touching any device (no compute call is made here)."""
import ctypes
import os
import re
import subprocess

import pytest

import quantized_linear_layer_amd as qll

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qll.h")

OK, NULL, SHAPE, ALIGN, WORKSPACE = 0, -1, -2, -3, -4
SIZE_MAX = 2 ** 64 - 1


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(qll_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return qll.load()


def test_library_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 11
    for name in names:
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", qll.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\sT\s(qll_\w+)", out))
    assert set(names) <= exported
    assert exported <= set(names), f"undeclared exports: {exported - set(names)}"


def test_library_is_built_for_gfx950():
    # the offload bundle inside libqll.so names its target triple
    out = subprocess.run(["strings", qll.LIB_PATH], capture_output=True, text=True, check=True).stdout
    assert "amdgcn-amd-amdhsa--gfx950" in out


def test_status_strings(L):
    for rc in (0, -1, -2, -3, -4, -5, -6):
        assert qll.qll_status_string(rc) != "unknown status"
    assert qll.qll_status_string(-99) == "unknown status"


def test_workspace_sizes(L):
    assert qll.qll_workspace_bytes(qll.QLL_OP_SGEMM, 4096, 4096, 4096) == 0
    ws = qll.qll_workspace_bytes(qll.QLL_OP_SGEMM, 1, 4096, 4096)
    assert 0 < ws <= 4096 * 4096 * 4
    assert ws % (4096 * 4) == 0
    assert qll.qll_workspace_bytes(qll.QLL_OP_Q4_0_Q8_0_GEMM, 1, 4096, 4096) == 0
    assert qll.qll_workspace_bytes(qll.QLL_OP_Q4_0_Q8_0_GEMM, 512, 4096, 33) == SIZE_MAX
    assert qll.qll_workspace_bytes(qll.QLL_OP_Q4_0_Q8_0_GEMM, 9, 64, 2 ** 24) == SIZE_MAX  # GEMM k limit
    assert qll.qll_workspace_bytes(qll.QLL_OP_Q4_0_Q8_0_GEMM, 1, 64, 2 ** 24) == 0        # the GEMV has none
    for m in range(2, 65):                                                                 # small-m kernels
        assert qll.qll_workspace_bytes(qll.QLL_OP_Q4_0_Q8_0_GEMM, m, 4096, 14336) == 0
    assert qll.qll_workspace_bytes(qll.QLL_OP_Q4_0_Q8_0_GEMM, 8, 64, 2 ** 24) == 0         # m <= 8: no k limit
    assert qll.qll_workspace_bytes(qll.QLL_OP_Q4_0_Q8_0_GEMM, 65, 4096, 14336) > 0         # the 128-row GEMM
    assert qll.qll_workspace_bytes(qll.QLL_OP_Q4_0_Q8_0_GEMM, 64, 128256, 4096) == 0
    assert qll.qll_workspace_bytes(qll.QLL_OP_Q4_0_Q8_0_GEMM, 65, 128256, 4096) > 0
    assert qll.qll_workspace_bytes(qll.QLL_OP_TERNARY_GEMM, 64, 6912, 2560) == 0
    assert qll.qll_workspace_bytes(qll.QLL_OP_TERNARY_GEMM, 64, 6912, 2561) == SIZE_MAX
    # the fused entry: none where its single launch is the faster route
    assert qll.qll_workspace_bytes(qll.QLL_OP_Q4_0_GEMV_F32, 1, 4096, 4096) == 0
    assert qll.qll_workspace_bytes(qll.QLL_OP_Q4_0_GEMV_F32, 1, 14336, 4096) >= 128 * 34
    assert qll.qll_workspace_bytes(qll.QLL_OP_Q4_0_GEMV_F32, 8, 4096, 14336) >= 8 * 448 * 34
    assert qll.qll_workspace_bytes(qll.QLL_OP_Q4_0_GEMV_F32, 9, 4096, 4096) == SIZE_MAX
    assert qll.qll_workspace_bytes(qll.QLL_OP_Q4_0_GEMV_F32, 2, 8, 48) == SIZE_MAX
    assert qll.qll_workspace_bytes(99, 1, 1, 1) == SIZE_MAX
    assert qll.qll_workspace_bytes(qll.QLL_OP_SGEMM, 0, 4, 4) == SIZE_MAX


GOOD = ctypes.c_void_p(0x10000)
MIS = ctypes.c_void_p(0x10004)  # not 16-byte aligned
NUL = None


def test_pack_errors(L):
    assert L.qll_pack_q4_0(NUL, GOOD, GOOD, 4, 64, None) == NULL
    assert L.qll_pack_q4_0(GOOD, GOOD, GOOD, 4, 48, None) == SHAPE
    assert L.qll_pack_q4_0(GOOD, GOOD, GOOD, 0, 64, None) == SHAPE
    assert L.qll_pack_q4_0(GOOD, MIS, GOOD, 4, 64, None) == ALIGN
    assert L.qll_pack_ternary(GOOD, NUL, 4, 64, None) == NULL
    assert L.qll_pack_ternary(GOOD, GOOD, 4, 24, None) == SHAPE
    assert L.qll_pack_ternary(MIS, GOOD, 4, 32, None) == ALIGN


def test_q4_errors(L):
    assert L.qll_quantize_q8_0(NUL, GOOD, 1, 64, None) == NULL
    assert L.qll_quantize_q8_0(GOOD, GOOD, 1, 40, None) == SHAPE
    assert L.qll_quantize_q8_0(GOOD, GOOD, -1, 64, None) == SHAPE
    assert L.qll_quantize_q8_0(GOOD, MIS, 1, 64, None) == ALIGN
    assert L.qll_q4_0_q8_0_gemv(GOOD, GOOD, NUL, 8, 64, None) == NULL
    assert L.qll_q4_0_q8_0_gemv(GOOD, GOOD, GOOD, 8, 65, None) == SHAPE
    assert L.qll_q4_0_q8_0_gemv(GOOD, GOOD, GOOD, 8, 49152 + 32, None) == SHAPE  # beyond the LDS-staged k
    assert L.qll_q4_0_q8_0_gemm(GOOD, GOOD, GOOD, 1, 8, 49152 + 32, NUL, 0, None) == SHAPE  # m = 1: the GEMV
    assert L.qll_q4_0_q8_0_gemv(GOOD, GOOD, GOOD, 2 ** 31, 64, None) == SHAPE
    assert L.qll_q4_0_q8_0_gemv(MIS, GOOD, GOOD, 8, 64, None) == ALIGN
    assert L.qll_q4_0_q8_0_gemm(GOOD, NUL, GOOD, 4, 8, 64, NUL, 0, None) == NULL
    assert L.qll_q4_0_q8_0_gemm(GOOD, GOOD, GOOD, 4, 8, 16, NUL, 0, None) == SHAPE
    assert L.qll_q4_0_q8_0_gemm(GOOD, GOOD, MIS, 4, 8, 64, NUL, 0, None) == ALIGN
    assert L.qll_q4_0_q8_0_gemm(GOOD, GOOD, GOOD, 16, 8, 2 ** 24, GOOD, 2 ** 40, None) == SHAPE
    assert L.qll_q4_0_q8_0_gemv_f32(GOOD, NUL, GOOD, 1, 8, 64, NUL, 0, None) == NULL
    assert L.qll_q4_0_q8_0_gemv_f32(GOOD, GOOD, GOOD, 0, 8, 64, NUL, 0, None) == SHAPE
    assert L.qll_q4_0_q8_0_gemv_f32(GOOD, GOOD, GOOD, 9, 8, 64, NUL, 0, None) == SHAPE
    assert L.qll_q4_0_q8_0_gemv_f32(GOOD, GOOD, GOOD, 2, 8, 48, NUL, 0, None) == SHAPE
    assert L.qll_q4_0_q8_0_gemv_f32(GOOD, MIS, GOOD, 2, 8, 64, NUL, 0, None) == ALIGN
    assert L.qll_q4_0_q8_0_gemv_f32(GOOD, GOOD, GOOD, 2, 8, 64, MIS, 2 ** 20, None) == ALIGN  # a workspace in use
    # decode-packed weights: the pack and the GEMV on them
    assert qll.qll_q4_0_decode_packed_bytes(8, 64) == 8 * (2 * 16 + 16)
    assert qll.qll_q4_0_decode_packed_bytes(3, 4096) == 3 * 128 * 18
    assert qll.qll_q4_0_decode_packed_bytes(2, 14336 + 32) == 2 * (449 * 16 + 57 * 16)
    assert qll.qll_q4_0_decode_packed_bytes(8, 48) == SIZE_MAX
    assert L.qll_q4_0_decode_pack(NUL, GOOD, 8, 64, None) == NULL
    assert L.qll_q4_0_decode_pack(GOOD, GOOD, 8, 48, None) == SHAPE
    assert L.qll_q4_0_decode_pack(GOOD, MIS, 8, 64, None) == ALIGN
    assert L.qll_q4_0_decode_packed_q8_0_gemv(GOOD, NUL, GOOD, 8, 64, None) == NULL
    assert L.qll_q4_0_decode_packed_q8_0_gemv(GOOD, GOOD, GOOD, 0, 64, None) == SHAPE
    assert L.qll_q4_0_decode_packed_q8_0_gemv(GOOD, GOOD, GOOD, 8, 49152 + 32, None) == SHAPE
    assert L.qll_q4_0_decode_packed_q8_0_gemv(MIS, GOOD, GOOD, 8, 64, None) == ALIGN
    # repacked weights: the repack and the GEMM on them
    assert L.qll_q4_0_repack(NUL, GOOD, 8, 64, None) == NULL
    assert L.qll_q4_0_repack(GOOD, GOOD, 8, 48, None) == SHAPE
    assert L.qll_q4_0_repack(GOOD, GOOD, 0, 64, None) == SHAPE
    assert L.qll_q4_0_repack(GOOD, MIS, 8, 64, None) == ALIGN
    assert L.qll_q4_0_repacked_q8_0_gemm(GOOD, GOOD, GOOD, 4, 8, 64, NUL, 0, None) == NULL
    assert L.qll_q4_0_repacked_q8_0_gemm(GOOD, GOOD, GOOD, 4, 8, 80, GOOD, 2 ** 40, None) == SHAPE
    # 32-bit block offsets inside the kernel: k below 2^24
    assert L.qll_q4_0_repacked_q8_0_gemm(GOOD, GOOD, GOOD, 4, 8, 2 ** 24, GOOD, 2 ** 40, None) == SHAPE
    assert L.qll_q4_0_repacked_q8_0_gemm(GOOD, GOOD, GOOD, 4, 8, 2 ** 25 - 32, GOOD, 2 ** 40, None) == SHAPE
    assert qll.qll_workspace_bytes(qll.QLL_OP_Q4_0_REPACKED_GEMM, 4, 8, 2 ** 24) == SIZE_MAX
    assert qll.qll_workspace_bytes(qll.QLL_OP_Q4_0_REPACKED_GEMM, 4, 8, 2 ** 24 - 32) < SIZE_MAX
    assert L.qll_q4_0_repacked_q8_0_gemm(GOOD, GOOD, MIS, 4, 8, 64, GOOD, 2 ** 40, None) == ALIGN
    assert L.qll_q4_0_repacked_q8_0_gemm(GOOD, GOOD, GOOD, 4, 8, 64, MIS, 2 ** 40, None) == ALIGN
    assert L.qll_q4_0_repacked_q8_0_gemm(GOOD, GOOD, GOOD, 4, 8, 64, GOOD, 16, None) == WORKSPACE


def test_noalloc_gemm_errors(L):
    SCRATCH = -7
    assert L.qll_q4_0_q8_0_gemm_noalloc(NUL, GOOD, GOOD, 16, 8, 64, None) == NULL
    assert L.qll_q4_0_q8_0_gemm_noalloc(GOOD, GOOD, GOOD, 16, 8, 48, None) == SHAPE
    assert L.qll_q4_0_q8_0_gemm_noalloc(GOOD, GOOD, GOOD, 16, 8, 2 ** 24, None) == SHAPE
    assert L.qll_q4_0_q8_0_gemm_noalloc(GOOD, GOOD, MIS, 16, 8, 64, None) == ALIGN
    # a shape whose workspace exceeds the static scratch is refused before any device call
    assert qll.qll_workspace_bytes(qll.QLL_OP_Q4_0_Q8_0_GEMM, 4096, 64, 14336) > qll.QLL_NOALLOC_SCRATCH_BYTES
    assert L.qll_q4_0_q8_0_gemm_noalloc(GOOD, GOOD, GOOD, 4096, 64, 14336, None) == SCRATCH
    assert "static" in qll.qll_status_string(SCRATCH)
    # every 8B-class prefill layer at m = 512 fits
    for k, n in ((4096, 14336), (14336, 4096), (4096, 4096), (4096, 128256)):
        assert qll.qll_workspace_bytes(qll.QLL_OP_Q4_0_Q8_0_GEMM, 512, n, k) <= qll.QLL_NOALLOC_SCRATCH_BYTES


def test_q8w_errors(L):
    assert L.qll_q8_0_q8_0_gemv(GOOD, NUL, GOOD, 8, 64, None) == NULL
    assert L.qll_q8_0_q8_0_gemv(GOOD, GOOD, GOOD, 8, 65, None) == SHAPE
    assert L.qll_q8_0_q8_0_gemv(GOOD, GOOD, GOOD, 8, 49152 + 32, None) == SHAPE
    assert L.qll_q8_0_q8_0_gemv(MIS, GOOD, GOOD, 8, 64, None) == ALIGN
    assert L.qll_q8_0_repack(GOOD, NUL, 8, 64, None) == NULL
    assert L.qll_q8_0_repack(GOOD, GOOD, 8, 40, None) == SHAPE
    assert L.qll_q8_0_repack(MIS, GOOD, 8, 64, None) == ALIGN
    assert L.qll_q8_0_repacked_q8_0_gemm(GOOD, GOOD, NUL, 4, 8, 64, GOOD, 2 ** 40, None) == NULL
    assert L.qll_q8_0_repacked_q8_0_gemm(GOOD, GOOD, GOOD, 0, 8, 64, GOOD, 2 ** 40, None) == SHAPE
    assert L.qll_q8_0_repacked_q8_0_gemm(GOOD, GOOD, GOOD, 4, 8, 2 ** 24, GOOD, 2 ** 40, None) == SHAPE
    assert qll.qll_workspace_bytes(qll.QLL_OP_Q8_0_REPACKED_GEMM, 4, 8, 2 ** 24) == SIZE_MAX
    assert L.qll_q8_0_repacked_q8_0_gemm(GOOD, MIS, GOOD, 4, 8, 64, GOOD, 2 ** 40, None) == ALIGN
    assert L.qll_q8_0_repacked_q8_0_gemm(GOOD, GOOD, GOOD, 4, 8, 64, GOOD, 1, None) == WORKSPACE
    assert qll.qll_q8_0_repacked_bytes(1, 32) == 6400
    assert qll.qll_q8_0_repacked_bytes(130, 64) == 2 * 2 * 6400
    assert qll.qll_q8_0_repacked_bytes(8, 40) == SIZE_MAX
    assert qll.qll_workspace_bytes(qll.QLL_OP_Q8_0_REPACKED_GEMM, 512, 4096, 4096) == \
        qll.qll_workspace_bytes(qll.QLL_OP_Q4_0_REPACKED_GEMM, 512, 4096, 4096)


def test_gemm_nt_errors(L):
    assert L.qll_gemm_nt(NUL, GOOD, 0, GOOD, 2, 2, 2, NUL, 0, None) == NULL
    assert L.qll_gemm_nt(GOOD, GOOD, 3, GOOD, 2, 2, 2, NUL, 0, None) == SHAPE
    assert L.qll_gemm_nt(GOOD, GOOD, -1, GOOD, 2, 2, 2, NUL, 0, None) == SHAPE
    assert L.qll_gemm_nt(GOOD, GOOD, 1, GOOD, 2, 0, 2, NUL, 0, None) == SHAPE
    assert L.qll_gemm_nt(GOOD, MIS, 2, GOOD, 2, 2, 2, NUL, 0, None) == ALIGN
    # bf16 weights, m > 1, k % 16 == 0: the split activations need a workspace
    assert L.qll_gemm_nt(GOOD, GOOD, 1, GOOD, 2, 8, 32, NUL, 0, None) == WORKSPACE
    assert L.qll_gemm_nt(GOOD, GOOD, 1, GOOD, 2, 8, 32, MIS, 2 ** 40, None) == ALIGN
    split_x = 4 * 256 * 3 * 128 * 16 * 2                            # three bf16 copies of X (512 x 4096)
    assert qll.qll_workspace_bytes(qll.QLL_OP_GEMM_NT_BF16, 4096, 4096, 4096) == 8 * split_x   # no K split
    need = qll.qll_workspace_bytes(qll.QLL_OP_GEMM_NT_BF16, 512, 4096, 4096)
    assert need == split_x + 4 * 512 * 4096 * 4                      # 128 tiles: K split 4 ways, f32 partials
    assert qll.qll_workspace_bytes(qll.QLL_OP_GEMM_NT_BF16, 1, 4096, 4096) == 0   # the GEMV needs none
    assert qll.qll_workspace_bytes(qll.QLL_OP_GEMM_NT_BF16, 8, 4096, 4100) == 0   # k % 16 != 0: f32 path
    # f16 and f32 weights: a workspace holding the split activations and the
    # bf16 weight planes selects the bf16 matrix core (a smaller one or none:
    # widened on the f32 one, which no call here may reach: the pointers are
    # fake, so every call below must fail its host-side checks)
    planes = 2 * 4096 * 4096 * 2
    assert qll.qll_workspace_bytes(qll.QLL_OP_GEMM_NT_F16, 4096, 4096, 4096) == 8 * split_x + planes
    assert qll.qll_workspace_bytes(qll.QLL_OP_GEMM_NT_F16, 512, 4096, 4096) == split_x + planes + 4 * 512 * 4096 * 4
    assert qll.qll_workspace_bytes(qll.QLL_OP_GEMM_NT_F16, 1, 4096, 4096) == 0
    assert qll.qll_workspace_bytes(qll.QLL_OP_GEMM_NT_F16, 8, 4096, 4100) == 0
    assert qll.qll_workspace_bytes(qll.QLL_OP_GEMM_NT_F32, 4096, 4096, 4096) == 8 * split_x + 3 * 4096 * 4096 * 2


def test_repacked_sizes(L):
    L.qll_q4_0_repacked_bytes.restype = ctypes.c_size_t
    assert qll.qll_q4_0_repacked_bytes(1, 32) == 3328
    assert qll.qll_q4_0_repacked_bytes(129, 64) == 2 * 2 * 3328
    assert qll.qll_q4_0_repacked_bytes(128256, 4096) == 1002 * 128 * 3328
    assert qll.qll_q4_0_repacked_bytes(8, 48) == SIZE_MAX
    need = qll.qll_workspace_bytes(qll.QLL_OP_Q4_0_REPACKED_GEMM, 512, 4096, 4096)
    # at least the prepared activations: 6144 + 256 bytes per 128 rows and block
    assert need >= 4 * 128 * 6400
    assert qll.qll_workspace_bytes(qll.QLL_OP_Q4_0_REPACKED_GEMM, 1, 1, 32) > 0
    assert qll.qll_workspace_bytes(qll.QLL_OP_Q4_0_REPACKED_GEMM, 4, 8, 48) == SIZE_MAX


def test_sgemm_errors(L):
    assert L.qll_sgemm(NUL, GOOD, GOOD, 2, 2, 2, NUL, 0, None) == NULL
    assert L.qll_sgemm(GOOD, GOOD, GOOD, 2, 0, 2, NUL, 0, None) == SHAPE
    assert L.qll_sgemm(GOOD, GOOD, GOOD, 2 ** 30, 2 ** 30, 2, NUL, 0, None) == SHAPE
    assert L.qll_sgemm(GOOD, MIS, GOOD, 2, 2, 2, NUL, 0, None) == ALIGN
    need = qll.qll_workspace_bytes(qll.QLL_OP_SGEMM, 1, 4096, 4096)
    assert L.qll_sgemm(GOOD, GOOD, GOOD, 1, 4096, 4096, NUL, 0, None) == WORKSPACE
    assert L.qll_sgemm(GOOD, GOOD, GOOD, 1, 4096, 4096, GOOD, need - 1, None) == WORKSPACE
    # m > 1: a workspace of this size selects the bf16 matrix core
    need_core = qll.qll_workspace_bytes(qll.QLL_OP_SGEMM_BF16, 4096, 4096, 4096)
    assert need_core == 8 * (4 * 256 * 3 * 128 * 16 * 2) + 3 * 4096 * 4096 * 2
    assert L.qll_sgemm(GOOD, GOOD, GOOD, 4096, 4096, 4096, MIS, need_core, None) == ALIGN
    assert L.qll_sgemm(GOOD, GOOD, GOOD, 1, 4096, 4096, MIS, need, None) == ALIGN


def test_ternary_errors(L):
    f = ctypes.c_float(1.0)
    assert L.qll_quantize_i8_rows(GOOD, GOOD, NUL, GOOD, 1, 16, None) == NULL
    assert L.qll_quantize_i8_rows(GOOD, GOOD, GOOD, GOOD, 1, 0, None) == SHAPE
    assert L.qll_quantize_i8_rows(GOOD, GOOD, GOOD, MIS, 1, 16, None) == ALIGN
    assert L.qll_ternary_gemv(GOOD, f, GOOD, GOOD, NUL, GOOD, 4, 32, None) == NULL
    assert L.qll_ternary_gemv(GOOD, f, GOOD, GOOD, GOOD, GOOD, 4, 40, None) == SHAPE
    assert L.qll_ternary_gemv(GOOD, f, GOOD, GOOD, GOOD, GOOD, 4, 65536 + 16, None) == SHAPE
    assert L.qll_ternary_gemm(GOOD, f, GOOD, GOOD, GOOD, GOOD, 1, 4, 65536 + 16, None) == SHAPE  # m = 1: the GEMV
    assert L.qll_ternary_gemv(GOOD, f, MIS, GOOD, GOOD, GOOD, 4, 32, None) == ALIGN
    assert L.qll_ternary_gemm(GOOD, f, GOOD, GOOD, GOOD, NUL, 4, 4, 32, None) == NULL
    assert L.qll_ternary_gemm(GOOD, f, GOOD, GOOD, GOOD, GOOD, 4, 4, 8, None) == SHAPE
    assert L.qll_ternary_gemm(GOOD, f, GOOD, GOOD, GOOD, MIS, 4, 4, 32, None) == ALIGN


def test_python_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(64, dtype=torch.float32)
    with pytest.raises(ValueError, match="CUDA"):
        qll._ptr(x, 4, "x")
