"""Parity of the int8 matrix-core small-m kernel (the Q4_0 x Q8_0 GEMM entry
at 2 <= m <= 32) against the oracle.  The shapes drive every split of a row
tile's blocks over its waves (1, 2, 4 and 8 waves; at most 4 with 32 staged
activation rows) with each staged activation tile height (4, 8, 16 and 32
rows), the workgroups that share activation stages on tall matrices, ragged last row tiles,
ragged last stages, and rows of fewer than eight blocks (run by the
GEMV-style kernel in groups of eight activation rows).  Float outputs within
1e-4 * sum_b |term_b|; with unit scales every output is an integer below
2^24, exact in any summation order, and must match bit for bit."""
import numpy as np
import pytest

import oracle as O
import quantized_linear_layer_amd as qll
import synth
from gpu_util import assert_within, host, pack_q4_0, q4_gemm, quantize_q8_0

pytestmark = pytest.mark.gpu
TOL = 1e-4

# (m, n, k, (16-row weight tiles per wave, waves per row tile), or "shared":
# workgroups sharing activation stages; None: rows under eight blocks, which
# run the GEMV-style kernel by groups of eight activation rows)
CASES = [
    (2, 33, 4096, (1, 8)),        # few row tiles: the widest split; ragged last tile
    (5, 33, 4096, (1, 8)),
    (16, 17, 4128, (1, 8)),       # 129 blocks
    (8, 257, 14336, (1, 8)),
    (4, 2000, 2048, (1, 4)),
    (3, 33, 512, (1, 1)),
    (7, 33, 512, (1, 1)),
    (16, 14336, 4096, (1, 2)),    # the 8B-class up projection
    (9, 9000, 1024, (1, 2)),
    (3, 20001, 256, (1, 1)),      # one stage
    (3, 9000, 1024, (1, 2)),
    (6, 2000, 2048, (1, 4)),
    (7, 9000, 1024, (1, 2)),
    (8, 70001, 512, "shared"),
    (12, 129, 608, (1, 1)),       # 19 blocks: a last stage that starts inside the one before
    (12, 20001, 1056, (1, 2)),
    (32, 1000, 2048, (1, 4)),     # 32-row activation tiles
    (24, 8001, 1056, (1, 2)),     # 33 blocks
    (20, 70000, 512, "shared"),
    (17, 20001, 2048, (2, 1)),
    (12, 129, 256, (1, 1)),       # eight blocks: one stage
    (13, 33, 2048, (1, 4)),
    (4, 20001, 1024, (1, 2)),
    (7, 32768, 1024, "shared"),
    (13, 32768, 256, "shared"),
    (13, 32768, 1024, "shared"),
    (9, 32808, 1056, "shared"),   # a last workgroup with waves wholly past n; 33 blocks
    (17, 40001, 4128, "shared"),  # 129 blocks
    (29, 33, 256, (1, 1)),
    (29, 9000, 1024, (2, 2)),
    (32, 9, 32, None),            # one block
    (31, 3, 96, None),
    (12, 129, 224, None),         # seven blocks
]


def _split(m, n, k):
    # the launcher's choices (q4_small_mfma.hip).  From n = 32768 at m > 4:
    # "shared", workgroups of four waves of two 16-row weight tiles sharing
    # each activation stage.  Otherwise (16-row weight tiles per wave, waves
    # per row tile): two tiles from n = 8192 at m > 16, else one; waves per
    # row tile the largest split, at most 8 (2 with two-tile waves), whose
    # workgroups all fit on the 256 CUs at once (160 KB of LDS each; a wave
    # holds two stage buffers of 3 or 5 KB of weight rows and 2, 3, 5 or 9
    # KB for 4, 8, 16 or 32 staged activation rows) and that leaves each
    # wave two eight-block stages.  None where the row has fewer than eight
    # blocks.
    if k < 256:
        return None
    if n >= 32768 and m > 4:
        return "shared"
    rt = 2 if n >= 8192 and m > 16 else 1
    mp = 4 if m <= 4 else 8 if m <= 8 else 16 if m <= 16 else 32
    per_wave = 2 * 1024 * ({1: 3, 2: 5}[rt] + {4: 2, 8: 3, 16: 5, 32: 9}[mp])
    tiles, nst = -(-n // (16 * rt)), -(-(k // 32) // 8)
    for ks in ((2,) if rt == 2 else (8, 4, 2)):
        if nst >= 2 * ks and tiles <= 256 * (160 * 1024 // (ks * per_wave)):
            return (rt, ks)
    return (rt, 1)


def _case(seed, m, n, k):
    rng = np.random.default_rng(seed)
    codes, d_bits = synth.q4_0_weights(rng, n, k)
    x = synth.normal_f32(rng, (m, k))
    return codes, d_bits, x


@pytest.mark.parametrize("m,n,k,ks", CASES)
def test_small_m_mfma_shapes(qll_gpu, m, n, k, ks):
    assert _split(m, n, k) == ks  # the case covers the tiling and split it is listed for
    # and reaches this kernel (the GEMM entry keeps the GEMV-style kernel at
    # m = 2 from n = 8192 and at m <= 4 from n = 32768)
    assert ks is None or not ((m == 2 and n >= 8192) or (m <= 4 and n >= 32768))
    codes, d_bits, x = _case(m * 1009 + n * 7 + k, m, n, k)
    y = host(q4_gemm(pack_q4_0(codes, d_bits), quantize_q8_0(x), m, n, k)).reshape(m, n)
    y_ref, mag = O.q4_0_q8_0(O.pack_q4_0(codes, d_bits), O.quantize_q8_0(x), m, n, k)
    assert_within(y, y_ref, mag, TOL, f"small-m MFMA m={m} n={n} k={k}")


def _int_reference(xq, codes, m, n, k):
    # y = sum over blocks of (q_w - 8) . q_x with every scale 1, in int64
    qx = np.frombuffer(xq, np.uint8).reshape(m, k // 32, 34)[:, :, 2:].view(np.int8).reshape(m, k).astype(np.int64)
    return qx @ (codes.astype(np.int64) - 8).T


@pytest.mark.parametrize("m,n,k", [(16, 40, 14336), (32, 33, 4096), (7, 1000, 96), (20, 17, 4128)])
def test_small_m_mfma_unit_scales_bit_exact(qll_gpu, m, n, k):
    rng = np.random.default_rng(m * 3 + n + k)
    codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
    d_bits = np.full((n, k // 32), 0x3c00, np.uint16)
    x = rng.integers(-126, 127, (m, k)).astype(np.float32)
    x[:, ::32] = np.where(rng.random((m, k // 32)) < 0.5, 127.0, -127.0)  # d_x = 1 in every block
    xq = O.quantize_q8_0(x)
    want = _int_reference(xq, codes, m, n, k)
    assert np.abs(want).max() < 2 ** 24
    y = host(q4_gemm(pack_q4_0(codes, d_bits), quantize_q8_0(x), m, n, k)).reshape(m, n)
    assert np.array_equal(y.astype(np.float64), want.astype(np.float64))


def test_small_m_mfma_one_hot(qll_gpu):
    # activation row i is 127 at position p_i and 0 elsewhere: y[i, j] =
    # d_w[j, p_i / 32] * (code[j, p_i] - 8) * 127 exactly (d_x = 1)
    m, n, k = 32, 70, 1024
    rng = np.random.default_rng(5)
    codes, d_bits = synth.q4_0_weights(rng, n, k)
    pos = rng.choice(k, m, replace=False)
    x = np.zeros((m, k), np.float32)
    x[np.arange(m), pos] = 127.0
    y = host(q4_gemm(pack_q4_0(codes, d_bits), quantize_q8_0(x), m, n, k)).reshape(m, n)
    dw = d_bits.view(np.float16).astype(np.float64)
    want = dw[:, pos // 32].T * (codes[:, pos].T.astype(np.float64) - 8.0) * 127.0
    assert np.array_equal(y.astype(np.float64), want)


# 33 <= m <= 64: groups of at most 32 activation rows,
# a last group of one row on the GEMV, of 2..8 rows on the small-m kernels,
# rows of fewer than eight blocks on the GEMV-style kernel by eights
@pytest.mark.parametrize("m,n,k", [(33, 300, 4096), (40, 1000, 1056), (64, 17, 14336), (48, 40000, 512),
                                   (37, 129, 96), (57, 14336, 4096), (64, 40000, 1056), (49, 32769, 256)])
def test_small_m_groups(qll_gpu, m, n, k):
    assert qll.qll_workspace_bytes(qll.QLL_OP_Q4_0_Q8_0_GEMM, m, n, k) == 0  # the small-m path
    codes, d_bits, x = _case(m * 3 + n + k, m, n, k)
    y = host(q4_gemm(pack_q4_0(codes, d_bits), quantize_q8_0(x), m, n, k)).reshape(m, n)
    y_ref, mag = O.q4_0_q8_0(O.pack_q4_0(codes, d_bits), O.quantize_q8_0(x), m, n, k)
    assert_within(y, y_ref, mag, TOL, f"small-m groups m={m} n={n} k={k}")


def test_small_m_mfma_deterministic(qll_gpu):
    m, n, k = 16, 300, 14336
    codes, d_bits, x = _case(77, m, n, k)
    w, xq = pack_q4_0(codes, d_bits), quantize_q8_0(x)
    y1, y2 = host(q4_gemm(w, xq, m, n, k)), host(q4_gemm(w, xq, m, n, k))
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
