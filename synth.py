"""Seeded synthetic inputs for the quantized linear layer.

This module holds none of the method's arithmetic: it only draws raw values
(4- and 8-bit codes, fp16 scales, ternary codes, f32 activations) from numpy's PCG64
generator in a fixed order.  Encoding them into Q4_0 blocks or packed ternary
words, and quantizing activations, is done separately by the HIP library
(on the device) and by the oracle (on the host), so both sides start from the
same raw draws and nothing else.

The shapes and value distributions follow the workloads of the pages: one
Q4_0 layer of 512x512, an f32 GEMM of 4096^3 with its m = 1 GEMV, a BitNet
ternary 2560 -> 6912 layer at m = 1 and m = 64, and the Q4_0 decode (m = 1)
and prefill (m = 512) linears of an 8B-class transformer, the same shapes
with Q8_0 weights.
"""
import numpy as np

# (k, n) of the 8B-class linear shapes: up/gate, down, attention, vocab.
SHAPES_8B = ((4096, 14336), (14336, 4096), (4096, 4096), (4096, 128256))

SEED_Q4_SMALL = 1001
SEED_F32 = 1002
SEED_TERNARY = 1003
SEED_Q4_DECODE = 1004   # + shape index
SEED_Q4_PREFILL_X = 2004  # + shape index
SEED_Q8W_DECODE = 3004    # + shape index: Q8_0 weights of the same shapes


def q4_0_weights(rng, n, k):
    """Raw Q4_0 draws: codes uint8[n][k] uniform in [0, 15] and fp16 scales
    ~ U(0.001, 0.01) (f64 -> f32 -> f16, round to nearest even) as uint16 bits
    [n][k/32]."""
    assert k % 32 == 0
    codes = rng.integers(0, 16, size=(n, k // 32, 32), dtype=np.uint8).reshape(n, k)
    d = rng.uniform(0.001, 0.01, size=(n, k // 32)).astype(np.float32).astype(np.float16)
    return codes, d.view(np.uint16)


def q8_0_weights(rng, n, k):
    """Raw Q8_0 weight draws: codes int8[n][k] uniform in [-127, 127] (the
    range the Q8_0 quantizer produces) and fp16 scales ~ U(0.001, 0.01) as
    uint16 bits [n][k/32]."""
    assert k % 32 == 0
    codes = rng.integers(-127, 128, size=(n, k // 32, 32), dtype=np.int16).astype(np.int8).reshape(n, k)
    d = rng.uniform(0.001, 0.01, size=(n, k // 32)).astype(np.float32).astype(np.float16)
    return codes, d.view(np.uint16)


def normal_f32(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32)


def uniform_f32(rng, shape, lo=-1.0, hi=1.0):
    return rng.uniform(lo, hi, size=shape).astype(np.float32)


def ternary_codes(rng, n, k):
    """Ternary codes uint8[n][k] uniform over {0, 1, 2} (weight = code - 1)."""
    return rng.integers(0, 3, size=(n, k), dtype=np.uint8)


# ---------------------------------------------------------------- workloads

def q4_small(seed=SEED_Q4_SMALL, n=512, k=512, m=1):
    """Q4_0 x Q8_0 GEMV 512x512: codes, fp16 scales, then x ~ N(0,1)."""
    rng = np.random.default_rng(seed)
    codes, d_bits = q4_0_weights(rng, n, k)
    x = normal_f32(rng, (m, k))
    return codes, d_bits, x


def f32_gemm(seed=SEED_F32, m=4096, n=4096, k=4096):
    """f32 GEMM C = A.B with A, B ~ U(-1, 1), row-major; then the m = 1 GEMV
    activation x ~ U(-1, 1) of length k drawn after A and B."""
    rng = np.random.default_rng(seed)
    a = uniform_f32(rng, (m, k))
    b = uniform_f32(rng, (k, n))
    x = uniform_f32(rng, (1, k))
    return a, b, x


def ternary_layer(seed=SEED_TERNARY, n=6912, k=2560, m=64):
    """BitNet layer: codes, one absmean-style f32 scale ~ U(0.01, 0.1), then
    x ~ N(0,1) of m rows (the m = 1 case uses row 0)."""
    rng = np.random.default_rng(seed)
    codes = ternary_codes(rng, n, k)
    w_scale = np.float32(rng.uniform(0.01, 0.1))
    x = normal_f32(rng, (m, k))
    return codes, w_scale, x


def q4_decode(shape_index, k=None, n=None):
    """8B-class Q4_0 decode layer number `shape_index`: W draws then x (m = 1)."""
    k0, n0 = SHAPES_8B[shape_index]
    k = k or k0
    n = n or n0
    rng = np.random.default_rng(SEED_Q4_DECODE + shape_index)
    codes, d_bits = q4_0_weights(rng, n, k)
    x = normal_f32(rng, (1, k))
    return codes, d_bits, x


def q4_prefill_x(shape_index, m=512, k=None):
    """Prefill activations for 8B-class shape `shape_index` (the weights are
    those of q4_decode with the same index): x ~ N(0,1) of m rows."""
    k = k or SHAPES_8B[shape_index][0]
    rng = np.random.default_rng(SEED_Q4_PREFILL_X + shape_index)
    return normal_f32(rng, (m, k))


def q8w_decode(shape_index, k=None, n=None):
    """8B-class layer number `shape_index` with Q8_0 weights: W draws then x
    (m = 1); the prefill activations are those of q4_prefill_x."""
    k0, n0 = SHAPES_8B[shape_index]
    k = k or k0
    n = n or n0
    rng = np.random.default_rng(SEED_Q8W_DECODE + shape_index)
    codes, d_bits = q8_0_weights(rng, n, k)
    x = normal_f32(rng, (1, k))
    return codes, d_bits, x
