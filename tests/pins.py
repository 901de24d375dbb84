"""Pins of the oracle: checks against what the pages and the mathematics fix,
never against the oracle itself.  Each check takes a loaded oracle library
`L` (so that tests/test_oracle_mutations.py can run the same checks against
copies of the oracle with a planted mistake and see them fail).

Kinds of pin used (the pages print no worked numeric example for this path):
  * an independent library: numpy's IEEE binary16 conversion, numpy f64
    matmul on dequantized operands, numpy integer einsum;
  * closed forms: unit scales (the output is an integer), one-hot
    activations (the output is one weight times 127), identity matrices;
  * invariants: round trips of the byte formats, quantizer bounds,
    idempotence, the ternary identity;
  * special cases: exact ties, zero blocks, zero rows;
  * exact rational arithmetic (Python fractions): the quantizers' IEEE f32
    quotient and product, rounded to binary32 from the exact value, on inputs
    chosen so that this rounding lands on a .5 the exact value misses.
The byte layouts are built here with numpy from their definitions (Q4_0:
fp16 d little-endian then 16 bytes, low nibble = element t, high nibble =
element t + 16; Q8_0: fp16 d then 32 int8; ternary: code s at bits 2s).
"""
from fractions import Fraction

import numpy as np

import oracle as O

# --------------------------------------------------------------------------- helpers (numpy)


def np_pack_q4_0(codes, d_bits):
    n, k = codes.shape
    nb = k // 32
    c = codes.reshape(n, nb, 32).astype(np.uint8)
    blk = np.empty((n, nb, 18), np.uint8)
    blk[:, :, 0:2] = d_bits.astype("<u2").reshape(n, nb, 1).view(np.uint8)
    blk[:, :, 2:18] = c[:, :, :16] | (c[:, :, 16:] << 4)
    return blk.reshape(n, nb * 18)


def np_pack_q8_0(q, d_bits):
    m, k = q.shape
    nb = k // 32
    blk = np.empty((m, nb, 34), np.uint8)
    blk[:, :, 0:2] = d_bits.astype("<u2").reshape(m, nb, 1).view(np.uint8)
    blk[:, :, 2:34] = q.reshape(m, nb, 32).view(np.uint8)
    return blk.reshape(m, nb * 34)


def np_pack_ternary(codes):
    n, k = codes.shape
    c = codes.reshape(n, k // 16, 16).astype(np.uint64)
    shifts = (2 * np.arange(16, dtype=np.uint64))
    return (c << shifts).sum(axis=2).astype(np.uint32)


def np_half(d_bits):
    return d_bits.astype(np.uint16).view(np.float16).astype(np.float64)


def rne_binary32(r):
    """The binary32 value nearest to the rational r (ties to even), as a
    Fraction: 24 significant bits in the normal range, multiples of 2^-149
    below it (IEEE 754 round-to-nearest-even; overflow is not reached here)."""
    if r == 0:
        return Fraction(0)
    a = abs(r)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)  # 2^e <= a < 2^(e+1), or the subnormal range
    scale = Fraction(2) ** (23 - e)
    v = a * scale
    n = v.numerator // v.denominator
    rem = v - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return (Fraction(n) / scale) * (1 if r > 0 else -1)


def round_half_away(r):
    """Nearest integer to the rational r, halves away from zero."""
    a = abs(r)
    n = a.numerator // a.denominator
    if a - n >= Fraction(1, 2):
        n += 1
    return n if r >= 0 else -n


def _f32_tie_crossings(rng, count, quotient):
    """`count` (amax, [x...]) sets whose f32 step (x / d with d = f32(amax/127)
    when `quotient`, else x * s with s = f32(127/amax)) rounds onto k + 1/2
    while the exact value lies strictly below it, so rounding the exact value
    and rounding the f32 result give different codes."""
    out = []
    while len(out) < count:
        amax = np.float32(rng.uniform(0.5, 100.0))
        scale = rne_binary32(Fraction(float(amax)) / 127 if quotient else Fraction(127) / Fraction(float(amax)))
        xs = []
        while len(xs) < 31:
            k = int(rng.integers(0, 126))
            target = (k + Fraction(1, 2)) * scale if quotient else (k + Fraction(1, 2)) / scale
            x = Fraction(float(np.float32(float(target))))
            exact = x / scale if quotient else x * scale
            if abs(x) < Fraction(float(amax)) and round_half_away(exact) != round_half_away(rne_binary32(exact)):
                xs.append(float(x) * (1 if rng.integers(0, 2) else -1))
        out.append((amax, xs))
    return out


def rand_q4(rng, n, k):
    codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
    d = rng.uniform(0.001, 0.01, (n, k // 32)).astype(np.float32).astype(np.float16).view(np.uint16)
    return codes, d


def rand_q8(rng, m, k):
    q = rng.integers(-127, 128, (m, k), dtype=np.int64).astype(np.int8)
    d = rng.uniform(0.001, 0.05, (m, k // 32)).astype(np.float32).astype(np.float16).view(np.uint16)
    return q, d


# --------------------------------------------------------------------------- fp16


def check_half_to_double_exhaustive(L):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = O.half_to_double(bits, L=L)
    want = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def _edge_floats():
    vals = []
    # every half value, its neighbours in f32 and the exact midpoints between halves
    h = np.arange(0, 0x7c00, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    mids = (h[:-1] + h[1:]) / 2.0  # exact in f64; representable in f32 (needs <= 12 bits)
    vals.append(h.astype(np.float32))
    vals.append(mids.astype(np.float32))
    m32 = mids.astype(np.float32)
    vals.append(np.nextafter(m32, np.float32(np.inf)))
    vals.append(np.nextafter(m32, np.float32(0)))
    vals.append(np.array([65504, 65519.99, 65520, 65536, 1e30, np.inf, 2.0 ** -24, 2.0 ** -25,
                          2.0 ** -25 * 1.0000001, 2.0 ** -26, 1e-45, 0.0], np.float32))
    v = np.concatenate(vals)
    return np.concatenate([v, -v])


def check_float_to_half(L, n_random=2_000_000):
    rng = np.random.default_rng(7)
    rnd = rng.integers(0, 2 ** 32, n_random, dtype=np.uint64).astype(np.uint32).view(np.float32)
    x = np.concatenate([_edge_floats(), rnd, np.array([np.nan], np.float32)])
    got = O.float_to_half(x, L=L)
    with np.errstate(over="ignore", invalid="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    nan = np.isnan(x)
    gh = got.view(np.float16)
    assert np.all(np.isnan(gh[nan]))
    assert np.array_equal(got[~nan], want[~nan])


# --------------------------------------------------------------------------- Q4_0 / Q8_0 formats


def check_q4_0_pack_roundtrip(L):
    rng = np.random.default_rng(11)
    for n, k in ((1, 32), (3, 64), (7, 96), (5, 256)):
        codes, d = rand_q4(rng, n, k)
        w = O.pack_q4_0(codes, d, L=L)
        assert np.array_equal(w, np_pack_q4_0(codes, d))
        c2, d2 = O.unpack_q4_0(w, n, k, L=L)
        assert np.array_equal(c2, codes) and np.array_equal(d2, d)
        assert c2.max() <= 15


def check_q8_0_unpack(L):
    rng = np.random.default_rng(12)
    q, d = rand_q8(rng, 3, 128)
    q2, d2 = O.unpack_q8_0(np_pack_q8_0(q, d), 3, 128, L=L)
    assert np.array_equal(q2, q) and np.array_equal(d2, d)


def check_q8_0_quantize_ties(L):
    # A block holding 127.0 has amax = 127 so d = 127/127 = 1 exactly and
    # x/d = x: each value below is an exact tie or a near-tie.
    vals = [127.0, 0.5, -0.5, 2.5, -2.5, 126.5, -126.5, 1.5, -1.5, 0.49999997, -0.49999997,
            3.5000002, 0.0, -0.0, 64.0, -127.0]
    want = [127, 1, -1, 3, -3, 127, -127, 2, -2, 0, 0, 4, 0, 0, 64, -127]
    x = np.zeros((1, 32), np.float32)
    x[0, :len(vals)] = vals
    xq = O.quantize_q8_0(x, L=L)
    q, d = O.unpack_q8_0(xq, 1, 32, L=L)
    assert d[0, 0] == 0x3c00  # fp16 1.0
    assert q[0, :len(want)].tolist() == want
    assert np.all(q[0, len(want):] == 0)


def check_q8_0_quantize_invariants(L):
    rng = np.random.default_rng(13)
    x = rng.standard_normal((4, 512)).astype(np.float32)
    x[1, 64:96] = 0.0                      # an all-zero block
    x[2, 0:32] *= np.float32(1e-3)         # a small block
    x[3, 32:64] = -np.abs(x[3, 32:64])     # an all-negative block
    q, d = O.unpack_q8_0(O.quantize_q8_0(x, L=L), 4, 512, L=L)
    xb = x.reshape(4, 16, 32).astype(np.float64)
    qb = q.reshape(4, 16, 32).astype(np.int64)
    amax = np.abs(xb).max(axis=2)
    for i in range(4):
        for b in range(16):
            if amax[i, b] == 0:
                assert np.all(qb[i, b] == 0) and d[i, b] == 0
                continue
            # the element of largest magnitude maps to +-127 with its sign
            t = np.argmax(np.abs(xb[i, b]))
            assert qb[i, b, t] == np.sign(xb[i, b, t]) * 127
            assert np.abs(qb[i, b]).max() == 127
            # every code is the nearest integer to x / (amax/127): within 1/2
            # (tiny slack for the f32 rounding of d and of the quotient)
            dd = amax[i, b] / 127.0
            assert np.all(np.abs(xb[i, b] / dd - qb[i, b]) <= 0.5 + 1e-5)
            # signs agree
            assert np.all((qb[i, b] == 0) | (np.sign(qb[i, b]) == np.sign(xb[i, b])))
            # the stored scale is the nearest fp16 of amax/127
            assert abs(np_half(np.array([d[i, b]]))[0] - dd) <= max(dd * 2.0 ** -11, 2.0 ** -25) * 1.0001


def check_q8_0_quantize_f32_quotient(L):
    # The code is round-half-away of the IEEE f32 quotient x/d, d = f32(amax/127).
    # Each x below sits where that quotient rounds to k + 1/2 but the exact
    # x/d lies below it: f32 division gives k + 1, an exact (or f64) division
    # gives k.  The expected code is derived with exact rationals.
    rng = np.random.default_rng(15)
    sets = _f32_tie_crossings(rng, 6, quotient=True)
    x = np.zeros((1, 32 * len(sets)), np.float32)
    want = np.zeros(x.shape[1], np.int64)
    want_d = []
    for b, (amax, xs) in enumerate(sets):
        d = rne_binary32(Fraction(float(amax)) / 127)
        x[0, 32 * b] = -amax if b % 2 else amax
        x[0, 32 * b + 1:32 * b + 32] = xs
        for t in range(32):
            xt = Fraction(float(x[0, 32 * b + t]))
            want[32 * b + t] = max(-127, min(127, round_half_away(rne_binary32(xt / d))))
        want_d.append(np.float32(float(d)).astype(np.float16).view(np.uint16))
    q, dbits = O.unpack_q8_0(O.quantize_q8_0(x, L=L), 1, x.shape[1], L=L)
    assert np.array_equal(q[0].astype(np.int64), want)
    assert np.array_equal(dbits[0], np.array(want_d, np.uint16))


def check_q8_0_idempotent(L):
    # x = fp16(d) * q with some |q| = 127 quantizes back to the same q and d.
    rng = np.random.default_rng(14)
    q = rng.integers(-127, 128, (2, 64)).astype(np.int64)
    q[:, 0] = 127
    q[:, 32] = -127
    d = np.array([[0x2e66, 0x1c00], [0x3c00, 0x3555]], np.uint16)  # fp16 scales
    x = (np.repeat(np_half(d), 32, axis=1) * q).astype(np.float32)
    q2, d2 = O.unpack_q8_0(O.quantize_q8_0(x, L=L), 2, 64, L=L)
    assert np.array_equal(q2.astype(np.int64), q)
    assert np.array_equal(d2, d)


# --------------------------------------------------------------------------- Q4_0 x Q8_0


def check_q4_0_q8_0_brute_force(L):
    rng = np.random.default_rng(21)
    for m, n, k in ((1, 1, 32), (1, 64, 256), (3, 17, 96), (4, 33, 160)):
        codes, dw = rand_q4(rng, n, k)
        q, dx = rand_q8(rng, m, k)
        w = np_pack_q4_0(codes, dw)
        xq = np_pack_q8_0(q, dx)
        y, mag = O.q4_0_q8_0(w, xq, m, n, k, L=L)
        wf = np.repeat(np_half(dw), 32, axis=1) * (codes.astype(np.float64) - 8.0)
        xf = np.repeat(np_half(dx), 32, axis=1) * q.astype(np.float64)
        ybf = xf @ wf.T
        assert np.all(np.abs(y - ybf) <= 1e-12 * mag + 1e-300)
        # mag is the sum over blocks of |term_b|
        prod = xf[:, None, :] * wf[None, :, :]
        tb = prod.reshape(m, n, k // 32, 32).sum(axis=3)
        assert np.allclose(mag, np.abs(tb).sum(axis=2), rtol=1e-12, atol=0)
        # block sums are the exact integers sum_t (q - 8) * qx
        s = O.q4_0_q8_0_block_sums(w, xq, m, n, k, L=L)
        want = np.einsum("ibt,jbt->ijb", q.reshape(m, -1, 32).astype(np.int64),
                         codes.reshape(n, -1, 32).astype(np.int64) - 8)
        assert np.array_equal(s.astype(np.int64), want)
        # the sampled entry agrees bit for bit with the full one
        ii = rng.integers(0, m, 9)
        jj = rng.integers(0, n, 9)
        ys, ms = O.q4_0_q8_0_sampled(w, xq, m, n, k, ii, jj, L=L)
        assert np.array_equal(ys, y[ii, jj]) and np.array_equal(ms, mag[ii, jj])


def check_q4_0_q8_0_unit_scales(L):
    # dw = dx = 1: the output is exactly the integer sum of the block sums.
    rng = np.random.default_rng(22)
    m, n, k = 2, 9, 320
    codes = rng.integers(0, 16, (n, k), dtype=np.uint8)
    q = rng.integers(-127, 128, (m, k)).astype(np.int8)
    one = np.uint16(0x3c00)
    w = np_pack_q4_0(codes, np.full((n, k // 32), one))
    xq = np_pack_q8_0(q, np.full((m, k // 32), one))
    y, _ = O.q4_0_q8_0(w, xq, m, n, k, L=L)
    want = q.astype(np.int64) @ (codes.astype(np.int64) - 8).T
    assert np.array_equal(y, want.astype(np.float64))


def check_q4_0_q8_0_one_hot(L):
    # x = 0 except x_p = 127: block p//32 has d = 1 and q_p = 127, the other
    # blocks are zero, so y_j = dw[j, p//32] * (code[j, p] - 8) * 127.
    rng = np.random.default_rng(23)
    n, k = 5, 128
    codes, dw = rand_q4(rng, n, k)
    w = np_pack_q4_0(codes, dw)
    for p in list(range(32)) + [37, 64 + 15, 64 + 16, 127]:
        x = np.zeros((1, k), np.float32)
        x[0, p] = 127.0
        xq = O.quantize_q8_0(x, L=L)
        y, _ = O.q4_0_q8_0(w, xq, 1, n, k, L=L)
        want = np_half(dw[:, p // 32]) * (codes[:, p].astype(np.float64) - 8.0) * 127.0
        assert np.array_equal(y[0], want), p


def check_q4_0_q8_0_zero_cases(L):
    rng = np.random.default_rng(24)
    n, k = 4, 64
    codes, dw = rand_q4(rng, n, k)
    x = rng.standard_normal((1, k)).astype(np.float32)
    # all codes 8 -> every weight is 0
    w8 = np_pack_q4_0(np.full((n, k), 8, np.uint8), dw)
    y, mag = O.q4_0_q8_0(w8, O.quantize_q8_0(x, L=L), 1, n, k, L=L)
    assert np.all(y == 0) and np.all(mag == 0)
    # x = 0 -> d = 0, q = 0
    y, mag = O.q4_0_q8_0(np_pack_q4_0(codes, dw), O.quantize_q8_0(np.zeros((1, k), np.float32), L=L),
                         1, n, k, L=L)
    assert np.all(y == 0) and np.all(mag == 0)


# --------------------------------------------------------------------------- Q8_0 x Q8_0


def check_q8_0_pack(L):
    rng = np.random.default_rng(41)
    for n, k in ((1, 32), (5, 96), (3, 320)):
        q, d = rand_q8(rng, n, k)
        q[0, 0] = -128  # the full int8 range is a valid weight code
        w = O.pack_q8_0(q, d, L=L)
        assert np.array_equal(w, np_pack_q8_0(q, d))
        q2, d2 = O.unpack_q8_0(w, n, k, L=L)
        assert np.array_equal(q2, q) and np.array_equal(d2, d)


def check_q8_0_q8_0_brute_force(L):
    rng = np.random.default_rng(42)
    for m, n, k in ((1, 1, 32), (1, 40, 256), (3, 17, 96), (4, 9, 160)):
        qw, dw = rand_q8(rng, n, k)
        qw[rng.random((n, k)) < 0.02] = -128
        q, dx = rand_q8(rng, m, k)
        w = np_pack_q8_0(qw, dw)
        xq = np_pack_q8_0(q, dx)
        y, mag = O.q8_0_q8_0(w, xq, m, n, k, L=L)
        wf = np.repeat(np_half(dw), 32, axis=1) * qw.astype(np.float64)
        xf = np.repeat(np_half(dx), 32, axis=1) * q.astype(np.float64)
        assert np.all(np.abs(y - xf @ wf.T) <= 1e-12 * mag + 1e-300)
        prod = xf[:, None, :] * wf[None, :, :]
        tb = prod.reshape(m, n, k // 32, 32).sum(axis=3)
        assert np.allclose(mag, np.abs(tb).sum(axis=2), rtol=1e-12, atol=0)
        s = O.q8_0_q8_0_block_sums(w, xq, m, n, k, L=L)
        want = np.einsum("ibt,jbt->ijb", q.reshape(m, -1, 32).astype(np.int64),
                         qw.reshape(n, -1, 32).astype(np.int64))
        assert np.array_equal(s.astype(np.int64), want)
        ii = rng.integers(0, m, 9)
        jj = rng.integers(0, n, 9)
        ys, ms = O.q8_0_q8_0_sampled(w, xq, m, n, k, ii, jj, L=L)
        assert np.array_equal(ys, y[ii, jj]) and np.array_equal(ms, mag[ii, jj])


def check_q8_0_q8_0_unit_scales(L):
    # dw = dx = 1: the output is exactly the integer dot product, including the
    # extreme codes -128 and 127 on the weight side
    rng = np.random.default_rng(43)
    m, n, k = 3, 7, 256
    qw = rng.integers(-128, 128, (n, k)).astype(np.int8)
    qw[0, :32] = -128
    qw[1, :32] = 127
    q = rng.integers(-127, 128, (m, k)).astype(np.int8)
    one = np.uint16(0x3c00)
    y, _ = O.q8_0_q8_0(np_pack_q8_0(qw, np.full((n, k // 32), one)), np_pack_q8_0(q, np.full((m, k // 32), one)),
                       m, n, k, L=L)
    assert np.array_equal(y, (q.astype(np.int64) @ qw.astype(np.int64).T).astype(np.float64))


def check_q8_0_q8_0_one_hot(L):
    # x_p = 127 alone: y_j = dw[j, p//32] * qw[j, p] * 127
    rng = np.random.default_rng(44)
    n, k = 6, 128
    qw, dw = rand_q8(rng, n, k)
    w = np_pack_q8_0(qw, dw)
    for p in (0, 1, 31, 32, 77, 127):
        x = np.zeros((1, k), np.float32)
        x[0, p] = 127.0
        y, _ = O.q8_0_q8_0(w, O.quantize_q8_0(x, L=L), 1, n, k, L=L)
        want = np_half(dw[:, p // 32]) * qw[:, p].astype(np.float64) * 127.0
        assert np.array_equal(y[0], want), p


# --------------------------------------------------------------------------- f32 GEMM


def check_sgemm_numpy(L):
    rng = np.random.default_rng(31)
    for m, n, k in ((1, 1, 1), (7, 11, 13), (33, 17, 23), (48, 192, 128), (1, 40, 300)):
        a = rng.uniform(-1, 1, (m, k)).astype(np.float32)
        b = rng.uniform(-1, 1, (k, n)).astype(np.float32)
        c, mag = O.sgemm(a, b, L=L)
        a64, b64 = a.astype(np.float64), b.astype(np.float64)
        assert np.all(np.abs(c - a64 @ b64) <= 1e-12 * mag)
        assert np.allclose(mag, np.abs(a64) @ np.abs(b64), rtol=1e-12, atol=0)
        ii = rng.integers(0, m, 5)
        jj = rng.integers(0, n, 5)
        cs, ms = O.sgemm_sampled(a, b, ii, jj, L=L)
        assert np.array_equal(cs, c[ii, jj]) and np.array_equal(ms, mag[ii, jj])


def check_sgemm_exact(L):
    rng = np.random.default_rng(32)
    a = rng.uniform(-1, 1, (9, 13)).astype(np.float32)
    c, _ = O.sgemm(a, np.eye(13, dtype=np.float32), L=L)
    assert np.array_equal(c, a.astype(np.float64))
    ai = rng.integers(-2, 3, (6, 21)).astype(np.float32)
    bi = rng.integers(-2, 3, (21, 10)).astype(np.float32)
    c, _ = O.sgemm(ai, bi, L=L)
    assert np.array_equal(c, (ai.astype(np.int64) @ bi.astype(np.int64)).astype(np.float64))
    c, _ = O.sgemm(np.ones((3, 37), np.float32), np.ones((37, 5), np.float32), L=L)
    assert np.all(c == 37.0)


# --------------------------------------------------------------------------- NT GEMM


def np_bf16_widen(bits):
    # bf16 is the upper half of an IEEE f32 (NaN patterns stay NaN)
    with np.errstate(invalid="ignore"):
        return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def np_f16_widen(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def _rand_w(rng, n, k, wdtype):
    w32 = rng.uniform(-1, 1, (n, k)).astype(np.float32)
    if wdtype == "f32":
        return w32, w32.astype(np.float64)
    if wdtype == "bf16":
        bits = (w32.view(np.uint32) >> 16).astype(np.uint16)  # truncation: any bf16 pattern will do
        return bits, np_bf16_widen(bits)
    bits = w32.astype(np.float16).view(np.uint16)
    return bits, np_f16_widen(bits)


def check_gemm_nt_numpy(L):
    rng = np.random.default_rng(51)
    for wdtype in ("f32", "bf16", "f16"):
        for m, n, k in ((1, 1, 1), (1, 37, 300), (7, 11, 13), (33, 17, 96)):
            a = rng.uniform(-1, 1, (m, k)).astype(np.float32)
            w, w64 = _rand_w(rng, n, k, wdtype)
            c, mag = O.gemm_nt(a, w, wdtype, L=L)
            a64 = a.astype(np.float64)
            assert np.all(np.abs(c - a64 @ w64.T) <= 1e-12 * mag), wdtype
            assert np.allclose(mag, np.abs(a64) @ np.abs(w64).T, rtol=1e-12, atol=0)
            ii = rng.integers(0, m, 5)
            jj = rng.integers(0, n, 5)
            cs, ms = O.gemm_nt_sampled(a, w, wdtype, ii, jj, L=L)
            assert np.array_equal(cs, c[ii, jj]) and np.array_equal(ms, mag[ii, jj])


def check_gemm_nt_exact(L):
    # identity weights give A back; small integers give exact integer products;
    # NT with W equals NN with W^T (the plain orientation's oracle)
    rng = np.random.default_rng(52)
    a = rng.uniform(-1, 1, (5, 24)).astype(np.float32)
    eye = np.eye(24, dtype=np.float32)
    for wdtype, w in (("f32", eye), ("bf16", (eye.view(np.uint32) >> 16).astype(np.uint16)),
                      ("f16", eye.astype(np.float16).view(np.uint16))):
        c, _ = O.gemm_nt(a, w, wdtype, L=L)
        assert np.array_equal(c, a.astype(np.float64)), wdtype
    ai = rng.integers(-3, 4, (6, 40)).astype(np.float32)
    wi = rng.integers(-3, 4, (9, 40)).astype(np.float32)
    want = (ai.astype(np.int64) @ wi.astype(np.int64).T).astype(np.float64)
    for wdtype, w in (("f32", wi), ("bf16", (wi.view(np.uint32) >> 16).astype(np.uint16)),
                      ("f16", wi.astype(np.float16).view(np.uint16))):
        c, _ = O.gemm_nt(ai, w, wdtype, L=L)
        assert np.array_equal(c, want), wdtype
    # the same products in the same p order as the plain orientation with B = W^T
    a2 = rng.uniform(-1, 1, (5, 30)).astype(np.float32)
    b = rng.uniform(-1, 1, (30, 12)).astype(np.float32)
    c_nt, m_nt = O.gemm_nt(a2, np.ascontiguousarray(b.T), "f32", L=L)
    c_nn, m_nn = O.sgemm(a2, b, L=L)
    assert np.array_equal(c_nt, c_nn) and np.array_equal(m_nt, m_nn)


def check_gemm_nt_bf16_f16_widening(L):
    # every bf16 and f16 bit pattern that is finite, one weight at a time:
    # x = [1, 0, ...] picks w[j][0], so C[0][j] must be the exact widening
    for wdtype, widen in (("bf16", np_bf16_widen), ("f16", np_f16_widen)):
        bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
        vals = widen(bits)
        keep = np.isfinite(vals)
        wcol = bits[keep]
        w = np.zeros((wcol.size, 2), np.uint16)
        w[:, 0] = wcol
        a = np.array([[1.0, 0.0]], np.float32)
        c, _ = O.gemm_nt(a, w, wdtype, L=L)
        assert np.array_equal(c[0], vals[keep]), wdtype


# --------------------------------------------------------------------------- ternary


def check_ternary_pack_roundtrip(L):
    rng = np.random.default_rng(41)
    for n, k in ((1, 16), (3, 48), (7, 160)):
        codes = rng.integers(0, 3, (n, k), dtype=np.uint8)
        words = O.pack_ternary(codes, L=L)
        assert np.array_equal(words, np_pack_ternary(codes))
        back = O.unpack_ternary(words, n, k, L=L)
        assert np.array_equal(back, codes) and back.max() <= 2


def check_quantize_i8_rows(L):
    rng = np.random.default_rng(42)
    x = rng.standard_normal((3, 160)).astype(np.float32)
    x[1] = 0.0
    q, s, t = O.quantize_i8_rows(x, L=L)
    assert s[1] == 0 and t[1] == 0 and np.all(q[1] == 0)
    for i in (0, 2):
        amax = np.abs(x[i].astype(np.float64)).max()
        assert abs(float(s[i]) - 127.0 / amax) <= 127.0 / amax * 2.0 ** -23
        j = np.argmax(np.abs(x[i]))
        assert q[i, j] == np.sign(x[i, j]) * 127
        assert np.all(np.abs(x[i].astype(np.float64) * (127.0 / amax) - q[i]) <= 0.5 + 1e-4)
        assert t[i] == int(q[i].astype(np.int64).sum())
    # exact ties with act_scale = 1 (the row holds 127.0)
    xt = np.zeros((1, 16), np.float32)
    xt[0, :8] = [127.0, 0.5, -0.5, 2.5, -2.5, 126.5, -126.5, -127.0]
    q, s, t = O.quantize_i8_rows(xt, L=L)
    assert s[0] == 1.0
    assert q[0, :8].tolist() == [127, 1, -1, 3, -3, 127, -127, -127]
    assert t[0] == 127 + 1 - 1 + 3 - 3 + 127 - 127 - 127


def check_quantize_i8_rows_f32_product(L):
    # q = round-half-away of the IEEE f32 product x*s, s = f32(127/amax).
    # Each x below makes that product round to k + 1/2 while the exact x*s
    # lies below it (f32: k + 1, exact or f64: k).  Expected values from
    # exact rationals.
    rng = np.random.default_rng(16)
    sets = _f32_tie_crossings(rng, 4, quotient=False)
    x = np.zeros((len(sets), 48), np.float32)
    for i, (amax, xs) in enumerate(sets):
        x[i, 5] = -amax if i % 2 else amax
        x[i, 6:37] = xs
    q, s, t = O.quantize_i8_rows(x, L=L)
    for i, (amax, _) in enumerate(sets):
        sc = rne_binary32(Fraction(127) / Fraction(float(amax)))
        want = [max(-127, min(127, round_half_away(rne_binary32(Fraction(float(v)) * sc)))) for v in x[i]]
        assert Fraction(float(s[i])) == sc
        assert q[i].astype(np.int64).tolist() == want
        assert int(t[i]) == sum(want)


def check_ternary_brute_force(L):
    rng = np.random.default_rng(43)
    for m, n, k in ((1, 1, 16), (1, 37, 160), (5, 19, 64)):
        codes = rng.integers(0, 3, (n, k), dtype=np.uint8)
        x = rng.standard_normal((m, k)).astype(np.float32)
        w_scale = np.float32(0.0421)
        q, s, t = O.quantize_i8_rows(x, L=L)
        words = np_pack_ternary(codes)
        y, mag, dots = O.ternary(words, w_scale, q, s, t, n, k, with_dots=True, L=L)
        wt = codes.astype(np.int64) - 1
        want_dot = q.astype(np.int64) @ wt.T
        assert np.array_equal(dots.astype(np.int64), want_dot)
        ybf = want_dot.astype(np.float64) * float(w_scale) / s.astype(np.float64)[:, None]
        assert np.all(np.abs(y - ybf) <= 1e-12 * mag)
        magbf = (np.abs(q.astype(np.int64)) @ np.abs(wt).T) * float(w_scale) / s.astype(np.float64)[:, None]
        assert np.allclose(mag, magbf, rtol=1e-12, atol=0)
        ii = rng.integers(0, m, 6)
        jj = rng.integers(0, n, 6)
        ys, ms = O.ternary_sampled(words, w_scale, q, s, t, n, k, ii, jj, L=L)
        assert np.array_equal(ys, y[ii, jj]) and np.array_equal(ms, mag[ii, jj])


def check_ternary_one_hot_and_unit(L):
    rng = np.random.default_rng(44)
    n, k = 6, 64
    codes = rng.integers(0, 3, (n, k), dtype=np.uint8)
    words = np_pack_ternary(codes)
    for p in list(range(16)) + [17, 40, 63]:
        x = np.zeros((1, k), np.float32)
        x[0, p] = 127.0
        q, s, t = O.quantize_i8_rows(x, L=L)
        assert s[0] == 1.0 and t[0] == 127
        y, _ = O.ternary(words, np.float32(1.0), q, s, t, n, k, L=L)
        assert np.array_equal(y[0], 127.0 * (codes[:, p].astype(np.float64) - 1.0)), p
    # unit scale: integer-valued x with max |x| = 127 -> act_scale = 1, y = dot
    xi = rng.integers(-127, 128, (2, k)).astype(np.float32)
    xi[:, 3] = 127.0
    q, s, t = O.quantize_i8_rows(xi, L=L)
    assert np.all(s == 1.0) and np.array_equal(q.astype(np.float32), xi)
    y, _ = O.ternary(words, np.float32(1.0), q, s, t, n, k, L=L)
    assert np.array_equal(y, (xi.astype(np.int64) @ (codes.astype(np.int64) - 1).T).astype(np.float64))
    # a zero row gives exactly zero
    q, s, t = O.quantize_i8_rows(np.zeros((1, k), np.float32), L=L)
    y, mag = O.ternary(words, np.float32(0.5), q, s, t, n, k, L=L)
    assert np.all(y == 0) and np.all(mag == 0)


def check_ternary_rejects_code_3(L):
    words = np.array([[3]], np.uint32)  # code 3 at position 0
    q = np.ones((1, 16), np.int8)
    try:
        O.ternary(words, np.float32(1.0), q, np.ones(1, np.float32), np.array([16], np.int32), 1, 16, L=L)
    except O.OracleError:
        return
    raise AssertionError("code 3 accepted")


ALL = [v for k, v in sorted(globals().items()) if k.startswith("check_")]
