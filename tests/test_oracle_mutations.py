"""Planted mistakes in the oracle must fail its pins (CPU only).

Each mutation below is a plausible slip in oracle.c (a dropped term, a wrong
sign, index or shift, a transposed operand, a wrong rounding rule).  The test
compiles a copy of oracle.c with that one change, runs every pin of pins.py
against it in a child process, and requires at least one pin to fail.  This
is the evidence that the pins pin the oracle, not just exercise it.

Two slips are deliberately absent because they are equivalent (no input can
tell them apart): loosening the early "a >= 65520" overflow test of the
binary16 conversion (the exponent check after rounding gives the same
infinity), and the +-127 clamps of the quantizers (|x/d| <= 127 (1 + 2^-23)
after the f32 division, so the clamps never act; they stay as a guard).
"""
import concurrent.futures as cf
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTATIONS = {
    # binary16
    "half_subnormal_scale": ("v = ldexp((double)f, -24);", "v = ldexp((double)f, -23);"),
    "half_exponent_bias": ("ldexp((double)(1024 + f), e - 25)", "ldexp((double)(1024 + f), e - 24)"),
    "half_ties_up": ("return (fmod(r, 2.0) == 0.0) ? r : r + 1.0;", "return r + 1.0;"),
    "half_overflow_edge": ("if (a >= 65520.0)", "if (a >= 65504.0)"),
    # Q4_0 format
    "q4_pack_high_shift": ("blk[2 + t] = (uint8_t)(c[t] | (c[t + 16] << 4));",
                           "blk[2 + t] = (uint8_t)(c[t] | (c[t + 16] << 3));"),
    "q4_unpack_swapped": ("c[t] = blk[2 + t] & 0x0f;\n                c[t + 16] = blk[2 + t] >> 4;",
                          "c[t] = blk[2 + t] >> 4;\n                c[t + 16] = blk[2 + t] & 0x0f;"),
    # Q8_0 quantizer
    "q8_scale_128": ("float d = amax / 127.0f;", "float d = amax / 128.0f;"),
    "q8_round_floor_half": ("float r = roundf(xb[t] / d);", "float r = floorf(xb[t] / d + 0.5f);"),
    "q8_round_even": ("float r = roundf(xb[t] / d);", "float r = rintf(xb[t] / d);"),
    "q8_quotient_f64": ("float r = roundf(xb[t] / d);", "float r = (float)round((double)xb[t] / (double)d);"),
    "q8_small_block_zeroed": ("if (d != 0.0f) {\n                    float r = roundf(xb[t] / d);",
                              "if (d > 1e-3f) {\n                    float r = roundf(xb[t] / d);"),
    # Q4_0 x Q8_0 dot
    "dot_nibble_order": ("int qw = wblk[2 + t] & 0x0f;\n        s += (qw - 8) * (int8_t)xblk[2 + t];\n    }\n"
                         "    for (int t = 16; t < 32; t++) {\n        int qw = wblk[2 + t - 16] >> 4;",
                         "int qw = wblk[2 + t] >> 4;\n        s += (qw - 8) * (int8_t)xblk[2 + t];\n    }\n"
                         "    for (int t = 16; t < 32; t++) {\n        int qw = wblk[2 + t - 16] & 0x0f;"),
    "dot_high_nibble_index": ("int qw = wblk[2 + t - 16] >> 4;", "int qw = wblk[2 + t - 15] >> 4;"),
    "dot_dropped_offset": ("int qw = wblk[2 + t] & 0x0f;\n        s += (qw - 8) * (int8_t)xblk[2 + t];",
                           "int qw = wblk[2 + t] & 0x0f;\n        s += qw * (int8_t)xblk[2 + t];"),
    "dot_offset_sign": ("int qw = wblk[2 + t - 16] >> 4;\n        s += (qw - 8) * (int8_t)xblk[2 + t];",
                        "int qw = wblk[2 + t - 16] >> 4;\n        s += (qw + 8) * (int8_t)xblk[2 + t];"),
    "dot_scale_dw_twice": ("double s = half[load_u16le(wb)] * half[load_u16le(xb)];",
                           "double s = half[load_u16le(wb)] * half[load_u16le(wb)];"),
    "dot_half_table": ("t[h] = orc_half_to_double((uint16_t)h);", "t[h] = orc_half_to_double((uint16_t)(h ^ 1));"),
    "dot_mag_signed": ("m += fabs(term);", "m += term;"),
    "dot_x_block_index": ("const uint8_t *xb = xrow + b * 34;", "const uint8_t *xb = xrow + (nb - 1 - b) * 34;"),
    # Q8_0 x Q8_0 dot
    "q8w_weight_unsigned": ("int qw = (int8_t)wblk[2 + t];", "int qw = wblk[2 + t];"),
    "q8w_weight_block_stride": ("const uint8_t *wblk = wrow + b * 34;", "const uint8_t *wblk = wrow + b * 32;"),
    "q8w_scale_dx_twice": ("double sc = orc_half_to_double(load_u16le(wblk)) * orc_half_to_double(load_u16le(xblk));",
                           "double sc = orc_half_to_double(load_u16le(xblk)) * orc_half_to_double(load_u16le(xblk));"),
    "q8w_mag_signed": ("sum_abs += fabs(term);", "sum_abs += term;"),
    "q8w_pack_d_big_endian": ("store_u16le(out, d_bits[j * nb + b]);",
                              "out[0] = (uint8_t)(d_bits[j * nb + b] >> 8); out[1] = (uint8_t)d_bits[j * nb + b];"),
    # NT GEMM, f32/bf16/f16 weights
    "nt_weight_index_nn": ("widen_weight(w, wtype, j * k + p, half)", "widen_weight(w, wtype, p * k + j, half)"),
    "nt_bf16_shift_15": ("uint32_t bits = (uint32_t)h << 16;", "uint32_t bits = (uint32_t)h << 15;"),
    "nt_f16_read_as_bf16": ("    return half[h];\n}", "    return (double)h;\n}"),
    "nt_mag_signed": ("sum_abs += fabs(prod);", "sum_abs += prod;"),
    # f32 GEMM
    "sgemm_b_column": ("double prod = (double)a[i * k + p] * (double)bt[j * k + p];",
                       "double prod = (double)a[i * k + p] * (double)bt[(j ^ 1) * k + p];"),
    "sgemm_a_column": ("double prod = (double)a[i * k + p] * (double)bt[j * k + p];",
                       "double prod = (double)a[i * k + (k - 1 - p)] * (double)bt[j * k + p];"),
    "sgemm_transpose_index": ("t[j * rows + p] = b[p * cols + j];", "t[j * rows + p] = b[j * cols + p];"),
    "sgemm_f32_accumulate": ("double acc = 0.0, m = 0.0;\n    for (int64_t p = 0; p < k; p++) {",
                             "float acc = 0.0f; double m = 0.0;\n    for (int64_t p = 0; p < k; p++) {"),
    # ternary
    "ternary_pack_msb_first": ("word |= (uint32_t)c << (2 * s);", "word |= (uint32_t)c << (30 - 2 * s);"),
    "ternary_dot_msb_first": ("int c = (int)((wrow[t / 16] >> (2 * (t % 16))) & 3u);",
                              "int c = (int)((wrow[t / 16] >> (30 - 2 * (t % 16))) & 3u);"),
    "ternary_identity_sign": ("int32_t dot = dot_c - asum;", "int32_t dot = dot_c + asum;"),
    "ternary_scale_multiplied": ("*y = (double)dot * (double)w_scale / (double)s;",
                                 "*y = (double)dot * (double)w_scale * (double)s;"),
    "i8_scale_inverted": ("float s = (amax == 0.0f) ? 0.0f : 127.0f / amax;",
                          "float s = (amax == 0.0f) ? 0.0f : amax / 127.0f;"),
    "i8_round_trunc": ("float r = roundf(xr[t] * s);", "float r = truncf(xr[t] * s);"),
    "i8_product_f64": ("float r = roundf(xr[t] * s);", "float r = (float)round((double)xr[t] * (double)s);"),
    "i8_sum_dropped": ("sum += v;", "sum += (v > 0) ? v : 0;"),
}

RUNNER = r"""
import sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle, pins
L = oracle.load({lib!r})
failed = []
for check in pins.ALL:
    try:
        check(L)
    except Exception as e:  # a failed assertion or an oracle error status
        failed.append(check.__name__)
print(",".join(failed))
"""


def _run_mutant(name, tmp):
    find, repl = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(find) == 1, f"mutation {name}: pattern not found exactly once"
    path = os.path.join(tmp, f"{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(find, repl))
    lib = os.path.join(tmp, f"lib{name}.so")
    subprocess.run(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-fopenmp", path,
                    "-o", lib, "-lm"], check=True)
    code = RUNNER.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300,
                       env=dict(os.environ, OMP_NUM_THREADS="2"))
    if r.returncode != 0:  # a crash also counts as caught, but say so
        return name, "crashed: " + r.stderr[-200:]
    return name, r.stdout.strip()


def test_every_mutation_is_caught():
    with tempfile.TemporaryDirectory() as tmp, cf.ThreadPoolExecutor(4) as ex:
        results = dict(ex.map(lambda n: _run_mutant(n, tmp), sorted(MUTATIONS)))
    survivors = [n for n, failed in results.items() if not failed]
    assert not survivors, f"mutations not caught by any pin: {survivors}"


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_pattern_present(name):
    assert open(SRC).read().count(MUTATIONS[name][0]) == 1
