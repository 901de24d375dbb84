"""Writes tests/golden/*.txt from the oracle only (never from the HIP path).

The pages print no worked numeric example for this path, so the stored values
here are regression anchors of the oracle on the small Q4_0 x Q8_0 layer
(512 x 512, seed 1001) and the hashes of the seeded generator's raw draws:
they make any later change of the oracle's arithmetic or of the generator
visible.  Run:  python tests/golden/make_golden.py
"""
import hashlib
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path[:0] = [os.path.dirname(os.path.dirname(HERE))]

import oracle  # noqa: E402
import synth  # noqa: E402


def draws_digest():
    codes, d_bits, x = synth.q4_small()
    tc, ws, tx = synth.ternary_layer(n=64, k=256, m=2)
    h = hashlib.sha256()
    for a in (codes, d_bits, x, tc, np.array([ws]), tx):
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def small_q4_outputs():
    codes, d_bits, x = synth.q4_small()
    w = oracle.pack_q4_0(codes, d_bits)
    xq = oracle.quantize_q8_0(x)
    y, mag = oracle.q4_0_q8_0(w, xq, 1, 512, 512)
    return xq, y[0], mag[0]


def main():
    xq, y, mag = small_q4_outputs()
    with open(os.path.join(HERE, "q4_small_512x512.txt"), "w") as f:
        f.write("# Oracle output of the Q4_0 x Q8_0 GEMV, n = k = 512, seed 1001 (synth.q4_small).\n")
        f.write("# Written by tests/golden/make_golden.py from oracle/ only.\n")
        f.write(f"# draws_sha256 {draws_digest()}\n")
        f.write(f"# xq_sha256 {hashlib.sha256(xq.tobytes()).hexdigest()}\n")
        f.write("# j  y_ref(f64 hex)  mag(f64 hex)\n")
        for j in range(y.size):
            f.write(f"{j} {float(y[j]).hex()} {float(mag[j]).hex()}\n")


if __name__ == "__main__":
    main()
