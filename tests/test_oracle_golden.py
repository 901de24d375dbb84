"""The oracle still reproduces its stored regression anchor (CPU only)."""
import hashlib
import os

import numpy as np

import oracle
import synth

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load():
    meta, rows = {}, []
    for line in open(os.path.join(HERE, "q4_small_512x512.txt")):
        if line.startswith("# draws_sha256") or line.startswith("# xq_sha256"):
            k, v = line[2:].split()
            meta[k] = v
        elif not line.startswith("#"):
            j, y, mag = line.split()
            rows.append((int(j), float.fromhex(y), float.fromhex(mag)))
    return meta, rows


def test_generator_draws_are_stable():
    import make_golden
    meta, _ = _load()
    assert make_golden.draws_digest() == meta["draws_sha256"]


def test_oracle_matches_anchor():
    import make_golden
    meta, rows = _load()
    xq, y, mag = make_golden.small_q4_outputs()
    assert hashlib.sha256(xq.tobytes()).hexdigest() == meta["xq_sha256"]
    assert np.array_equal(y, np.array([r[1] for r in rows]))
    assert np.array_equal(mag, np.array([r[2] for r in rows]))
