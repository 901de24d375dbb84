"""Host-side pieces of bench.py that need no GPU: the Q8_0 weight records it
lays out itself must be the oracle's block_q8_0 bytes (the benchmark never
calls the oracle outside its cpu_baseline leg)."""
import numpy as np

import bench
import oracle as O
import synth


def test_q8_0_block_bytes_match_oracle_packing():
    rng = np.random.default_rng(11)
    for n, k in [(1, 32), (7, 96), (33, 4096)]:
        codes, d_bits = synth.q8_0_weights(rng, n, k)
        codes[0, 0] = -128
        assert np.array_equal(bench.q8_0_block_bytes(np, codes, d_bits), O.pack_q8_0(codes, d_bits).reshape(-1))


def test_gpus_above_one_exit_with_message(capsys):
    import sys
    argv = sys.argv
    sys.argv = ["bench.py", "--gpus", "2"]
    try:
        try:
            bench.main()
            raise AssertionError("bench.main() returned for --gpus 2")
        except SystemExit as e:
            assert e.code == 2
    finally:
        sys.argv = argv
    assert "one GPU" in capsys.readouterr().err


def test_host_cpus_counts_physical_cores():
    phys, logical, _ = bench.host_cpus()
    assert 1 <= phys <= logical


def test_r4_keeps_four_significant_digits():
    assert bench.r4(1234.5678) == 1235.0 and bench.r4(0.000123456) == 0.0001235 and bench.r4(None) is None
