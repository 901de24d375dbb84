"""The oracle against its pins (CPU only).  The checks live in pins.py."""
import pytest

import oracle
import pins


@pytest.mark.parametrize("check", pins.ALL, ids=[c.__name__[6:] for c in pins.ALL])
def test_pin(check):
    check(oracle.lib())


def test_every_oracle_entry_is_pinned():
    # each exported oracle routine is exercised by at least one pin
    import inspect
    src = inspect.getsource(pins)
    for name in ("half_to_double", "float_to_half", "pack_q4_0", "unpack_q4_0", "quantize_q8_0",
                 "unpack_q8_0", "q4_0_q8_0(", "q4_0_q8_0_sampled", "q4_0_q8_0_block_sums", "sgemm(",
                 "sgemm_sampled", "pack_ternary", "unpack_ternary", "quantize_i8_rows", "ternary(",
                 "ternary_sampled", "pack_q8_0", "q8_0_q8_0(", "q8_0_q8_0_sampled", "q8_0_q8_0_block_sums", "gemm_nt(", "gemm_nt_sampled"):
        assert "O." + name in src, name
