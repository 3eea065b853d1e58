"""The parity checks catch the mistakes they are there for.

A backward that flushed bf16 subnormal inputs to zero (in the dg sum or the
outputs) must fail the subnormal-row case that the GPU test runs: the
oracle's own backward, computed with every subnormal grad_out and value
element taken as zero, is checked against the exact oracle and must be
rejected, while the exact oracle passes."""
import numpy as np
import pytest

import oracle
from numerics import subnormal_rows_case
from parity import check_bwd


def _flush(bits):
    out = bits.copy()
    out[(bits & 0x7F80) == 0] &= 0x8000
    return out


def test_flushed_subnormals_fail_the_backward_check():
    inp = subnormal_rows_case()
    _, saved = oracle.fwd_bf16(inp["x"], inp["kv"], inp["weight"], inp["mask"], threads=8)
    dx, dkv, dw = oracle.bwd_bf16(inp["x"], _flush(inp["kv"]), inp["weight"], saved, _flush(inp["grad_out"]),
                                  threads=8)
    with pytest.raises(AssertionError, match="grad_x"):
        check_bwd(inp, saved, dx, dkv, dw, threads=8)
    dx, dkv, dw = oracle.bwd_bf16(inp["x"], inp["kv"], inp["weight"], saved, inp["grad_out"], threads=8)
    st = check_bwd(inp, saved, dx, dkv, dw, threads=8)
    assert st["dx_bit_equal_frac"] == 1.0
    assert np.count_nonzero((inp["grad_out"][:32] & 0x7F80) == 0) == inp["grad_out"][:32].size
