"""Host-side pieces of the benchmark: the byte accounting and the threaded
oracle baseline (one thread per block of rows gives the same bits as one
call over the whole batch)."""
from __future__ import annotations

import numpy as np
import pytest

import bench
import synth
from tests import helpers


@pytest.mark.parametrize("name,n", [("tiny", 2), ("small", 3), ("small", 8)])
def test_threaded_oracle_equals_one_call(name, n):
    case = synth.make_case(name, seed=5, permute_tokens=True)
    out1, conv1, ssm1, _ = helpers.run_spec(case)
    c = helpers.clone(case)
    out = np.zeros(helpers.out_shape(case), np.uint16)
    bench.oracle_threaded(case["dims"], c, bench.oracle_row_blocks(case, n), out)
    np.testing.assert_array_equal(out, out1)
    np.testing.assert_array_equal(c["conv_state"], conv1)
    np.testing.assert_array_equal(c["ssm_state"], ssm1)


def test_byte_accounting_of_the_k3_batch64_step():
    # 192 tokens of 8192 channels; 64 rows with a valid conv slot and state
    # load; 192 per-token stores of 32 x 64 KiB tiles (the survey's total,
    # with the ring read counted once per column it reads)
    case = synth.make_case("qwen3next_k3_b64", seed=0, with_pools=False)
    tile = 32 * 128 * 128 * 4
    assert bench.state_bytes(case) == (64 + 192) * tile
    assert bench.algorithmic_bytes(case) == 550069764
