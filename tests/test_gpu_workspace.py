"""Prefill rows never read workspace bytes they did not write.

The workspace is caller-owned scratch ("gdn_workspace_bytes"): its padding
rows past the last token and the rows of neighbouring prefill rows are read
by whole-tile loads and dropped where used.  Filling it with NaN bit
patterns before the call must leave every output and state as the oracle
has them (a NaN that reached a product would spread through a row)."""
from __future__ import annotations

import pytest
import torch

from tests.gpu_util import Gpu, assert_out_close, assert_states_close, gpu_available, say
from tests import helpers
from tests.test_gpu_parity import _rows_case

import numpy as np

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU and libgdn.so")]


@pytest.mark.parametrize("dk", [32, 64, 128])
def test_prefill_ignores_workspace_contents(dk):
    # prefill rows ending one short of and one past a 64-token chunk, a
    # longer row and a one-token row, random initial states
    case, slots = _rows_case(70 + dk, [63, 65, 130, 1], dk, Hk=4, Hv=8)
    out_ref, conv_ref, ssm_ref, _ = helpers.run_nonspec(case)
    import speculative_decoding_causal_amd as gdn
    g = Gpu(case)
    d, ns = case["dims"], case["nonspec"]
    nbytes = gdn.gdn_workspace_bytes(g.cfg, d["L"], d["num_slots"], ns["num_non_spec_tokens"],
                                     ns["num_prefills"])
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")  # NaN in fp32 and bf16
    say(f"prefill dk={dk} on a NaN-filled workspace of {nbytes} bytes")
    g.attention(workspace=ws)
    assert_out_close(g.host_out(), out_ref)
    np.testing.assert_array_equal(g.host_conv(slots), conv_ref[slots])
    assert_states_close(g.host_ssm(slots), ssm_ref[slots])
