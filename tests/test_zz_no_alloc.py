"""gdn_attention_static: the allocation-free variant of gdn_attention (prefill
scratch from the library's static per-GPU array).  Two calls in a row, the
second on a smaller batch, each compared with gdn_attention on the same
inputs (bit for bit: the same kernels) and with the CPU oracle (outputs
within 2e-2 + 2e-2|y|, SSM tiles within 1e-3, conv rings exact)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from tests import helpers
from tests.gpu_util import (Gpu, assert_out_close, assert_states_close, gpu_available, i32, say,
                            u8)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU and libgdn.so")]


def _mixed(seed, prefill_lens, Nd, Ns):
    return synth.make_case("mixed", seed=seed, Ns=Ns, K=3, Nd=Nd, prefill_lens=prefill_lens,
                           Hk=4, Hv=8, dk=128, dv=128, num_slots=96)


def _call_static(g):
    import speculative_decoding_causal_amd as gdn
    ns, sp = g.case["nonspec"], g.case["spec"]
    gdn.gdn_attention_static(
        g.cfg, g.qkv, g.a, g.b, g.w, g.bias, g.A_log, g.dt_bias, g.conv, g.ssm, g.out,
        num_decodes=ns["num_decodes"], num_prefills=ns["num_prefills"],
        num_non_spec_tokens=ns["num_non_spec_tokens"], query_start_loc=i32(ns["query_start_loc"]),
        non_spec_state_indices=i32(ns["cache_indices"]),
        has_initial_state=u8(ns.get("has_initial_state")),
        non_spec_token_indx=i32(ns.get("token_indx")),
        spec_query_start_loc=i32(sp["spec_query_start_loc"]),
        spec_state_indices=i32(sp["spec_state_indices"]),
        num_accepted_tokens=i32(sp["num_accepted_tokens"]),
        spec_token_indx=i32(sp.get("spec_token_indx")), num_spec_tokens=sp["num_spec_tokens"],
        conv_turns=g.turns)


def test_static_scratch_matches_workspace_call_twice():
    # the second batch is smaller: its unit map and scratch rows lie inside
    # what the first call left in the shared array
    for seed, plens, nd, ns in ((61, (300, 130), 6, 5), (62, (70,), 3, 2)):
        case = _mixed(seed, plens, nd, ns)
        ref = Gpu(case)
        say(f"gdn_attention (workspace): prefills {plens}, {nd} decodes, {ns} spec rows")
        ref.attention()
        st = Gpu(case)
        say(f"gdn_attention_static: prefills {plens}, {nd} decodes, {ns} spec rows")
        _call_static(st)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(st.host_out(), ref.host_out())
        np.testing.assert_array_equal(st.host_conv(), ref.host_conv())
        np.testing.assert_array_equal(st.host_ssm(), ref.host_ssm())
        out_ref, conv_ref, ssm_ref = helpers.run_case(case, out=np.full(
            helpers.out_shape(case), 0x5A5A, np.uint16))
        assert_out_close(st.host_out(), out_ref)
        np.testing.assert_array_equal(st.host_conv(), conv_ref)
        slots = synth.referenced_slots(case)
        assert_states_close(st.host_ssm(slots), ssm_ref[slots])


def test_static_scratch_with_an_empty_prefill_row():
    # a prefill row of no tokens (as a graph pad row is) beside a real one:
    # the prefill kernels still get the static scratch
    case = _mixed(64, (90, 0), 3, 2)
    assert case["nonspec"]["num_prefills"] == 2
    ref = Gpu(case)
    ref.attention()
    st = Gpu(case)
    say("gdn_attention_static: prefills (90, 0), 3 decodes, 2 spec rows")
    _call_static(st)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(st.host_out(), ref.host_out())
    np.testing.assert_array_equal(st.host_conv(), ref.host_conv())
    np.testing.assert_array_equal(st.host_ssm(), ref.host_ssm())
    out_ref, conv_ref, ssm_ref = helpers.run_case(case, out=np.full(
        helpers.out_shape(case), 0x5A5A, np.uint16))
    assert_out_close(st.host_out(), out_ref)
    np.testing.assert_array_equal(st.host_conv(), conv_ref)
    slots = synth.referenced_slots(case)
    assert_states_close(st.host_ssm(slots), ssm_ref[slots])
