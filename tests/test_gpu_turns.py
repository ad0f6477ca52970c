"""The row kernel with turn counters: one workgroup per (row, v-head) for
launches of one row set (spec rows, or decodes), the last of a k-head's
workgroups to read the shared q/k conv channels rolling them ("[GDN]
Spec-decoding-aware attention kernel", "Changes": stage the pre-state, then
roll), one workgroup per CU for rows of two tokens or more on at least
four units per CU (32 rows of 32 v-heads on MI355X's 256 CUs), several per
CU otherwise.  On grids of at least two units per CU the last eighth of the
units is claimed at run time by the last workgroup of each CU (a wrapping
count in the NULL slot's counter cell).  Compared bit for bit with the
(row, k-head) form (no counters), which holds one k-head's channels in one
workgroup, and with the oracle; every counter is back at 0 after every
call."""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest

import synth
from tests import helpers
from tests.gpu_util import (Gpu, assert_out_close, assert_states_close, gpu_available, say,
                            spec_rows_of)
from tests.test_gpu_parity import check_spec_case
from tests.test_gpu_per_token import per_token_case
from tests.test_layout import per_k_head

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU and libgdn.so")]


def _same(a, b):
    np.testing.assert_array_equal(a.host_out(), b.host_out())
    np.testing.assert_array_equal(a.host_conv(), b.host_conv())
    np.testing.assert_array_equal(a.host_ssm(), b.host_ssm())


def _zero_turns(g):
    assert int(g.turns.abs().sum().item()) == 0, "turn counters not back at 0"


def _k4(seed, Ns=96, G=2, **kw):
    # Qwen3-Next-like heads, rows of up to four tokens, 96 rows: twelve
    # (row, v-head) units per CU, one workgroup per CU
    Hk = 32 // G
    return synth.make_case("qwen3next_k3_b64", seed=seed, K=4, Ns=Ns, Hk=Hk, Hv=32,
                           num_slots=4 * Ns + 16, permute_tokens=True, **kw)


@pytest.mark.parametrize("seed,null_p", [(0, 0.0), (1, 0.15)])
def test_vhead_units_match_khead_units_and_oracle(seed, null_p):
    case = _k4(400 + seed, null_p=null_p)
    a = check_spec_case(case)            # with counters; every row against the oracle
    _zero_turns(a)
    b = Gpu(case, turns=False)
    say(f"(row, k-head) form, seed {seed}")
    b.spec()
    _same(a, b)


def test_vhead_units_ragged_rows():
    rng = np.random.default_rng(410)
    lens = rng.integers(1, 5, 96)
    lens[0] = 4                           # rows of up to four tokens
    case = _k4(410, lens=lens)
    a = check_spec_case(case)
    _zero_turns(a)
    b = Gpu(case, turns=False)
    b.spec()
    _same(a, b)


def test_vhead_units_dynamic_tail_padded_rows():
    # 93 rows: the grid is padded to 96 rows, and the padded units sit in
    # the dynamically claimed tail (its last units), beside one-token rows
    # and NULL slots; two chained calls, so the second starts from the
    # count the first left (it must be back at 0)
    rng = np.random.default_rng(415)
    lens = rng.integers(1, 5, 93)
    lens[0] = 4
    lens[-3:] = 1
    case = _k4(415, Ns=93, lens=lens, null_p=0.15)
    a, b = Gpu(case), Gpu(case, turns=False)
    for step in range(2):
        say(f"dynamic tail, 93 ragged rows, call {step}")
        a.spec()
        b.spec()
        _zero_turns(a)
        _same(a, b)
    c = helpers.clone(case)
    for step in range(2):
        out, conv, ssm, _ = helpers.run_spec(c)
        c["conv_state"], c["ssm_state"] = conv, ssm
    sp = case["spec"]
    glob, slots = spec_rows_of(sp, range(sp["num_spec_decodes"]))
    assert_out_close(a.host_out(), out, glob)
    np.testing.assert_array_equal(a.host_conv(slots), conv[slots])
    assert_states_close(a.host_ssm(slots), ssm[slots])


def test_vhead_units_four_vheads_per_khead():
    # G = 4: four workgroups share a k-head's q/k channels (counts 0..3)
    case = _k4(420, Ns=96, G=4)
    a = check_spec_case(case)
    _zero_turns(a)
    b = Gpu(case, turns=False)
    b.spec()
    _same(a, b)


def test_vhead_units_per_k_head_qkv_layout():
    # reorder_input=False: a unit's v channels sit inside its k-head's block
    case = _k4(430)
    d = case["dims"]
    grouped = Gpu(case)
    inter = dict(case)
    inter["mixed_qkv"] = per_k_head(case["mixed_qkv"], d["Hk"], d["Hv"], d["dk"], d["dv"])
    per = Gpu(inter)
    per.cfg = dataclasses.replace(per.cfg, reorder_input=False)
    say("per-k-head layout with counters")
    grouped.spec()
    per.spec()
    _same(grouped, per)
    _zero_turns(per)
    ref = Gpu(case, turns=False)
    ref.spec()
    _same(grouped, ref)


def test_vhead_units_per_token_conv_slots():
    # per-token conv windows: the last reader of the load slot writes the
    # q/k windows of every token's slot
    case = per_token_case(440, 96, 4, Hk=16, Hv=32)
    a = check_spec_case(case)
    _zero_turns(a)
    b = Gpu(case, turns=False)
    b.spec()
    _same(a, b)


def test_vhead_units_chained_calls():
    # two steps on the same pools, the second reading what the first rolled
    case = _k4(450)
    a, b = Gpu(case), Gpu(case, turns=False)
    sp = case["spec"]
    for step in range(2):
        say(f"chained step {step}")
        a.spec()
        b.spec()
        _zero_turns(a)
        _same(a, b)
    # the oracle over the same two steps
    c = helpers.clone(case)
    for step in range(2):
        out, conv, ssm, _ = helpers.run_spec(c)
        c["conv_state"], c["ssm_state"] = conv, ssm
    glob, slots = spec_rows_of(sp, range(sp["num_spec_decodes"]))
    assert_out_close(a.host_out(), out, glob)
    np.testing.assert_array_equal(a.host_conv(slots), conv[slots])
    assert_states_close(a.host_ssm(slots), ssm[slots])


@pytest.mark.parametrize("Ns", [64, 0])
def test_vhead_units_with_decodes(Ns):
    # decodes and spec rows in one row-kernel launch (per k-head with or
    # without counters), and decodes alone (one token per row, per v-head
    # with counters)
    case = synth.make_case("mixed", seed=460, Ns=Ns, K=4, Nd=32, prefill_lens=())
    ref_out, ref_conv, ref_ssm = helpers.run_case(case)
    a, b = Gpu(case), Gpu(case, turns=False)
    say("decodes + spec rows with counters")
    a.attention()
    b.attention()
    _zero_turns(a)
    _same(a, b)
    named = synth.referenced_slots(case)
    np.testing.assert_array_equal(a.host_conv(named), ref_conv[named])
    assert_states_close(a.host_ssm(named), ref_ssm[named])
    rows = case["nonspec"]["token_indx"]
    if Ns:
        rows = np.concatenate([case["spec"]["spec_token_indx"], rows])
    assert_out_close(a.host_out(), ref_out, np.sort(rows))


def test_vhead_units_decodes_null_slots_no_initial_state():
    # A decode-only launch (one row set, so per v-head with counters) whose
    # rows include NULL cache slots (no ring, no state read or store) and
    # rows without an initial state (ring and state read as zeros, then
    # written): against the (row, k-head) form bit for bit and the oracle.
    nd = 96
    case = helpers.small_case(seed=470, Hk=16, Hv=32, dk=128, dv=128, K=1, T=nd, L=3,
                              num_slots=2 * nd + 8)
    rng = np.random.default_rng(471)
    slots = rng.choice(np.arange(1, case["dims"]["num_slots"]), nd, replace=False)
    slots[rng.random(nd) < 0.15] = 0
    his = (rng.random(nd) < 0.7).astype(np.uint8)
    tix = rng.permutation(nd).astype(np.int32)
    case["nonspec"] = helpers.nonspec_meta([1] * nd, slots, his=his, tix=tix, num_decodes=nd)
    case["spec"] = None
    case["name"] = "nonspec"
    out_ref, conv_ref, ssm_ref, _ = helpers.run_nonspec(case)
    a, b = Gpu(case), Gpu(case, turns=False)
    say("decodes with NULL slots and no initial state, with and without counters")
    a.attention()
    b.attention()
    _zero_turns(a)
    _same(a, b)
    assert_out_close(a.host_out(), out_ref)
    named = np.unique(slots[slots > 0])
    np.testing.assert_array_equal(a.host_conv(named), conv_ref[named])
    assert_states_close(a.host_ssm(named), ssm_ref[named])
    free = np.setdiff1d(np.arange(1, case["dims"]["num_slots"]), named)[:8]
    np.testing.assert_array_equal(a.host_ssm(free), case["ssm_state"][free])
