"""HIP path with per-token conv checkpoint slots ("[XE2] Support MTP of QWEN
model", conv-checkpoint review thread) against the oracle: ragged rows, NULL
slots, token_indx permutations, chains of calls that read the windows earlier
calls saved, and a batch with decodes."""
from __future__ import annotations

import numpy as np
import pytest

from tests import helpers
from tests.gpu_util import (Gpu, assert_out_close, assert_states_close, gpu_available, say,
                            spec_rows_of)
from tests.test_gpu_parity import check_spec_case

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU and libgdn.so")]

W = 4


def per_token_case(seed, Ns, K, T_extra=0, null_p=0.2, Hk=4, Hv=8, dk=128):
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, K + 1, Ns)
    T = int(lens.sum())
    S = Ns * K + 8
    case = helpers.small_case(seed=seed, Hk=Hk, Hv=Hv, dk=dk, dv=dk, K=K, T=T + T_extra,
                              L=W - 1, num_slots=S)
    case["dims"]["conv_layout"] = 1
    slots = rng.permutation(np.arange(1, S))[:Ns * K].reshape(Ns, K).astype(np.int32)
    slots[rng.random(slots.shape) < null_p] = 0
    nacc = np.array([rng.integers(1, n + 1) for n in lens], np.int32)
    sqsl = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    tix = rng.permutation(T).astype(np.int32)
    case["spec"] = helpers.spec_meta(sqsl, slots, nacc, tix)
    case["name"] = f"per-token K={K}"
    return case


@pytest.mark.parametrize("K", [2, 3, 4, 8])
def test_per_token_spec_parity(K):
    check_spec_case(per_token_case(400 + K, Ns=12, K=K))


def test_per_token_chained_calls():
    # Three calls on the same pools, each row keeping its K slots: every call
    # reads the window an earlier call saved at the slot of token n_acc - 1.
    rng = np.random.default_rng(410)
    Ns, K = 6, 3
    case = per_token_case(410, Ns=Ns, K=K, T_extra=2 * Ns * K, null_p=0.0)
    ssi = case["spec"]["spec_state_indices"]
    c = helpers.clone(case)
    g = Gpu(case)
    out_ref = np.zeros((case["num_actual_tokens"], case["dims"]["Hv"], case["dims"]["dv"]),
                       np.uint16)
    base = 0
    for call in range(3):
        lens = rng.integers(1, K + 1, Ns)
        sqsl = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        T = int(lens.sum())
        nacc = np.array([rng.integers(1, n + 1) for n in lens], np.int32)
        tix = (base + rng.permutation(T)).astype(np.int32)
        spec = helpers.spec_meta(sqsl, ssi, nacc, tix)
        o, ring, ssm, _ = helpers.run_spec(c, spec, out=out_ref)
        c["conv_state"], c["ssm_state"], out_ref = ring, ssm, o
        say(f"per-token chained call {call}: T={T}")
        g.spec(spec)
        base += T
    used = np.arange(base)
    assert_out_close(g.host_out(), out_ref, used)
    slots = np.unique(ssi[ssi > 0])
    np.testing.assert_array_equal(g.host_conv(slots), c["conv_state"][slots])
    assert_states_close(g.host_ssm(slots), c["ssm_state"][slots])


def test_per_token_with_decodes():
    # Decode rows use the plain window update on their one-window slots; the
    # spec rows save a window per token.
    Ns, K, Nd = 8, 3, 5
    case = per_token_case(420, Ns=Ns, K=K, T_extra=Nd, null_p=0.1)
    sp = case["spec"]
    T_spec = sp["num_spec_tokens"]
    S = case["dims"]["num_slots"]
    used = set(np.unique(sp["spec_state_indices"]).tolist())
    free = [s for s in range(1, S) if s not in used]
    dslots = free[:Nd]
    rng = np.random.default_rng(421)
    his = rng.integers(0, 2, Nd).tolist()
    rows = rng.permutation(T_spec + Nd).astype(np.int32)
    sp["spec_token_indx"] = rows[Nd:]
    case["nonspec"] = helpers.nonspec_meta([1] * Nd, dslots, his=his, tix=rows[:Nd])
    o1, r1, s1, _ = helpers.run_nonspec(case)
    c = helpers.clone(case)
    c["conv_state"], c["ssm_state"] = r1, s1
    out_ref, conv_ref, ssm_ref, _ = helpers.run_spec(c, out=o1)
    g = Gpu(case)
    say("per-token spec rows + decodes")
    g.attention()
    assert_out_close(g.host_out(), out_ref)
    slots = np.array(sorted((used - {0}) | set(dslots)))
    np.testing.assert_array_equal(g.host_conv(slots), conv_ref[slots])
    assert_states_close(g.host_ssm(slots), ssm_ref[slots])
