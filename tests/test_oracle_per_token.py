"""Pins of the oracle's per-token conv checkpoint layout ("[XE2] Support MTP of
QWEN model", review of the spec conv kernel): after spec token t the conv
window (the last W-1 inputs) is saved to that token's slot, as the SSM state
is, and the next round reads the window from the slot of token n_acc - 1.
A slot holds exactly one window (state_len = W - 1)."""
from __future__ import annotations

import numpy as np
import pytest

from tests.helpers import clone, nonspec_meta, run_nonspec, run_spec, small_case, spec_meta

W = 4


def per_token_case(seed, K, T, num_slots=16):
    case = small_case(seed=seed, K=K, T=T, L=W - 1, num_slots=num_slots)
    case["dims"]["conv_layout"] = 1
    return case


def rolled(case):
    c = clone(case)
    c["dims"]["conv_layout"] = 0
    return c


def decode_chain(case, slot, rows):
    """Sequential one-token decodes on `slot` over the given global rows (the
    plain conv-state update: the window is the last W-1 inputs)."""
    c = rolled(case)
    outs, states, windows = [], [], []
    for r in rows:
        o, ring, ssm, _ = run_nonspec(c, nonspec_meta([1], [slot], his=[1], tix=[r]))
        c["conv_state"], c["ssm_state"] = ring, ssm
        outs.append(o[r].copy())
        states.append(ssm[slot].copy())
        windows.append(ring[slot].copy())
    return outs, states, windows


def test_single_token_rows_equal_rolled_layout():
    # One token per row on a W-1 ring: both layouts read the slot's window and
    # write the window after the token back to the same slot.
    case = per_token_case(50, K=1, T=3)
    spec = spec_meta([0, 1, 2, 3], [[4], [0], [7]], [1, 1, 1], tix=[2, 0, 1])
    a = run_spec(case, spec)
    b = run_spec(rolled(case), spec)
    for x, y in zip(a[:3], b[:3]):
        np.testing.assert_array_equal(x, y)


def test_saved_windows_are_the_last_inputs():
    # Brute force: slot ssi[t] holds inputs t-W+2..t of (loaded window ++
    # row inputs), oldest first; NULL slots and unnamed slots keep their bytes.
    K = 3
    case = per_token_case(51, K=K, T=2 * K)
    ssi = [[3, 0, 5], [8, 9, 10]]
    nacc = [2, 3]
    tix = [4, 0, 2, 5, 1, 3]
    spec = spec_meta([0, K, 2 * K], ssi, nacc, tix=tix)
    _, ring, _, _ = run_spec(case, spec)
    pre = case["conv_state"]
    x = case["mixed_qkv"]
    for b in range(2):
        load = ssi[b][nacc[b] - 1]                            # NULL (<= 0) reads zeros
        seq = list(pre[load] if load > 0 else np.zeros_like(pre[0]))  # W-1 columns, oldest first
        seq += [x[r] for r in tix[b * K:(b + 1) * K]]
        for t in range(K):
            s = ssi[b][t]
            if s > 0:
                np.testing.assert_array_equal(ring[s], np.stack(seq[t + 1:t + W]))
    untouched = [s for s in range(16) if s not in (3, 5, 8, 9, 10)]
    np.testing.assert_array_equal(ring[untouched], pre[untouched])


def test_null_load_slot_reads_zeros():
    # Load slot NULL: the window is zeros whatever slot 0 holds, so the window
    # saved after token 1 is (0, x0, x1).
    K = 2
    case = per_token_case(52, K=K, T=K)
    spec = spec_meta([0, K], [[0, 6]], [1])
    a = run_spec(case, spec)
    c = clone(case)
    c["conv_state"][0] = 0x4049                 # bf16 3.14 in every column of slot 0
    b = run_spec(c, spec)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1][1:], b[1][1:])
    np.testing.assert_array_equal(b[1][0], c["conv_state"][0])   # NULL: never written
    np.testing.assert_array_equal(a[2], b[2])
    zero = np.zeros_like(case["conv_state"][0][0])
    seq = [zero] * (W - 1) + [case["mixed_qkv"][0], case["mixed_qkv"][1]]
    np.testing.assert_array_equal(a[1][6], np.stack(seq[2:2 + W - 1]))


@pytest.mark.parametrize("n1,n2", [(1, 3), (2, 1), (3, 2)])
def test_rollback_equals_decodes_over_accepted_prefix(n1, n2):
    # Call A reads slot ssi[K-1]; call B accepts n1 of A's tokens, call C n2
    # of B's.  Every output and state equal decodes over the accepted history.
    K = 3
    case = per_token_case(53 + 3 * n1 + n2, K=K, T=3 * K)
    ssi = [3, 4, 5]
    case["conv_state"][12] = case["conv_state"][5]
    case["ssm_state"][12] = case["ssm_state"][5]
    c = clone(case)
    res = {}
    for call, n, base in (("A", K, 0), ("B", n1, K), ("C", n2, 2 * K)):
        o, ring, ssm, _ = run_spec(c, spec_meta([0, K], [ssi], [n],
                                                tix=list(range(base, base + K))))
        c["conv_state"], c["ssm_state"] = ring, ssm
        res[call] = (o, {t: ssm[ssi[t]].copy() for t in range(K)},
                     {t: ring[ssi[t]].copy() for t in range(K)})
    hist_b = list(range(0, n1))
    outs, states, windows = decode_chain(case, 12, hist_b + list(range(K, 2 * K)))
    o, st, win = res["B"]
    for t in range(K):
        np.testing.assert_array_equal(o[K + t], outs[n1 + t])
        np.testing.assert_array_equal(st[t], states[n1 + t])
        np.testing.assert_array_equal(win[t], windows[n1 + t])
    hist_c = hist_b + list(range(K, K + n2))
    outs, states, windows = decode_chain(case, 12, hist_c + list(range(2 * K, 3 * K)))
    o, st, win = res["C"]
    for t in range(K):
        np.testing.assert_array_equal(o[2 * K + t], outs[len(hist_c) + t])
        np.testing.assert_array_equal(st[t], states[len(hist_c) + t])
        np.testing.assert_array_equal(win[t], windows[len(hist_c) + t])


def test_layout_preconditions():
    # spec_cache_indices has no meaning here, and a slot holds one window
    case = per_token_case(54, K=2, T=2)
    with pytest.raises(ValueError):
        run_spec(case, spec_meta([0, 2], [[3, 4]], [1], cache=[3]))
    longer = small_case(seed=54, K=2, T=2, L=W, num_slots=16)
    longer["dims"]["conv_layout"] = 1
    with pytest.raises(ValueError):
        run_spec(longer, spec_meta([0, 2], [[3, 4]], [1]))
