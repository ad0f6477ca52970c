"""Pins of the CPU oracle against facts fixed by the pages and by mathematics
(closed forms, invariants, library routines, brute force).  No GPU.

Each pin is chosen so that a plausible mistake in the oracle (a wrong window
offset or roll shift, a transposed state, a dropped decay, a wrong sign, a
wrong GQA mapping, gates read at the wrong row) makes at least one test fail.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest
import scipy.special as sps
import torch

import oracle
import synth
from tests.helpers import (clone, nonspec_meta, run_nonspec, run_spec,
                           small_case, spec_meta)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
f32 = synth.from_bf16


# --------------------------------------------------------------------------
# bf16 rounding


def test_bf16_round_special_values():
    r = oracle.bf16_round
    assert r(1.0) == 0x3F80
    assert r(1.0 + 2 ** -8) == 0x3F80          # tie -> even (mantissa 0)
    assert r(1.0 + 3 * 2 ** -8) == 0x3F82      # tie -> even (mantissa 2)
    assert r(1.0 + 2 ** -8 + 2 ** -30) == 0x3F81  # just above the tie
    assert r(-2.0) == 0xC000
    assert r(2 ** -133) == 0x0001              # smallest subnormal
    assert r(1.5 * 2 ** -133) == 0x0002        # tie -> even
    assert r(0.5 * 2 ** -133) == 0x0000        # tie -> even (zero)
    assert r((2 - 2 ** -7) * 2 ** 127) == 0x7F7F  # largest finite
    assert r((2 - 2 ** -8) * 2 ** 127) == 0x7F80  # tie at the top -> inf
    assert r(float("inf")) == 0x7F80
    assert r(-0.0) == 0x8000


def test_bf16_round_matches_bit_trick_on_float32_values():
    # Two independent roundings (value-based in the oracle, bit-based in the
    # input generator) must agree on every float32 input.
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(4000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-38).astype(np.float32),
        (rng.standard_normal(2000) * 1e30).astype(np.float32)])
    want = synth.to_bf16(x)
    got = np.array([oracle.bf16_round(float(v)) for v in x], np.uint16)
    np.testing.assert_array_equal(got, want)


# --------------------------------------------------------------------------
# gates: closed forms and library routines


def _gate(a, b, A_log, dt=0.0):
    al, be = oracle.gates(synth.to_bf16(np.array([[a]], np.float32)),
                          synth.to_bf16(np.array([[b]], np.float32)),
                          np.array([A_log], np.float32), np.array([dt], np.float32))
    return al[0, 0], be[0, 0]


def test_gate_closed_forms():
    al, be = _gate(0.3, 0.0, -np.inf)
    assert al == 1.0 and be == 0.5               # exp(-0 * sp) = 1, sigmoid(0)
    al, _ = _gate(0.0, 0.0, 0.0)
    assert abs(al - 0.5) < 1e-15                 # softplus(0) = ln 2
    al, _ = _gate(20.0, 0.0, 5.0)
    assert al == 0.0                             # exp(-e^5 * 20) underflows
    al, _ = _gate(30.0, 0.0, 0.0)
    assert abs(al - math.exp(-30.0)) < 1e-25     # softplus(x > 20) = x
    _, be = _gate(0.0, 20.0, 0.0)
    assert abs(be - 1.0 / (1.0 + math.exp(-20.0))) < 1e-16
    _, be = _gate(0.0, -20.0, 0.0)
    assert abs(be - 2.0611536e-9) < 1e-15
    _, be = _gate(0.0, float("inf"), 0.0)
    assert be == 1.0


def test_gates_match_scipy():
    rng = np.random.default_rng(2)
    n, Hv = 64, 8
    a = synth.to_bf16(3 * rng.standard_normal((n, Hv), dtype=np.float32))
    b = synth.to_bf16(3 * rng.standard_normal((n, Hv), dtype=np.float32))
    A_log = rng.uniform(-1, 3, Hv).astype(np.float32)
    dt = rng.standard_normal(Hv).astype(np.float32)
    al, be = oracle.gates(a, b, A_log, dt)
    x = f32(a).astype(np.float64) + dt.astype(np.float64)
    sp = np.logaddexp(0.0, x)                    # softplus
    np.testing.assert_allclose(al, np.exp(-np.exp(A_log.astype(np.float64)) * sp),
                               rtol=1e-12, atol=0)
    np.testing.assert_allclose(be, sps.expit(f32(b).astype(np.float64)),
                               rtol=1e-14, atol=0)


# --------------------------------------------------------------------------
# conv window and ring  (P1 "Changes": load shift n_acc-1 at cache_indices
# column 0; the current input goes to column state_len - K_call + t; the
# first state_len - K_call columns are a shift copy of the pre-state)


def _onehot_case(seed, W=4, K=3, Ns=3):
    case = small_case(seed=seed, W=W, K=K, T=Ns * K, activation=0,
                      use_qk_l2norm=1)
    C = case["conv_weight"].shape[0]
    w = np.zeros((C, W), np.float32)
    msel = np.arange(C) % W
    w[np.arange(C), msel] = 1.0
    case["conv_weight"] = synth.to_bf16(w)
    return case, msel


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_conv_window_offset_one_hot_taps(seed):
    W, K, Ns = 4, 3, 3
    case, msel = _onehot_case(seed, W, K, Ns)
    L = case["dims"]["L"]
    sqsl = [0, 3, 6, 9]
    ssi = [[1, 2, 3], [4, 5, 6], [7, 8, 9]]
    nacc = [1, 2, 3]                              # every offset once
    tix = np.random.default_rng(seed).permutation(9)
    spec = spec_meta(sqsl, ssi, nacc, tix)
    pre = case["conv_state"].copy()
    out, ring, _, y = run_spec(case, spec, with_conv=True)
    x = case["mixed_qkv"]
    C = x.shape[1]
    for bi in range(Ns):
        cs, n = ssi[bi][0], nacc[bi]
        rows = tix[sqsl[bi]:sqsl[bi + 1]]
        for j in range(K):
            for c in range(C):
                idx = j + msel[c]
                if idx < W - 1:
                    want = pre[cs, n - 1 + idx, c]
                else:
                    want = x[rows[idx - (W - 1)], c]
                assert y[rows[j], c] == f32(np.array([want]))[0]
        # ring: shift copy from column n, then the inputs at L-K+t
        for l in range(L):
            want = pre[cs, n + l] if l < L - K else x[rows[l - (L - K)]]
            np.testing.assert_array_equal(ring[cs, l], want)


def test_conv_matches_torch_conv1d():
    # The oracle's conv output equals torch's grouped conv1d (a library
    # routine) run on the explicit window ++ inputs, followed by SiLU.
    case = small_case(seed=4, W=4, K=3, T=6, activation=1)
    case["conv_bias"] = synth.to_bf16(
        np.random.default_rng(9).standard_normal(case["conv_weight"].shape[0]).astype(np.float32))
    spec = spec_meta([0, 3, 6], [[3, 4, 5], [6, 7, 8]], [2, 3])
    pre = case["conv_state"].copy()
    _, _, _, y = run_spec(case, spec, with_conv=True)
    W = 4
    w = torch.from_numpy(f32(case["conv_weight"]).astype(np.float64))[:, None, :]
    bias = torch.from_numpy(f32(case["conv_bias"]).astype(np.float64))
    for bi, (cs, n) in enumerate([(3, 2), (6, 3)]):
        hist = f32(pre[cs, n - 1:n - 1 + W - 1]).astype(np.float64)   # [W-1, C]
        xs = f32(case["mixed_qkv"][3 * bi:3 * bi + 3]).astype(np.float64)
        seq = torch.from_numpy(np.concatenate([hist, xs]).T.copy())[None]  # [1,C,W-1+K]
        ref = torch.nn.functional.silu(
            torch.nn.functional.conv1d(seq, w, bias, groups=w.shape[0]))[0].T.numpy()
        np.testing.assert_allclose(y[3 * bi:3 * bi + 3], ref, rtol=1e-12, atol=1e-12)


def test_nonspec_conv_tail_window_matches_torch_conv1d():
    case = small_case(seed=5, W=4, K=3, T=7, activation=1)
    ns = nonspec_meta([1, 6], [2, 5], his=[1, 1])
    pre = case["conv_state"].copy()
    _, ring, _, y = run_nonspec(case, ns, with_conv=True)
    L, W = case["dims"]["L"], 4
    w = torch.from_numpy(f32(case["conv_weight"]).astype(np.float64))[:, None, :]
    for (j0, T, slot) in [(0, 1, 2), (1, 6, 5)]:
        hist = f32(pre[slot, L - W + 1:]).astype(np.float64)
        xs = f32(case["mixed_qkv"][j0:j0 + T]).astype(np.float64)
        seq = torch.from_numpy(np.concatenate([hist, xs]).T.copy())[None]
        ref = torch.nn.functional.silu(
            torch.nn.functional.conv1d(seq, w, groups=w.shape[0]))[0].T.numpy()
        np.testing.assert_allclose(y[j0:j0 + T], ref, rtol=1e-12, atol=1e-12)
        full = np.concatenate([pre[slot], case["mixed_qkv"][j0:j0 + T]])
        np.testing.assert_array_equal(ring[slot], full[-L:])


def test_column0_contract_only_conv_slot_changes():
    # Canary pools: only slot cache_indices[:,0] of the conv pool changes,
    # and only the store slots of the SSM pool; slot 0 is never written.
    case = small_case(seed=6, K=3, T=6)
    case["conv_state"][:] = 0xABCD
    case["ssm_state"][:] = np.float32(7.25)
    spec = spec_meta([0, 3, 6], [[3, 4, 0], [6, 0, 8]], [1, 3])
    _, ring, ssm, _ = run_spec(case, spec)
    changed_conv = {s for s in range(ring.shape[0])
                    if not np.array_equal(ring[s], case["conv_state"][s])}
    changed_ssm = {s for s in range(ssm.shape[0])
                   if not np.array_equal(ssm[s], case["ssm_state"][s])}
    assert changed_conv == {3, 6}
    assert changed_ssm == {3, 4, 6, 8}


# --------------------------------------------------------------------------
# recurrence (gated delta rule)


def _identity_conv(case):
    C, W = case["conv_weight"].shape
    w = np.zeros((C, W), np.float32)
    w[:, W - 1] = 1.0            # y_j = x_j exactly
    case["conv_weight"] = synth.to_bf16(w)
    case["dims"]["activation"] = 0


def _set_blocks(case, row, q=None, k=None, v=None, kh=0, vh=0):
    d = case["dims"]
    Hk, dk, dv = d["Hk"], d["dk"], d["dv"]
    x = f32(case["mixed_qkv"]).copy()
    if q is not None:
        x[row, kh * dk:(kh + 1) * dk] = q
    if k is not None:
        x[row, Hk * dk + kh * dk:Hk * dk + (kh + 1) * dk] = k
    if v is not None:
        x[row, 2 * Hk * dk + vh * dv:2 * Hk * dk + (vh + 1) * dv] = v
    case["mixed_qkv"] = synth.to_bf16(x)


def test_exact_recall_orthonormal_keys():
    # beta = 1, decay = 1, scale = 1, keys e_0..e_{K-1}, zero initial state:
    # querying e_j returns v_j (the l2-norm eps only scales by 1/(1+eps)).
    K, dk = 4, 8
    case = small_case(seed=7, Hk=1, Hv=1, dk=dk, dv=6, K=K, T=K, scale=1.0)
    _identity_conv(case)
    case["A_log"][:] = -np.inf
    case["b"][:] = synth.to_bf16(np.full(case["b"].shape, np.inf, np.float32))
    rng = np.random.default_rng(0)
    vals = rng.standard_normal((K, 6)).astype(np.float32)
    qsel = [0, 0, 2, 1]                      # query a key already written
    for t in range(K):
        _set_blocks(case, t, q=np.eye(dk)[qsel[t]], k=np.eye(dk)[t], v=vals[t])
    spec = spec_meta([0, K], [[0, 2, 3, 4]], [1])   # NULL load -> zero state
    out, _, _, _ = run_spec(case, spec)
    for t in range(K):
        np.testing.assert_array_equal(out[t, 0], synth.to_bf16(vals[qsel[t]]))


def test_l2norm_eps_inside_the_square_root():
    # q = k = 2 e_1 (sum of squares 4) with eps = 12: the norm is
    # sqrt(4 + 12) = 4, so q_hat = k_hat = e_1 / 2 exactly.  With beta = 1,
    # decay 1, scale 1 and a zero prior state, S = v k_hat^T and
    # o = (k_hat . q_hat) v = v / 4, both exact in binary.  eps added outside
    # the root (2 / (2 + 12)) or dropped (e_1) gives v / 49 or v.
    dk, dv = 8, 4
    case = small_case(seed=12, Hk=1, Hv=1, dk=dk, dv=dv, K=1, T=1, eps=12.0, scale=1.0)
    _identity_conv(case)
    case["A_log"][:] = -np.inf
    case["b"][:] = synth.to_bf16(np.full(case["b"].shape, np.inf, np.float32))
    v = np.array([1.0, -2.0, 0.5, 3.0], np.float32)
    _set_blocks(case, 0, q=2 * np.eye(dk)[1], k=2 * np.eye(dk)[1], v=v)
    case["ssm_state"][3] = 0.0
    out, _, ssm, _ = run_spec(case, spec_meta([0, 1], [[3]], [1]))
    np.testing.assert_array_equal(out[0, 0], synth.to_bf16(v / 4))
    want = np.zeros((dv, dk), np.float32)
    want[:, 1] = v / 2
    np.testing.assert_array_equal(ssm[3, 0], want)


def test_last_write_recall_any_state():
    # beta = 1 and a unit key give S_t k_t = v_t whatever S_{t-1} and alpha;
    # the query equal to the key returns scale * v_t.
    K, dk, dv = 3, 16, 16
    case = small_case(seed=8, Hk=2, Hv=4, dk=dk, dv=dv, K=K, T=K, eps=0.0)
    _identity_conv(case)
    case["b"][:] = synth.to_bf16(np.full(case["b"].shape, np.inf, np.float32))
    x = f32(case["mixed_qkv"]).copy()
    Hk = 2
    x[:, :Hk * dk] = x[:, Hk * dk:2 * Hk * dk]          # q = k per k-head
    case["mixed_qkv"] = synth.to_bf16(x)
    spec = spec_meta([0, K], [[5, 6, 7]], [2])
    out, _, ssm, _ = run_spec(case, spec)
    scale = case["dims"]["scale"]
    xf = f32(case["mixed_qkv"]).astype(np.float64)
    for t in range(K):
        for h in range(4):
            v = xf[t, 2 * Hk * dk + h * dv:2 * Hk * dk + (h + 1) * dv]
            k = xf[t, Hk * dk + (h // 2) * dk:Hk * dk + (h // 2 + 1) * dk]
            k = k / np.linalg.norm(k)
            np.testing.assert_allclose(f32(out[t, h]), scale * v, rtol=2 ** -7, atol=1e-6)
            S = ssm[[5, 6, 7][t], h].astype(np.float64)
            np.testing.assert_allclose(S @ k, v, rtol=1e-5, atol=1e-5)


def test_forget_alpha_zero():
    # alpha = 0: S_t = beta v k^T, so o = scale * beta (k.q) v.
    K, dk, dv = 2, 16, 8
    case = small_case(seed=9, Hk=1, Hv=2, dk=dk, dv=dv, K=K, T=K)
    _identity_conv(case)
    case["A_log"][:] = 5.0
    case["a"][:] = synth.to_bf16(np.full(case["a"].shape, 20.0, np.float32))
    case["dt_bias"][:] = 0.0
    spec = spec_meta([0, K], [[3, 4]], [2])
    out, _, ssm, _ = run_spec(case, spec)
    d = case["dims"]
    xf = f32(case["mixed_qkv"]).astype(np.float64)
    bf = sps.expit(f32(case["b"]).astype(np.float64))
    for t in range(K):
        q = xf[t, :dk]
        k = xf[t, dk:2 * dk]
        q = q / np.sqrt(q @ q + 1e-6)
        k = k / np.sqrt(k @ k + 1e-6)
        for h in range(2):
            v = xf[t, 2 * dk + h * dv:2 * dk + (h + 1) * dv]
            want_S = bf[t, h] * np.outer(v, k)
            np.testing.assert_allclose(ssm[[3, 4][t], h], want_S, rtol=1e-6, atol=1e-7)
            want_o = d["scale"] * bf[t, h] * (k @ q) * v
            np.testing.assert_allclose(f32(out[t, h]), want_o, rtol=2 ** -8, atol=1e-6)


def test_hold_beta_zero():
    # beta ~ 3.7e-44 and alpha = 0.5: the state only decays, S_t = 0.5^(t+1) S_0.
    K = 3
    case = small_case(seed=10, Hk=1, Hv=1, dk=8, dv=8, K=K, T=K)
    case["b"][:] = synth.to_bf16(np.full(case["b"].shape, -100.0, np.float32))
    case["A_log"][:] = 0.0
    case["dt_bias"][:] = 0.0
    case["a"][:] = 0
    spec = spec_meta([0, K], [[2, 3, 4]], [2])      # load slot ssi[0][1] = 3
    S0 = case["ssm_state"][3, 0].astype(np.float64)
    _, _, ssm, _ = run_spec(case, spec)
    for t, st in enumerate([2, 3, 4]):
        np.testing.assert_allclose(ssm[st, 0], 0.5 ** (t + 1) * S0, rtol=1e-6, atol=1e-12)


def test_scalar_closed_form():
    # dk = dv = 1, eps = 0, k = 1: with alpha = 1/2 and beta = 1/2,
    # S_1 = 0.5 * S_0 * (1 - 0.5) + 0.5 * v = 0.25 S_0 + 0.5 v, o = scale S_1 q.
    case = small_case(seed=11, Hk=1, Hv=1, dk=1, dv=1, K=1, T=1, eps=0.0,
                      scale=1.0, L=3)
    _identity_conv(case)
    case["A_log"][:] = 0.0
    case["dt_bias"][:] = 0.0
    case["a"][:] = 0
    case["b"][:] = 0
    case["mixed_qkv"][0] = synth.to_bf16(np.array([-3.0, 1.0, 2.0], np.float32))
    case["ssm_state"][4, 0, 0, 0] = 0.75
    spec = spec_meta([0, 1], [[4]], [1])
    out, _, ssm, _ = run_spec(case, spec)
    S1 = 0.25 * 0.75 + 0.5 * 2.0                    # 1.1875, exact in fp32
    assert abs(ssm[4, 0, 0, 0] - S1) < 1e-7
    assert f32(out[0, 0])[0] == -S1                  # q = -3 normalises to -1


def _dense_reference(case, spec):
    """The gated delta rule written with explicit matrices,
    S_t = alpha S_{t-1} (I - beta k k^T) + beta v k^T, o_t = scale S_t q_t,
    fed by torch's grouped conv1d and scipy's sigmoid / softplus."""
    d = case["dims"]
    Hk, Hv, dk, dv, W = d["Hk"], d["Hv"], d["dk"], d["dv"], d["W"]
    G = Hv // Hk
    x = f32(case["mixed_qkv"]).astype(np.float64)
    w = torch.from_numpy(f32(case["conv_weight"]).astype(np.float64))[:, None, :]
    af = f32(case["a"]).astype(np.float64)
    bf = f32(case["b"]).astype(np.float64)
    A = case["A_log"].astype(np.float64)
    dt = case["dt_bias"].astype(np.float64)
    pool = case["ssm_state"].astype(np.float64)
    ring = case["conv_state"]
    outs, states = {}, {}
    sq = spec["spec_query_start_loc"]
    for bi in range(spec["num_spec_decodes"]):
        j0, j1 = sq[bi], sq[bi + 1]
        n = spec["num_accepted_tokens"][bi]
        ssi = spec["spec_state_indices"][bi]
        rows = (spec["spec_token_indx"][j0:j1] if spec["spec_token_indx"] is not None
                else np.arange(j0, j1))
        hist = f32(ring[ssi[0], n - 1:n - 1 + W - 1]).astype(np.float64)
        seq = torch.from_numpy(np.concatenate([hist, x[rows]]).T.copy())[None]
        y = torch.nn.functional.silu(
            torch.nn.functional.conv1d(seq, w, groups=w.shape[0]))[0].T.numpy()
        for h in range(Hv):
            i = h // G
            s0 = ssi[n - 1]
            S = pool[s0, h].copy() if s0 > 0 else np.zeros((dv, dk))
            for t, r in enumerate(rows):
                q = y[t, i * dk:(i + 1) * dk]
                k = y[t, Hk * dk + i * dk:Hk * dk + (i + 1) * dk]
                v = y[t, 2 * Hk * dk + h * dv:2 * Hk * dk + (h + 1) * dv]
                q = q / np.sqrt(q @ q + d["eps"])
                k = k / np.sqrt(k @ k + d["eps"])
                alpha = np.exp(-np.exp(A[h]) * np.logaddexp(0.0, af[r, h] + dt[h]))
                beta = sps.expit(bf[r, h])
                S = alpha * S @ (np.eye(dk) - beta * np.outer(k, k)) + beta * np.outer(v, k)
                outs[(r, h)] = d["scale"] * S @ q
                if ssi[t] > 0:
                    states[(ssi[t], h)] = S.copy()
    return outs, states


@pytest.mark.parametrize("seed", [0, 1])
def test_dense_matrix_brute_force(seed):
    # Non-symmetric states, G = 2 grouping, ragged rows, permuted token rows.
    case = small_case(seed=20 + seed, Hk=2, Hv=4, dk=8, dv=5, K=3, T=5)
    tix = np.random.default_rng(seed).permutation(5)
    spec = spec_meta([0, 3, 5], [[1, 2, 3], [4, 5, 0]], [3, 2], tix)
    out, _, ssm, _ = run_spec(case, spec)
    outs, states = _dense_reference(case, spec)
    for (r, h), o in outs.items():
        np.testing.assert_allclose(f32(out[r, h]), o, rtol=2 ** -7, atol=1e-5)
    for (s, h), S in states.items():
        np.testing.assert_allclose(ssm[s, h], S, rtol=1e-5, atol=1e-6)


def test_brute_force_tiny_workload():
    # The tiny workload (2 rows, K=2, 2/4 heads, dk=dv=16) against the dense
    # fp64 formulation.
    case = synth.make_case("tiny", seed=3)
    out, _, ssm, _ = run_spec(case)
    outs, states = _dense_reference(case, case["spec"])
    for (r, h), o in outs.items():
        np.testing.assert_allclose(f32(out[r, h]), o, rtol=2 ** -7, atol=1e-5)
    for (s, h), S in states.items():
        np.testing.assert_allclose(ssm[s, h], S, rtol=1e-5, atol=1e-6)


# --------------------------------------------------------------------------
# slot logic and rollback (P1 "Changes", P1 review thread: K=N aligned ring
# equals non-spec decode, NULL_BLOCK_ID suppresses pool I/O)


def test_null_load_equals_zero_state():
    case = small_case(seed=12, K=3, T=3)
    spec_null = spec_meta([0, 3], [[4, 0, 6]], [2])
    out_null, _, _, _ = run_spec(case, spec_null)
    c2 = clone(case)
    c2["ssm_state"][9] = 0.0
    out_zero, _, _, _ = run_spec(c2, spec_meta([0, 3], [[4, 9, 6]], [2]))
    np.testing.assert_array_equal(out_null, out_zero)


def test_null_store_leaves_slots_untouched():
    case = small_case(seed=13, K=3, T=3)
    spec = spec_meta([0, 3], [[4, 0, 6]], [1])
    _, _, ssm, _ = run_spec(case, spec)
    np.testing.assert_array_equal(ssm[0], case["ssm_state"][0])
    untouched = [s for s in range(ssm.shape[0]) if s not in (4, 6)]
    np.testing.assert_array_equal(ssm[untouched], case["ssm_state"][untouched])


def _decode_chain(case, slot, rows):
    """Sequential one-token non-spec decodes over the given global rows."""
    c = clone(case)
    outs = []
    states = []
    for r in rows:
        ns = nonspec_meta([1], [slot], his=[1], tix=[r])
        o, ring, ssm, _ = run_nonspec(c, ns)
        c["conv_state"], c["ssm_state"] = ring, ssm
        outs.append(o[r].copy())
        states.append(ssm[slot].copy())
    return outs, states, c


def test_k1_spec_equals_decode_on_minimal_ring():
    # K = 1 spec on an L = W-1 ring is a plain decode, bit for bit.
    case = small_case(seed=14, K=1, T=1)             # L = W - 1 = 3
    spec = spec_meta([0, 1], [[5]], [1])
    out_s, ring_s, ssm_s, _ = run_spec(case, spec)
    outs, states, c = _decode_chain(case, 5, [0])
    np.testing.assert_array_equal(out_s[0], outs[0])
    np.testing.assert_array_equal(ring_s, c["conv_state"])
    np.testing.assert_array_equal(ssm_s, c["ssm_state"])


@pytest.mark.parametrize("K", [2, 3, 4])
def test_all_accepted_spec_equals_sequential_decodes(K):
    case = small_case(seed=15 + K, K=K, T=K, num_slots=16)
    L = case["dims"]["L"]
    ssi = [2 + t for t in range(K)]
    cs = ssi[0]
    # Decode reference on slot 12 holding the same ring and the loaded state.
    case["conv_state"][12] = case["conv_state"][cs]
    case["ssm_state"][12] = case["ssm_state"][ssi[K - 1]]
    spec = spec_meta([0, K], [ssi], [K])
    out_s, ring_s, ssm_s, _ = run_spec(case, spec)
    outs, states, c = _decode_chain(case, 12, list(range(K)))
    for t in range(K):
        np.testing.assert_array_equal(out_s[t], outs[t])
        np.testing.assert_array_equal(ssm_s[ssi[t]], states[t])
    np.testing.assert_array_equal(ring_s[cs], c["conv_state"][12])
    assert L == 4 - 1 + K - 1


@pytest.mark.parametrize("n1,n2", [(1, 1), (1, 3), (2, 2), (3, 1), (2, 3)])
def test_rollback_equals_decodes_over_accepted_prefix(n1, n2):
    # Call A (all accepted before it), call B with n_acc = n1 of A's tokens,
    # call C with n_acc = n2 of B's tokens.  Every output and the state after
    # each token equal sequential decodes over the accepted history.
    K = 3
    case = small_case(seed=30 + 3 * n1 + n2, K=K, T=3 * K, num_slots=16)
    ssi = [3, 4, 5]
    case["conv_state"][12] = case["conv_state"][3]
    case["ssm_state"][12] = case["ssm_state"][5]
    c = clone(case)
    for call, n, base in (("A", K, 0), ("B", n1, K), ("C", n2, 2 * K)):
        spec = spec_meta([0, K], [ssi], [n], tix=list(range(base, base + K)))
        o, ring, ssm, _ = run_spec(c, spec)
        c["conv_state"], c["ssm_state"] = ring, ssm
        if call == "A":
            out_a, st_a = o, {t: ssm[ssi[t]].copy() for t in range(K)}
        elif call == "B":
            out_b, st_b = o, {t: ssm[ssi[t]].copy() for t in range(K)}
        else:
            out_c, st_c = o, {t: ssm[ssi[t]].copy() for t in range(K)}
    # reference: A's first n1 tokens, B's tokens (B's first n2 accepted), C
    hist_b = list(range(0, n1))
    outs_b, states_b, _ = _decode_chain(case, 12, hist_b + list(range(K, 2 * K)))
    for t in range(K):
        np.testing.assert_array_equal(out_b[K + t], outs_b[n1 + t])
        np.testing.assert_array_equal(st_b[t], states_b[n1 + t])
    hist_c = hist_b + list(range(K, K + n2))
    outs_c, states_c, _ = _decode_chain(case, 12, hist_c + list(range(2 * K, 3 * K)))
    for t in range(K):
        np.testing.assert_array_equal(out_c[2 * K + t], outs_c[len(hist_c) + t])
        np.testing.assert_array_equal(st_c[t], states_c[len(hist_c) + t])


def test_rollback_catches_per_slot_snapshot_layout():
    # The prior-art layout (a conv snapshot per draft token in its own slot,
    # page 1 "Problem") read through the rolled-history contract gives a
    # different window: make sure the rollback check would see it.
    K = 3
    case = small_case(seed=40, K=K, T=2 * K, num_slots=16)
    ssi = [3, 4, 5]
    c = clone(case)
    spec = spec_meta([0, K], [ssi], [K], tix=[0, 1, 2])
    _, ring, ssm, _ = run_spec(c, spec)
    c["conv_state"], c["ssm_state"] = ring, ssm
    good, _, _, _ = run_spec(c, spec_meta([0, K], [ssi], [1], tix=[3, 4, 5]))
    bad_ring = c["conv_state"].copy()
    bad_ring[3] = np.roll(bad_ring[3], 1, axis=0)      # misplaced history
    c["conv_state"] = bad_ring
    bad, _, _, _ = run_spec(c, spec_meta([0, K], [ssi], [1], tix=[3, 4, 5]))
    assert np.abs(f32(good[3:6]) - f32(bad[3:6])).max() > 1e-2


def test_has_initial_state_zero_reads_nothing():
    case = small_case(seed=41, K=3, T=4)
    ns = nonspec_meta([4], [7], his=[0], num_decodes=0)
    out_a, ring_a, ssm_a, _ = run_nonspec(case, ns)
    c2 = clone(case)
    c2["conv_state"][7] = 0
    c2["ssm_state"][7] = 0
    out_b, ring_b, ssm_b, _ = run_nonspec(c2, nonspec_meta([4], [7], his=[1], num_decodes=0))
    np.testing.assert_array_equal(out_a, out_b)
    np.testing.assert_array_equal(ring_a[7], ring_b[7])
    np.testing.assert_array_equal(ssm_a[7], ssm_b[7])


def test_prefill_equals_sequential_decodes():
    case = small_case(seed=42, K=3, T=9)
    ns = nonspec_meta([9], [6], his=[1], num_decodes=0)
    out_p, ring_p, ssm_p, _ = run_nonspec(case, ns)
    outs, states, c = _decode_chain(case, 6, list(range(9)))
    for t in range(9):
        np.testing.assert_array_equal(out_p[t], outs[t])
    np.testing.assert_array_equal(ring_p[6], c["conv_state"][6])
    np.testing.assert_array_equal(ssm_p[6], c["ssm_state"][6])


# --------------------------------------------------------------------------
# token_indx (P2 overview: token-index remapping; P3 "Purpose": gates read
# through the same indices as mixed_qkv)


def test_token_permutation_invariance():
    case = synth.make_case("tiny", seed=5)
    T = case["num_actual_tokens"]
    out_a, ring_a, ssm_a, _ = run_spec(case)
    perm = np.random.default_rng(5).permutation(T)
    c2 = clone(case)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(T)
    for k in ("mixed_qkv", "a", "b"):
        c2[k] = np.ascontiguousarray(case[k][inv])     # token j moves to row perm[j]
    c2["spec"]["spec_token_indx"] = perm.astype(np.int32)
    out_b, ring_b, ssm_b, _ = run_spec(c2)
    np.testing.assert_array_equal(out_b[perm], out_a)
    np.testing.assert_array_equal(ring_a, ring_b)
    np.testing.assert_array_equal(ssm_a, ssm_b)


@pytest.mark.parametrize("fixture", ["mixed_layout_gate_fix.json",
                                     "mixed_layout_displaced.json"])
def test_mixed_layout_fixture_equals_per_subset(fixture):
    with open(os.path.join(GOLDEN, fixture)) as f:
        fx = json.load(f)
    T = fx["num_actual_tokens"]
    K = max(fx["spec_row_lens"])
    case = small_case(seed=50, K=K, T=T, num_slots=32)
    stix = np.array(fx["spec_token_indx"], np.int32)
    ntix = np.array(fx["non_spec_token_indx"], np.int32)
    # Extreme gates on the non-spec rows: reading a spec token's gates from a
    # non-spec row would change its output far beyond rounding.
    case["a"][ntix] = synth.to_bf16(np.full((len(ntix), case["a"].shape[1]), 20.0, np.float32))
    case["b"][ntix] = synth.to_bf16(np.full((len(ntix), case["b"].shape[1]), -20.0, np.float32))
    Ns = len(fx["spec_row_lens"])
    sqsl = np.concatenate([[0], np.cumsum(fx["spec_row_lens"])])
    ssi = np.arange(1, 1 + Ns * K, dtype=np.int32).reshape(Ns, K)
    nacc = np.array([1 + (i % K) for i in range(Ns)], np.int32)
    spec = spec_meta(sqsl, ssi, nacc, stix)
    ns_slots = list(range(Ns * K + 1, Ns * K + 1 + len(fx["non_spec_row_lens"])))
    ns = nonspec_meta(fx["non_spec_row_lens"], ns_slots, tix=ntix,
                      num_decodes=sum(1 for l in fx["non_spec_row_lens"] if l == 1))
    # mixed: non-spec call then spec call on the same pools and output
    o1, r1, s1, _ = run_nonspec(case, ns)
    c = clone(case)
    c["conv_state"], c["ssm_state"] = r1, s1
    mixed_out, mixed_ring, mixed_ssm, _ = run_spec(c, spec, out=o1)
    # per subset: the spec rows alone, contiguous
    sub = clone(case)
    for k in ("mixed_qkv", "a", "b"):
        sub[k] = np.ascontiguousarray(case[k][stix])
    sub["num_actual_tokens"] = len(stix)
    spec_c = spec_meta(sqsl, ssi, nacc)
    so, sr, ss, _ = run_spec(sub, spec_c)
    np.testing.assert_array_equal(mixed_out[stix], so)
    for s in ssi.ravel():
        np.testing.assert_array_equal(mixed_ssm[s], ss[s])
        np.testing.assert_array_equal(mixed_ring[s], sr[s])
    # and the non-spec rows alone
    nsub = clone(case)
    for k in ("mixed_qkv", "a", "b"):
        nsub[k] = np.ascontiguousarray(case[k][ntix])
    nsub["num_actual_tokens"] = len(ntix)
    no, nr, nss, _ = run_nonspec(nsub, nonspec_meta(fx["non_spec_row_lens"], ns_slots,
                                                    num_decodes=ns["num_decodes"]))
    np.testing.assert_array_equal(mixed_out[ntix], no)
    for s in ns_slots:
        np.testing.assert_array_equal(mixed_ssm[s], nss[s])
        np.testing.assert_array_equal(mixed_ring[s], nr[s])
    # rows are written only where mapped: every row is mapped here
    assert set(stix) | set(ntix) == set(range(T))


def test_gate_gather_regression_is_detected():
    # Reading gates at the stream index instead of the global row would
    # differ: emulate that mistake on the inputs and check the outputs move.
    with open(os.path.join(GOLDEN, "mixed_layout_gate_fix.json")) as f:
        fx = json.load(f)
    case = small_case(seed=51, K=3, T=4, num_slots=16)
    case["a"][0] = synth.to_bf16(np.full(case["a"].shape[1], 20.0, np.float32))
    case["b"][0] = synth.to_bf16(np.full(case["b"].shape[1], -20.0, np.float32))
    spec = spec_meta([0, 3], [[1, 2, 3]], [2], fx["spec_token_indx"])
    good, _, _, _ = run_spec(case, spec)
    wrong = clone(case)
    wrong["a"][1:4] = case["a"][0:3]
    wrong["b"][1:4] = case["b"][0:3]
    bad, _, _, _ = run_spec(wrong, spec)
    assert np.abs(f32(good[1:4]) - f32(bad[1:4])).max() > 2e-2


# --------------------------------------------------------------------------
# preconditions


def test_oracle_rejects_bad_metadata():
    case = small_case(seed=60, K=3, T=3)
    with pytest.raises(ValueError):
        run_spec(case, spec_meta([0, 3], [[1, 2, 3]], [0]))      # n_acc < 1
    with pytest.raises(ValueError):
        run_spec(case, spec_meta([0, 2], [[1, 2, 3]], [3]))      # n_acc > T_b
    with pytest.raises(ValueError):
        run_spec(case, spec_meta([0, 3], [[1, 2, 99]], [1]))     # slot >= num_slots
