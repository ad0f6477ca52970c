"""Invariants of the HIP path that need no oracle (GPU against GPU, bit for
bit): spec verify with all tokens accepted equals sequential decodes; K=1
spec equals a decode on a minimal ring; rollback equals decodes over the
accepted prefix; the stage entry points compose to the fused step; ten runs
are byte-identical; unit gates with orthonormal keys recall v exactly;
garbage metadata values stay inside the tensors; token_indx permutations and the mixed layouts printed on
the gate-fix page equal per-subset runs; a rejected call touches nothing."""
from __future__ import annotations

import json
import os

import numpy as np
import pytest
import torch

import synth
from tests import helpers
from tests.gpu_util import Gpu, dev, gpu_available, i32, say, u8

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU and libgdn.so")]

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def qcase(seed, K, T, num_slots=24, **kw):
    return helpers.small_case(seed=seed, Hk=4, Hv=8, dk=128, dv=128, K=K, T=T,
                              num_slots=num_slots, **kw)


@pytest.mark.parametrize("K", [2, 3, 4])
def test_all_accepted_spec_equals_sequential_decodes(K):
    case = qcase(100 + K, K, K)
    ssi = list(range(2, 2 + K))
    case["conv_state"][20] = case["conv_state"][ssi[0]]
    case["ssm_state"][20] = case["ssm_state"][ssi[K - 1]]
    case["spec"] = helpers.spec_meta([0, K], [ssi], [K])
    gs = Gpu(case)
    say(f"all-accepted spec K={K}")
    gs.spec()
    gd = Gpu(case)
    states = []
    for t in range(K):
        gd.decode_row(t, 20)
        states.append(gd.host_ssm([20])[0])
    np.testing.assert_array_equal(gs.host_out()[:K], gd.host_out()[:K])
    for t in range(K):
        np.testing.assert_array_equal(gs.host_ssm([ssi[t]])[0], states[t])
    np.testing.assert_array_equal(gs.host_conv([ssi[0]])[0], gd.host_conv([20])[0])


def test_k1_spec_equals_decode_on_minimal_ring():
    case = qcase(110, 1, 1)          # L = W - 1
    case["spec"] = helpers.spec_meta([0, 1], [[5]], [1])
    gs = Gpu(case)
    gs.spec()
    gd = Gpu(case)
    gd.decode_row(0, 5)
    np.testing.assert_array_equal(gs.host_out(), gd.host_out())
    np.testing.assert_array_equal(gs.host_conv(), gd.host_conv())
    np.testing.assert_array_equal(gs.host_ssm(), gd.host_ssm())


@pytest.mark.parametrize("n1,n2", [(1, 3), (2, 1), (3, 2)])
def test_rollback_equals_decodes_over_accepted_prefix(n1, n2):
    K = 3
    case = qcase(120 + n1, K, 3 * K)
    ssi = [3, 4, 5]
    case["conv_state"][20] = case["conv_state"][3]
    case["ssm_state"][20] = case["ssm_state"][5]
    g = Gpu(case)
    say(f"rollback n1={n1} n2={n2}")
    for n, base in ((K, 0), (n1, K), (n2, 2 * K)):
        g.spec(helpers.spec_meta([0, K], [ssi], [n], tix=list(range(base, base + K))))
    ref = Gpu(case)
    hist = list(range(0, n1)) + list(range(K, K + n2))
    for r in hist:
        ref.decode_row(r, 20)
    snap_conv, snap_ssm = ref.host_conv([20])[0], ref.host_ssm([20])[0]
    for t, r in enumerate(range(2 * K, 3 * K)):
        ref.decode_row(r, 20)
        np.testing.assert_array_equal(g.host_ssm([ssi[t]])[0], ref.host_ssm([20])[0])
    np.testing.assert_array_equal(g.host_out()[2 * K:], ref.host_out()[2 * K:])
    del snap_conv, snap_ssm


def _stage(g, kind, meta, T, conv_out, max_row_tokens):
    import speculative_decoding_causal_amd as gdn
    common = dict(kind=kind, query_start_loc=i32(meta["qsl"]), num_tokens=T,
                  max_row_tokens=max_row_tokens, cache_indices=i32(meta.get("cache")),
                  state_indices=i32(meta.get("ssi")),
                  num_accepted_tokens=i32(meta.get("nacc")),
                  has_initial_state=u8(meta.get("his")), token_indx=i32(meta.get("tix")))
    gdn.gdn_conv_only(g.cfg, g.qkv, g.w, g.bias, g.conv, conv_out, **common)
    gdn.gdn_delta_rule_only(g.cfg, conv_out, g.a, g.b, g.A_log, g.dt_bias, g.ssm, g.out,
                            state_len=g.case["dims"]["L"], **common)


def test_stage_entry_points_compose_to_fused_spec():
    import speculative_decoding_causal_amd as gdn
    K, Ns = 3, 4
    case = qcase(130, K, Ns * K)
    tix = np.random.default_rng(3).permutation(Ns * K).astype(np.int32)
    ssi = np.arange(1, 1 + Ns * K, dtype=np.int32).reshape(Ns, K)
    nacc = np.array([1, 2, 3, 2], np.int32)
    case["spec"] = helpers.spec_meta([0, 3, 6, 9, 12], ssi, nacc, tix)
    fused = Gpu(case)
    fused.spec()
    staged = Gpu(case)
    y = torch.zeros(Ns * K, staged.cfg.conv_dim, dtype=torch.float32, device=dev())
    _stage(staged, gdn.GDN_ROWS_SPEC, dict(qsl=[0, 3, 6, 9, 12], ssi=ssi, nacc=nacc, tix=tix),
           Ns * K, y, K)
    np.testing.assert_array_equal(fused.host_out(), staged.host_out())
    np.testing.assert_array_equal(fused.host_conv(), staged.host_conv())
    np.testing.assert_array_equal(fused.host_ssm(), staged.host_ssm())


def test_stage_entry_points_compose_to_fused_decode():
    import speculative_decoding_causal_amd as gdn
    case = qcase(131, 3, 5)
    fused = Gpu(case)
    slots, his = [2, 4, 6, 8, 10], [1, 0, 1, 1, 1]
    ns = helpers.nonspec_meta([1] * 5, slots, his=his)
    fused.attention(ns=ns, spec=None)
    staged = Gpu(case)
    y = torch.zeros(5, staged.cfg.conv_dim, dtype=torch.float32, device=dev())
    _stage(staged, gdn.GDN_ROWS_NON_SPEC, dict(qsl=[0, 1, 2, 3, 4, 5], cache=slots, his=his),
           5, y, 1)
    np.testing.assert_array_equal(fused.host_out(), staged.host_out())
    np.testing.assert_array_equal(fused.host_conv(), staged.host_conv())
    np.testing.assert_array_equal(fused.host_ssm(), staged.host_ssm())


@pytest.mark.parametrize("K", [1, 4])
def test_ten_runs_byte_identical(K):
    # Determinism (spec-decoding kernel page, "Test Plan"): 10 runs from the
    # same pools give byte-equal core_attn_out, conv_state and ssm_state.
    case = synth.make_case("small", seed=140 + K, K=K, Hv=32, num_slots=128, null_p=0.0)
    first = None
    for _ in range(10):
        g = Gpu(case)
        g.spec()
        got = (g.host_out(), g.host_conv(), g.host_ssm())
        if first is None:
            first = got
        else:
            for x, y in zip(first, got):
                assert x.tobytes() == y.tobytes()


def test_exact_recall_unit_gates_one_hot_keys():
    # With alpha = beta = 1 and orthonormal keys the delta rule writes token
    # t's value into column k_t alone: reading with q_t = k_t returns v_t
    # exactly (bf16 outputs bit-equal to v_t), and each stored state holds
    # the rank-one writes so far, v_s in column k_s, zeros elsewhere.  Run
    # through the delta-rule stage, which takes the conv output as given, on
    # spec rows with a NULL load slot and permuted tokens.
    import speculative_decoding_causal_amd as gdn
    K, Ns = 4, 2
    T = Ns * K
    case = qcase(150, K, T, use_qk_l2norm=0, scale=1.0)
    d = case["dims"]
    Hk, Hv, dk, dv = d["Hk"], d["Hv"], d["dk"], d["dv"]
    G, C = Hv // Hk, synth.conv_dim(Hk, Hv, dk, dv)
    rng = np.random.default_rng(151)
    # softplus(-100) is below fp32's smallest normal, so alpha = exp(-that)
    # rounds to 1; sigmoid(100) rounds to 1
    case["a"] = synth.to_bf16(np.full((T, Hv), -100.0, np.float32))
    case["b"] = synth.to_bf16(np.full((T, Hv), 100.0, np.float32))
    case["A_log"] = np.zeros(Hv, np.float32)
    case["dt_bias"] = np.zeros(Hv, np.float32)
    tix = rng.permutation(T).astype(np.int32)
    ssi = np.array([[0, 3, 4, 5], [0, 7, 8, 9]], np.int32)
    v = synth.from_bf16(synth.to_bf16(rng.standard_normal((T, Hv, dv)).astype(np.float32)))
    cols = rng.permuted(np.tile(np.arange(dk), (Ns, Hk, 1)), axis=2)[:, :, :K]
    y = np.zeros((T, C), np.float32)
    for bb in range(Ns):
        for t in range(K):
            r = tix[bb * K + t]
            for i in range(Hk):
                y[r, i * dk + cols[bb, i, t]] = 1.0            # q
                y[r, (Hk + i) * dk + cols[bb, i, t]] = 1.0     # k
            y[r, 2 * Hk * dk:] = v[bb * K + t].reshape(-1)
    g = Gpu(case)
    say("exact recall, delta-rule stage")
    gdn.gdn_delta_rule_only(g.cfg, torch.from_numpy(y).to(dev()), g.a, g.b, g.A_log, g.dt_bias,
                            g.ssm, g.out, kind=gdn.GDN_ROWS_SPEC,
                            query_start_loc=i32([0, K, 2 * K]), num_tokens=T,
                            max_row_tokens=K, state_indices=i32(ssi),
                            num_accepted_tokens=i32([1] * Ns), token_indx=i32(tix),
                            state_len=d["L"])
    out = g.host_out()  # raw bf16 bits
    for j in range(T):
        np.testing.assert_array_equal(out[tix[j]], synth.to_bf16(v[j]))
    for bb in range(Ns):
        got = g.host_ssm(ssi[bb, 1:])
        for t in range(1, K):
            want = np.zeros((Hv, dv, dk), np.float32)
            for s in range(t + 1):
                for h in range(Hv):
                    want[h, :, cols[bb, h // G, s]] = v[bb * K + s, h]
            np.testing.assert_array_equal(got[t - 1], want)


def _guarded(t, fill, guard=8192):
    # t's values inside a buffer with `guard` canary elements on each side
    n = t.numel()
    buf = torch.full((n + 2 * guard,), fill, dtype=t.dtype, device=t.device)
    buf[guard:guard + n].copy_(t.reshape(-1))
    return buf, buf[guard:guard + n].view(t.shape)


def _guards_intact(buf, n, fill, guard=8192):
    want = torch.full((guard,), fill, dtype=buf.dtype, device=buf.device)
    return torch.equal(buf[:guard], want) and torch.equal(buf[guard + n:], want)


def _junk(rng, n, lo, hi):
    # per element one of: in range, any int32, -1, the first value past the
    # range, small values around zero
    pools = [rng.integers(lo, hi, n), rng.integers(-2 ** 31, 2 ** 31 - 1, n),
             np.full(n, -1), np.full(n, hi), rng.integers(-5, 5, n)]
    pick = rng.integers(0, len(pools), n)
    return np.array([pools[k][i] for i, k in enumerate(pick)], np.int32)


@pytest.mark.parametrize("seed,decodes,prefill,dk,per_token,Ns,K",
                         [(0, 0, 0, 128, 0, 16, 3), (1, 0, 0, 128, 0, 16, 3),
                          (2, 0, 0, 128, 0, 16, 3), (3, 5, 0, 128, 0, 16, 3),
                          (4, 5, 0, 128, 0, 16, 3), (5, 3, 150, 128, 0, 16, 3),
                          (6, 3, 150, 32, 0, 16, 3), (7, 0, 300, 64, 0, 16, 3),
                          (8, 0, 0, 128, 1, 16, 3), (9, 4, 0, 64, 1, 16, 3),
                          (10, 0, 0, 128, 0, 96, 4), (11, 6, 0, 128, 0, 96, 4),
                          (12, 0, 0, 128, 1, 96, 4)])
def test_garbage_metadata_stays_in_bounds(seed, decodes, prefill, dk, per_token, Ns, K):
    # Metadata values live in device memory and are not checked by the step
    # (the host checker is separate): the kernels clamp query_start_loc,
    # slots, num_accepted_tokens and token rows, so any values leave the
    # results unspecified but every access inside the tensors.  Checked with
    # canaries around the pools, the output and the turn counters; 96 rows
    # of four tokens and 32 v-heads take the (row, v-head) form, where
    # garbage slots put many rows on one counter, and every counter must
    # still be back at 0.
    import speculative_decoding_causal_amd as gdn
    T = Ns * K
    nprefills = 3 if prefill else 0
    nns = decodes + prefill           # the prefill rows share `prefill` tokens
    Hk, Hv = (16, 32) if Ns > 16 else (4, 8)
    case = helpers.small_case(seed=160 + seed, Hk=Hk, Hv=Hv, dk=dk, dv=dk, K=K, T=T + nns,
                              num_slots=24, L=3 if per_token else None)
    d = case["dims"]
    d["conv_layout"] = per_token       # per-token conv slots: one window per slot
    rng = np.random.default_rng(170 + seed)
    g = Gpu(case)
    conv_buf, conv = _guarded(g.conv, 0.5)
    ssm_buf, ssm = _guarded(g.ssm, 0.5)
    out_buf, out = _guarded(g.out, 0.5)
    turns_buf, turns = _guarded(g.turns, 0x5A5A5A5A)
    ws_buf = ws = None
    if nprefills:
        nbytes = gdn.gdn_workspace_bytes(g.cfg, d["L"], d["num_slots"], nns, nprefills)
        ws_buf, ws = _guarded(torch.zeros(nbytes, dtype=torch.uint8, device=dev()), 0x5A)
    spec = dict(spec_query_start_loc=i32(_junk(rng, Ns + 1, 0, T + 1)),
                spec_state_indices=i32(_junk(rng, Ns * K, 0, d["num_slots"]).reshape(Ns, K)),
                num_accepted_tokens=i32(_junk(rng, Ns, 1, K + 1)),
                spec_cache_indices=None if per_token else i32(_junk(rng, Ns, 0,
                                                                    d["num_slots"])),
                spec_token_indx=i32(_junk(rng, T, 0, T + nns)))
    say(f"garbage metadata seed={seed} decodes={decodes}")
    if decodes + nprefills == 0:
        gdn.gdn_spec_attention(g.cfg, g.qkv, g.a, g.b, g.w, None, g.A_log, g.dt_bias, conv, ssm,
                               spec["spec_query_start_loc"], spec["spec_state_indices"],
                               spec["num_accepted_tokens"], out,
                               spec_cache_indices=spec["spec_cache_indices"],
                               spec_token_indx=spec["spec_token_indx"], num_spec_tokens=T,
                               conv_turns=turns)
    else:
        rows = decodes + nprefills
        gdn.gdn_attention(g.cfg, g.qkv, g.a, g.b, g.w, None, g.A_log, g.dt_bias, conv, ssm, out,
                          num_decodes=decodes, num_prefills=nprefills, num_non_spec_tokens=nns,
                          query_start_loc=i32(_junk(rng, rows + 1, 0, nns + 1)),
                          non_spec_state_indices=i32(_junk(rng, rows, 0, d["num_slots"])),
                          has_initial_state=u8(rng.integers(0, 2, rows)),
                          non_spec_token_indx=i32(_junk(rng, nns, 0, T + nns)),
                          num_spec_tokens=T, workspace=ws, conv_turns=turns, **spec)
    torch.cuda.synchronize()
    if ws is not None:
        assert _guards_intact(ws_buf, ws.numel(), 0x5A)
    assert _guards_intact(turns_buf, turns.numel(), 0x5A5A5A5A)
    assert bool((turns == 0).all())
    assert _guards_intact(conv_buf, conv.numel(), 0.5)
    assert _guards_intact(ssm_buf, ssm.numel(), 0.5)
    assert _guards_intact(out_buf, out.numel(), 0.5)


def test_token_permutation_invariance():
    case = synth.make_case("small", seed=150)
    T = case["num_actual_tokens"]
    a = Gpu(case)
    a.spec()
    perm = np.random.default_rng(5).permutation(T)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(T)
    c2 = helpers.clone(case)
    for k in ("mixed_qkv", "a", "b"):
        c2[k] = np.ascontiguousarray(case[k][inv])
    c2["spec"]["spec_token_indx"] = perm.astype(np.int32)
    b = Gpu(c2)
    b.spec()
    np.testing.assert_array_equal(b.host_out()[perm], a.host_out())
    np.testing.assert_array_equal(a.host_conv(), b.host_conv())
    np.testing.assert_array_equal(a.host_ssm(), b.host_ssm())


@pytest.mark.parametrize("fixture", ["mixed_layout_gate_fix.json", "mixed_layout_displaced.json"])
def test_mixed_layout_fixture_equals_per_subset(fixture):
    with open(os.path.join(GOLDEN, fixture)) as f:
        fx = json.load(f)
    T = fx["num_actual_tokens"]
    K = max(fx["spec_row_lens"])
    case = qcase(160, K, T, num_slots=40)
    stix = np.array(fx["spec_token_indx"], np.int32)
    ntix = np.array(fx["non_spec_token_indx"], np.int32)
    Hv = case["a"].shape[1]
    case["a"][ntix] = synth.to_bf16(np.full((len(ntix), Hv), 20.0, np.float32))
    case["b"][ntix] = synth.to_bf16(np.full((len(ntix), Hv), -20.0, np.float32))
    Ns = len(fx["spec_row_lens"])
    sqsl = np.concatenate([[0], np.cumsum(fx["spec_row_lens"])]).astype(np.int32)
    ssi = np.arange(1, 1 + Ns * K, dtype=np.int32).reshape(Ns, K)
    nacc = np.array([1 + (i % K) for i in range(Ns)], np.int32)
    ns_slots = list(range(Ns * K + 1, Ns * K + 1 + len(fx["non_spec_row_lens"])))
    nd = sum(1 for l in fx["non_spec_row_lens"] if l == 1)
    case["spec"] = helpers.spec_meta(sqsl, ssi, nacc, stix)
    case["nonspec"] = helpers.nonspec_meta(fx["non_spec_row_lens"], ns_slots, tix=ntix,
                                           num_decodes=nd)
    mixed = Gpu(case)
    say(f"mixed fixture {fixture}")
    mixed.attention()
    sub = helpers.clone(case)
    for k in ("mixed_qkv", "a", "b"):
        sub[k] = np.ascontiguousarray(case[k][stix])
    sub["num_actual_tokens"] = len(stix)
    sub["spec"] = helpers.spec_meta(sqsl, ssi, nacc)
    gs = Gpu(sub)
    gs.spec()
    np.testing.assert_array_equal(mixed.host_out()[stix], gs.host_out())
    sl = ssi.ravel()
    np.testing.assert_array_equal(mixed.host_ssm(sl), gs.host_ssm(sl))
    np.testing.assert_array_equal(mixed.host_conv(sl), gs.host_conv(sl))
    nsub = helpers.clone(case)
    for k in ("mixed_qkv", "a", "b"):
        nsub[k] = np.ascontiguousarray(case[k][ntix])
    nsub["num_actual_tokens"] = len(ntix)
    nsub["spec"] = None
    nsub["nonspec"] = helpers.nonspec_meta(fx["non_spec_row_lens"], ns_slots, num_decodes=nd)
    gn = Gpu(nsub)
    gn.attention()
    np.testing.assert_array_equal(mixed.host_out()[ntix], gn.host_out())
    np.testing.assert_array_equal(mixed.host_ssm(ns_slots), gn.host_ssm(ns_slots))
    np.testing.assert_array_equal(mixed.host_conv(ns_slots), gn.host_conv(ns_slots))


def test_rejected_call_touches_nothing():
    import speculative_decoding_causal_amd as gdn
    case = synth.make_case("tiny", seed=170)
    g = Gpu(case)
    before = (g.host_out(), g.host_conv(), g.host_ssm())
    sp = case["spec"]
    with pytest.raises(gdn.GdnError) as e:
        gdn.gdn_spec_attention(g.cfg, g.qkv, g.a, g.b, g.w, None, g.A_log, g.dt_bias, g.conv,
                               g.ssm, i32(sp["spec_query_start_loc"]),
                               i32(sp["spec_state_indices"]), None, g.out,
                               num_spec_tokens=sp["num_spec_tokens"])
    assert e.value.status == gdn.GDN_ERR_SPEC_PAIR
    torch.cuda.synchronize()
    after = (g.host_out(), g.host_conv(), g.host_ssm())
    for x, y in zip(before, after):
        assert x.tobytes() == y.tobytes()


@pytest.mark.parametrize("name", ["tiny", "small", "qwen3next_k3_b64", "mixed"])
def test_generated_metadata_passes_host_checker(name):
    import speculative_decoding_causal_amd as gdn
    case = synth.make_case(name, seed=0, with_pools=False)
    d, sp, ns = case["dims"], case["spec"], case.get("nonspec") or {}
    cfg = gdn.GdnConfig(d["Hk"], d["Hv"], d["dk"], d["dv"], d["W"])
    rc = gdn.gdn_check_metadata_host(
        cfg, d["L"], d["num_slots"], case["num_actual_tokens"],
        num_decodes=ns.get("num_decodes", 0), num_prefills=ns.get("num_prefills", 0),
        num_non_spec_tokens=ns.get("num_non_spec_tokens", 0),
        num_spec_tokens=sp["num_spec_tokens"],
        query_start_loc=ns.get("query_start_loc"),
        non_spec_state_indices=ns.get("cache_indices"),
        non_spec_token_indx=ns.get("token_indx"),
        spec_query_start_loc=sp["spec_query_start_loc"],
        spec_state_indices=sp["spec_state_indices"],
        num_accepted_tokens=sp["num_accepted_tokens"],
        spec_token_indx=sp["spec_token_indx"])
    assert rc == gdn.GDN_OK, gdn.gdn_last_error()
