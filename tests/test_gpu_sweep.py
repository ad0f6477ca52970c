"""Seeded random sweep of the HIP path against the oracle: each case draws
its head size, head grouping, K, ring length, row count, ragged row lengths,
NULL-slot density and token order (spec batches), or its decodes and
prefill lengths around the 64-token chunk edges (mixed batches), so that
combinations the targeted tests pin one axis at a time also meet.  Every
draw is printed before it runs; the seeds are fixed, so a failure names a
case that reruns exactly."""
from __future__ import annotations

import numpy as np
import pytest

import synth
from tests import helpers
from tests.gpu_util import (Gpu, assert_out_close, assert_states_close, gpu_available, say,
                            spec_rows_of)
from tests.test_gpu_parity import check_spec_case

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU and libgdn.so")]

W = 4


def _heads(rng, dk):
    Hk = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 4, 8]))   # up to 1024 state rows per k-head at dk 128
    return Hk, Hk * G


def _fit_lds(K, dk, Hk, Hv, k_max_at_1024_rows):
    # 1024 state rows per k-head (dk 128, 8 v-heads per k-head) stage 8 KiB
    # of v and outputs per token in LDS: longer rows exceed it and are
    # rejected (GDN_ERR_UNSUPPORTED), so the draw keeps them within it
    return min(K, k_max_at_1024_rows) if dk * (Hv // Hk) == 1024 else K


def spec_draw(seed):
    rng = np.random.default_rng(7000 + seed)
    dk = int(rng.choice([16, 32, 64, 128]))
    Hk, Hv = _heads(rng, dk)
    K = _fit_lds(int(rng.integers(1, 7)), dk, Hk, Hv, 8)
    L = min(W - 1 + K - 1 + int(rng.choice([0, 1, 3])), 16)
    Ns = int(rng.integers(1, 11))
    ragged = bool(rng.integers(0, 2))
    lens = [int(x) for x in rng.integers(1, K + 1, size=Ns)] if ragged else None
    return dict(dk=dk, dv=dk, Hk=Hk, Hv=Hv, K=K, L=L, Ns=Ns, lens=lens,
                null_p=float(rng.choice([0.0, 0.15])), num_slots=128,
                permute=bool(rng.integers(0, 2)))


def mixed_draw(seed):
    rng = np.random.default_rng(9000 + seed)
    dk = int(rng.choice([16, 32, 64, 128]))
    Hk, Hv = _heads(rng, dk)
    K = int(rng.integers(2, 5))
    Np = int(rng.integers(1, 3))
    plens = tuple(int(x) for x in rng.choice([1, 17, 63, 64, 65, 130], size=Np))
    return dict(dk=dk, dv=dk, Hk=Hk, Hv=Hv, K=K, Ns=int(rng.integers(1, 9)),
                Nd=int(rng.integers(0, 9)), prefill_lens=plens, num_slots=128)


@pytest.mark.parametrize("seed", range(24))
def test_spec_sweep(seed):
    d = spec_draw(seed)
    say(f"spec sweep {seed}: {d}")
    over = {k: v for k, v in d.items() if k not in ("permute", "lens")}
    if d["lens"] is not None:
        over["lens"] = d["lens"]
    case = synth.make_case("small", seed=seed, permute_tokens=d["permute"], **over)
    check_spec_case(case)


@pytest.mark.parametrize("seed", range(10))
def test_mixed_sweep(seed):
    d = mixed_draw(seed)
    say(f"mixed sweep {seed}: {d}")
    case = synth.make_case("mixed", seed=seed, **d)
    o1, r1, s1, _ = helpers.run_nonspec(case)
    c = helpers.clone(case)
    c["conv_state"], c["ssm_state"] = r1, s1
    out_ref, conv_ref, ssm_ref, _ = helpers.run_spec(c, out=o1)
    g = Gpu(case)
    g.attention()
    assert_out_close(g.host_out(), out_ref)
    slots = synth.referenced_slots(case)
    np.testing.assert_array_equal(g.host_conv(slots), conv_ref[slots])
    assert_states_close(g.host_ssm(slots), ssm_ref[slots])


# ---- wider draws: layer options, the per-k-head input layout, long rows ----

def _options(case, rng):
    """Conv bias, identity activation and unnormalised q/k, each with p=1/2
    (unnormalised keys are scaled so that |k|^2 < 1 keeps the recurrence
    stable)."""
    d = case["dims"]
    d["activation"] = int(rng.integers(0, 2))
    d["use_qk_l2norm"] = int(rng.integers(0, 2))
    C = synth.conv_dim(d["Hk"], d["Hv"], d["dk"], d["dv"])
    bias = bool(rng.integers(0, 2))
    if bias:
        case["conv_bias"] = synth.to_bf16(0.5 * rng.standard_normal(C).astype(np.float32))
    if not d["use_qk_l2norm"]:
        case["conv_weight"] = synth.to_bf16(synth.from_bf16(case["conv_weight"]) / 16.0)
        if bias:
            case["conv_bias"] = synth.to_bf16(synth.from_bf16(case["conv_bias"]) / 16.0)
    return dict(act=d["activation"], l2norm=d["use_qk_l2norm"], bias=bias)


def _gpu(case, per_k_head):
    """The HIP path on the case, reading mixed_qkv in the per-k-head order
    (repacked, reorder_input off) when asked; pools and outputs keep the
    grouped channel order either way."""
    if not per_k_head:
        return Gpu(case)
    import dataclasses
    from tests.test_layout import per_k_head as repack
    d = case["dims"]
    inter = dict(case)
    inter["mixed_qkv"] = repack(case["mixed_qkv"], d["Hk"], d["Hv"], d["dk"], d["dv"])
    g = Gpu(inter)
    g.cfg = dataclasses.replace(g.cfg, reorder_input=False)
    return g


def wide_spec_draw(seed):
    rng = np.random.default_rng(11000 + seed)
    dk = int(rng.choice([16, 32, 64, 128]))
    Hk, Hv = _heads(rng, dk)
    K = _fit_lds(int(rng.choice([1, 2, 3, 4, 6, 8, 11, 14])), dk, Hk, Hv, 8)
    L = min(W - 1 + K - 1 + int(rng.choice([0, 0, 2])), 16)
    Ns = int(rng.integers(1, 9))
    lens = [int(x) for x in rng.integers(1, K + 1, size=Ns)] if rng.integers(0, 2) else None
    return rng, dict(dk=dk, dv=dk, Hk=Hk, Hv=Hv, K=K, L=L, Ns=Ns, lens=lens,
                     null_p=float(rng.choice([0.0, 0.2])), num_slots=128,
                     permute=bool(rng.integers(0, 2)), per_k_head=bool(rng.integers(0, 2)))


@pytest.mark.parametrize("seed", range(32))
def test_spec_sweep_wide(seed):
    rng, d = wide_spec_draw(seed)
    over = {k: v for k, v in d.items() if k not in ("permute", "lens", "per_k_head")}
    if d["lens"] is not None:
        over["lens"] = d["lens"]
    case = synth.make_case("small", seed=seed, permute_tokens=d["permute"], **over)
    opts = _options(case, rng)
    say(f"wide spec sweep {seed}: {d} {opts}")
    sp = case["spec"]
    out_ref, conv_ref, ssm_ref, _ = helpers.run_spec(case, sp)
    g = _gpu(case, d["per_k_head"])
    g.spec()
    rows = list(range(sp["num_spec_decodes"]))
    glob, slots = spec_rows_of(sp, rows)
    assert_out_close(g.host_out(), out_ref, glob)
    np.testing.assert_array_equal(g.host_conv(slots), conv_ref[slots])
    assert_states_close(g.host_ssm(slots), ssm_ref[slots])


@pytest.mark.parametrize("seed", range(16))
def test_mixed_sweep_wide(seed):
    rng = np.random.default_rng(13000 + seed)
    d = mixed_draw(100 + seed)
    case = synth.make_case("mixed", seed=100 + seed, **d)
    opts = _options(case, rng)
    pkh = bool(rng.integers(0, 2))
    say(f"wide mixed sweep {seed}: {d} {opts} per_k_head={pkh}")
    o1, r1, s1, _ = helpers.run_nonspec(case)
    c = helpers.clone(case)
    c["conv_state"], c["ssm_state"] = r1, s1
    out_ref, conv_ref, ssm_ref, _ = helpers.run_spec(c, out=o1)
    g = _gpu(case, pkh)
    g.attention()
    assert_out_close(g.host_out(), out_ref)
    slots = synth.referenced_slots(case)
    np.testing.assert_array_equal(g.host_conv(slots), conv_ref[slots])
    assert_states_close(g.host_ssm(slots), ssm_ref[slots])


@pytest.mark.parametrize("seed", range(12))
def test_per_token_slots_sweep(seed):
    # the per-token conv-slot contract (one window per token slot, L = W-1)
    from tests.test_gpu_per_token import per_token_case
    rng = np.random.default_rng(15000 + seed)
    dk = int(rng.choice([16, 32, 64, 128]))
    Hk, Hv = _heads(rng, dk)
    K = _fit_lds(int(rng.choice([1, 2, 3, 4, 6, 8, 12, 16])), dk, Hk, Hv, 12)   # ring: W-1
    Ns = int(rng.integers(1, 9))
    null_p = float(rng.choice([0.0, 0.2]))
    say(f"per-token slots sweep {seed}: dk={dk} Hk={Hk} Hv={Hv} K={K} Ns={Ns} null_p={null_p}")
    check_spec_case(per_token_case(15000 + seed, Ns=Ns, K=K, null_p=null_p, Hk=Hk, Hv=Hv, dk=dk))


@pytest.mark.parametrize("seed", range(12))
def test_stage_composition_sweep(seed):
    # gdn_conv_only then gdn_delta_rule_only give the fused spec step bit for
    # bit (the stage kernels read their stage at run time)
    import torch
    import speculative_decoding_causal_amd as gdn
    from tests.gpu_util import dev
    from tests.test_gpu_invariants import _stage
    d = spec_draw(100 + seed)
    over = {k: v for k, v in d.items() if k not in ("permute", "lens")}
    if d["lens"] is not None:
        over["lens"] = d["lens"]
    case = synth.make_case("small", seed=100 + seed, permute_tokens=d["permute"], **over)
    sp = case["spec"]
    say(f"stage composition sweep {seed}: {d}")
    fused = Gpu(case)
    fused.spec()
    staged = Gpu(case)
    T = sp["num_spec_tokens"]
    y = torch.zeros(staged.qkv.shape[0], staged.cfg.conv_dim, dtype=torch.float32, device=dev())
    meta = dict(qsl=sp["spec_query_start_loc"], ssi=sp["spec_state_indices"],
                nacc=sp["num_accepted_tokens"], tix=sp.get("spec_token_indx"),
                cache=sp.get("spec_cache_indices"))
    _stage(staged, gdn.GDN_ROWS_SPEC, meta, T, y, sp["spec_state_indices"].shape[1])
    np.testing.assert_array_equal(fused.host_out(), staged.host_out())
    np.testing.assert_array_equal(fused.host_conv(), staged.host_conv())
    np.testing.assert_array_equal(fused.host_ssm(), staged.host_ssm())


@pytest.mark.parametrize("seed", range(12))
def test_nonspec_only_sweep(seed):
    # decodes and prefills with no spec rows: the decodes launch alone, before
    # the prefill kernels; prefill lengths up to past 1024 tokens
    rng = np.random.default_rng(17000 + seed)
    dk = int(rng.choice([16, 32, 64, 128]))
    Hk, Hv = _heads(rng, dk)
    Np = int(rng.integers(1, 4))
    plens = tuple(int(x) for x in rng.choice([1, 2, 63, 64, 65, 129, 300, 1025], size=Np))
    d = dict(dk=dk, dv=dk, Hk=Hk, Hv=Hv, K=2, Ns=0, Nd=int(rng.integers(0, 9)),
             prefill_lens=plens, num_slots=64)
    say(f"non-spec only sweep {seed}: {d}")
    case = synth.make_case("mixed", seed=17000 + seed, **d)
    out_ref, conv_ref, ssm_ref, _ = helpers.run_nonspec(case)
    g = Gpu(case)
    g.attention(spec=None)
    ns = case["nonspec"]
    rows = ns["token_indx"]
    assert_out_close(g.host_out()[rows], out_ref[rows])
    slots = synth.referenced_slots(case)
    np.testing.assert_array_equal(g.host_conv(slots), conv_ref[slots])
    assert_states_close(g.host_ssm(slots), ssm_ref[slots])


@pytest.mark.parametrize("seed", range(6))
def test_spec_many_rows_sweep(seed):
    # hundreds of rows on small heads: grids far larger than one per CU,
    # slot and token indices in the thousands
    rng = np.random.default_rng(19000 + seed)
    dk = int(rng.choice([16, 32]))
    Hk, Hv = _heads(rng, dk)
    K = int(rng.integers(1, 5))
    Ns = int(rng.integers(100, 301))
    d = dict(dk=dk, dv=dk, Hk=Hk, Hv=Hv, K=K, Ns=Ns, num_slots=Ns * K + 9,
             null_p=float(rng.choice([0.0, 0.1])))
    say(f"many-row spec sweep {seed}: {d}")
    check_spec_case(synth.make_case("small", seed=19000 + seed, permute_tokens=True, **d))


@pytest.mark.parametrize("seed", range(16))
def test_conv_width_sweep(seed):
    # conv widths 1 .. 4 (width 1 has no history ring: L = 0 is allowed)
    rng = np.random.default_rng(23000 + seed)
    Wc = int(rng.integers(1, 5))
    dk = int(rng.choice([16, 32, 64, 128]))
    Hk, Hv = _heads(rng, dk)
    if seed % 2 == 0:
        K = int(rng.integers(1, 5))
        L = min(Wc - 1 + K - 1 + int(rng.choice([0, 2])), 16)
        d = dict(dk=dk, dv=dk, Hk=Hk, Hv=Hv, K=K, L=L, W=Wc, Ns=int(rng.integers(1, 9)),
                 null_p=0.1, num_slots=64)
        say(f"conv width sweep {seed} (spec): {d}")
        check_spec_case(synth.make_case("small", seed=23000 + seed, permute_tokens=True, **d))
        return
    plens = tuple(int(x) for x in rng.choice([1, 2, 3, 17, 64, 65], size=int(rng.integers(1, 3))))
    K = int(rng.integers(1, 4))
    d = dict(dk=dk, dv=dk, Hk=Hk, Hv=Hv, K=K, L=Wc - 1 + K - 1, W=Wc, Ns=int(rng.integers(0, 5)),
             Nd=int(rng.integers(0, 5)), prefill_lens=plens, num_slots=64)
    say(f"conv width sweep {seed} (mixed): {d}")
    case = synth.make_case("mixed", seed=23000 + seed, **d)
    o1, r1, s1, _ = helpers.run_nonspec(case)
    c = helpers.clone(case)
    c["conv_state"], c["ssm_state"] = r1, s1
    out_ref, conv_ref, ssm_ref, _ = (helpers.run_spec(c, out=o1) if d["Ns"] else
                                     (o1, r1, s1, None))
    g = Gpu(case)
    g.attention(spec="case" if d["Ns"] else None)
    rows = np.concatenate([case["nonspec"]["token_indx"], case["spec"]["spec_token_indx"]])
    assert_out_close(g.host_out()[rows], out_ref[rows])
    slots = synth.referenced_slots(case)
    np.testing.assert_array_equal(g.host_conv(slots), conv_ref[slots])
    assert_states_close(g.host_ssm(slots), ssm_ref[slots])


@pytest.mark.parametrize("kind", ["spec", "mixed"])
def test_width_one_without_ring(kind):
    # conv width 1 with state_len 0: the conv pool holds no bytes (its
    # pointer is NULL) and the step still matches the oracle
    d = dict(W=1, K=1, L=0, Hk=2, Hv=4, dk=32, dv=32, num_slots=32)
    say(f"width-1 conv without a ring ({kind})")
    if kind == "spec":
        check_spec_case(synth.make_case("small", seed=25000, Ns=6, permute_tokens=True, **d))
        return
    case = synth.make_case("mixed", seed=25001, Ns=3, Nd=3, prefill_lens=(17, 65), **d)
    o1, r1, s1, _ = helpers.run_nonspec(case)
    c = helpers.clone(case)
    c["conv_state"], c["ssm_state"] = r1, s1
    out_ref, _, ssm_ref, _ = helpers.run_spec(c, out=o1)
    g = Gpu(case)
    g.attention()
    assert_out_close(g.host_out(), out_ref)
    slots = synth.referenced_slots(case)
    assert_states_close(g.host_ssm(slots), ssm_ref[slots])
