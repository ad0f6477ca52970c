"""Parity of the HIP path (through the C ABI) with the CPU oracle on seeded
synthetic workloads: the tiny and small spec batches, the Qwen3-Next-shaped
K=3 batch-64 verify step (identity and permuted token_indx), the deep K=4
batch-256 step (every row), ragged and edge-case batches,
and the mixed batch (spec rows + decodes + two 1024-token prefills in a
shuffled token order).  Bit-exact on the conv ring and slot bookkeeping;
bf16 outputs within 2e-2; fp32 states within 1e-3 relative per tile."""
from __future__ import annotations

import numpy as np
import pytest

import synth
from tests import helpers
from tests.gpu_util import (Gpu, assert_out_close, assert_states_close, gpu_available,
                            OUT_CANARY, say, spec_rows_of, sub_spec)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU and libgdn.so")]


def check_spec_case(case, sample_rows=None):
    """Run the whole batch on the GPU; the oracle runs every row (or the
    sampled rows) and the two are compared on those rows and their slots."""
    sp = case["spec"]
    rows = list(range(sp["num_spec_decodes"])) if sample_rows is None else list(sample_rows)
    ref_spec = sp if sample_rows is None else sub_spec(sp, rows)
    out_ref, conv_ref, ssm_ref, _ = helpers.run_spec(case, ref_spec)
    g = Gpu(case)
    say(f"spec {case.get('name')} rows={sp['num_spec_decodes']} T={sp['num_spec_tokens']}")
    g.spec()
    glob, slots = spec_rows_of(sp, rows)
    out = g.host_out()
    assert_out_close(out, out_ref, glob)
    if sample_rows is None:
        rest = np.setdiff1d(np.arange(len(out)), glob)
        assert (out[rest] == OUT_CANARY).all(), "rows outside token_indx were written"
    conv_slots = slots
    np.testing.assert_array_equal(g.host_conv(conv_slots), conv_ref[conv_slots])
    assert_states_close(g.host_ssm(slots), ssm_ref[slots])
    # a few slots nobody names keep their bytes
    free = np.setdiff1d(np.arange(1, case["dims"]["num_slots"]),
                        synth.referenced_slots(case))[:8]
    if len(free):
        np.testing.assert_array_equal(g.host_conv(free), case["conv_state"][free])
        np.testing.assert_array_equal(g.host_ssm(free), case["ssm_state"][free])
    np.testing.assert_array_equal(g.host_conv([0]), case["conv_state"][[0]])
    np.testing.assert_array_equal(g.host_ssm([0]), case["ssm_state"][[0]])
    return g


@pytest.mark.parametrize("name,seed", [("tiny", 0), ("tiny", 1), ("small", 0), ("small", 1)])
def test_spec_small_workloads(name, seed):
    check_spec_case(synth.make_case(name, seed=seed))


@pytest.mark.parametrize("permute", [False, True])
def test_spec_qwen3next_k3_b64(permute):
    check_spec_case(synth.make_case("qwen3next_k3_b64", seed=3, permute_tokens=permute))


def test_spec_qwen3next_k3_b64_tp2():
    # the batch at one GPU's share of a two-way head split (8/16 heads)
    check_spec_case(synth.make_case("qwen3next_k3_b64_tp2", seed=5, permute_tokens=True))


def test_spec_deep_k4_b256():
    # every one of the 256 rows against the oracle (the generator forces at
    # least one all-rejected row, n_acc = 1)
    case = synth.make_case("deep_k4_b256", seed=4)
    assert (case["spec"]["num_accepted_tokens"] == 1).any()
    check_spec_case(case)


@pytest.mark.parametrize("lens", [[3, 1, 2, 3, 1, 1, 2, 3, 2], [1] * 7, [4, 4, 1, 3]])
def test_spec_ragged_rows(lens):
    # Short rows (a request that accepted no draft gets fewer tokens; no
    # rectangular assumption) with the tail row shorter than K.
    K = max(lens)
    case = synth.make_case("small", seed=7, K=K, Ns=len(lens), lens=lens, null_p=0.0,
                           Hv=32, num_slots=64)
    check_spec_case(case)


@pytest.mark.parametrize("rung", ["K1_full", "K4_full", "K3_nacc1", "K4_min1_max1"])
def test_spec_page_rungs(rung):
    # The acceptance rungs the replay harness reports (spec-decoding kernel
    # page, "Test Result"): fully accepted K=1 and K=4, n_acc=1 with K=3,
    # and a K=4 batch where every row has n_acc=1.
    K = {"K1_full": 1, "K4_full": 4, "K3_nacc1": 3, "K4_min1_max1": 4}[rung]
    case = synth.make_case("small", seed=11, K=K, Ns=12, Hv=32, num_slots=128, null_p=0.0)
    sp = case["spec"]
    if rung.endswith("full"):
        sp["num_accepted_tokens"][:] = K
    else:
        sp["num_accepted_tokens"][:] = 1
    check_spec_case(case)


def test_spec_null_slots_everywhere():
    case = synth.make_case("small", seed=12, null_p=0.6)
    check_spec_case(case)


def test_spec_unmapped_rows_untouched():
    # num_actual_tokens larger than the spec stream: other rows keep their bytes.
    case = synth.make_case("small", seed=13)
    T = case["num_actual_tokens"]
    extra = 5
    for k in ("mixed_qkv", "a", "b"):
        case[k] = np.concatenate([case[k], case[k][:extra]])
    case["num_actual_tokens"] = T + extra
    perm = np.random.default_rng(0).permutation(T + extra)[:T].astype(np.int32)
    case["spec"]["spec_token_indx"] = perm
    g = check_spec_case(case)
    untouched = np.setdiff1d(np.arange(T + extra), perm)
    assert (g.host_out()[untouched] == OUT_CANARY).all()


def test_mixed_batch_parity():
    case = synth.make_case("mixed", seed=5)
    o1, r1, s1, _ = helpers.run_nonspec(case)
    c = helpers.clone(case)
    c["conv_state"], c["ssm_state"] = r1, s1
    out_ref, conv_ref, ssm_ref, _ = helpers.run_spec(c, out=o1)
    g = Gpu(case)
    say("mixed: 32 spec rows + 32 decodes + 2x1024 prefill")
    g.attention()
    out = g.host_out()
    assert_out_close(out, out_ref)
    slots = synth.referenced_slots(case)
    np.testing.assert_array_equal(g.host_conv(slots), conv_ref[slots])
    assert_states_close(g.host_ssm(slots), ssm_ref[slots])
    free = np.setdiff1d(np.arange(1, case["dims"]["num_slots"]), slots)[:8]
    np.testing.assert_array_equal(g.host_ssm(free), case["ssm_state"][free])


@pytest.mark.parametrize("lens,his", [([1, 1, 63, 64, 65], [1, 0, 1, 0, 1]),
                                      ([1, 200, 7], [1, 1, 0])])
def test_nonspec_prefill_lengths(lens, his):
    # Prefill rows that end inside a 64-token segment, exactly on it and just
    # past it, with and without an initial state; decodes first.
    nd = sum(1 for l in lens if l == 1)
    T = sum(lens)
    case = helpers.small_case(seed=20, Hk=16, Hv=32, dk=128, dv=128, K=4, T=T,
                              num_slots=16)
    slots = list(range(3, 3 + len(lens)))
    tix = np.random.default_rng(1).permutation(T).astype(np.int32)
    ns = helpers.nonspec_meta(lens, slots, his=his, tix=tix, num_decodes=nd)
    case["nonspec"] = ns
    case["spec"] = None
    case["name"] = "nonspec"
    out_ref, conv_ref, ssm_ref, _ = helpers.run_nonspec(case)
    g = Gpu(case)
    say(f"non-spec rows {lens}")
    g.attention()
    assert_out_close(g.host_out(), out_ref)
    np.testing.assert_array_equal(g.host_conv(slots), conv_ref[slots])
    assert_states_close(g.host_ssm(slots), ssm_ref[slots])


def _prefill_case(seed, lens, his, dk=128, Hk=16, Hv=32, tweak=None):
    nd = sum(1 for l in lens if l == 1)
    T = sum(lens)
    case = helpers.small_case(seed=seed, Hk=Hk, Hv=Hv, dk=dk, dv=dk, K=4, T=T, num_slots=16)
    if tweak:
        tweak(case)
    slots = list(range(3, 3 + len(lens)))
    tix = np.random.default_rng(seed).permutation(T).astype(np.int32)
    case["nonspec"] = helpers.nonspec_meta(lens, slots, his=his, tix=tix, num_decodes=nd)
    case["spec"] = None
    case["name"] = "prefill"
    return case, slots


def _check_nonspec(case, slots):
    out_ref, conv_ref, ssm_ref, _ = helpers.run_nonspec(case)
    g = Gpu(case)
    say(f"prefill rows {case['nonspec']['query_start_loc'].tolist()} dk={case['dims']['dk']}")
    g.attention()
    assert_out_close(g.host_out(), out_ref)
    np.testing.assert_array_equal(g.host_conv(slots), conv_ref[slots])
    assert_states_close(g.host_ssm(slots), ssm_ref[slots])


def _rows_case(seed, lens, dk, Hk=2, Hv=4):
    """Prefill rows only (1-token rows included), slots 3.., random
    has_initial_state and a random token_indx."""
    rng = np.random.default_rng(seed)
    T = int(sum(lens))
    case = helpers.small_case(seed=seed, Hk=Hk, Hv=Hv, dk=dk, dv=dk, K=4, T=T,
                              num_slots=len(lens) + 4)
    slots = list(range(3, 3 + len(lens)))
    his = rng.integers(0, 2, len(lens)).tolist()
    tix = rng.permutation(T).astype(np.int32)
    case["nonspec"] = helpers.nonspec_meta(lens, slots, his=his, tix=tix, num_decodes=0)
    case["spec"] = None
    case["name"] = "prefill-rows"
    return case, [s for s, n in zip(slots, lens) if n > 0]


@pytest.mark.parametrize("dk", [32, 64])
def test_prefill_many_rows(dk):
    # 70 rows of 0..150 tokens (some empty, some of one token) around a
    # 700-token row: the 64-token unit map packs rows of every length, and
    # empty rows touch neither pool.
    rng = np.random.default_rng(50 + dk)
    lens = rng.integers(0, 151, 70)
    lens[rng.choice(70, 6, replace=False)] = 0
    lens[rng.choice(70, 4, replace=False)] = 1
    lens = lens.tolist()
    lens.insert(35, 700)
    case, touched = _rows_case(60 + dk, lens, dk)
    _check_nonspec(case, touched)


def test_prefill_rows_past_one_map_block():
    # 1100 rows of 0..3 tokens: the unit map is built 1024 rows at a time.
    rng = np.random.default_rng(7)
    lens = rng.integers(0, 4, 1100).tolist()
    case, touched = _rows_case(8, lens, 64, Hk=1, Hv=2)
    _check_nonspec(case, touched)


@pytest.mark.parametrize("dk", [64, 128])
def test_chunked_prefill_chunk_edges(dk):
    # Rows ending one short of, on, and one past a 64-token chunk, a short
    # row, and a 1024-token row; with and without an initial state.
    case, slots = _prefill_case(30 + dk, [63, 64, 65, 5, 1024], [1, 0, 1, 1, 0], dk=dk, Hk=4, Hv=8)
    _check_nonspec(case, slots)


def test_chunked_prefill_strong_decay():
    # log-decays down to about -16 per token (about -1000 per chunk): only
    # decay differences are exponentiated, so nothing overflows.
    def tweak(c):
        c["A_log"][:] = np.float32(np.log(16.0))
        c["a"][:] = synth.to_bf16(np.abs(synth.from_bf16(c["a"])) + 2.0)
    case, slots = _prefill_case(41, [200, 130], [1, 1], Hk=4, Hv=8, tweak=tweak)
    _check_nonspec(case, slots)


def test_chunked_prefill_no_decay_parallel_keys():
    # decay 1 and write strength near 1 with nearly parallel keys: the
    # (I + A)^-1 solve is at its least well conditioned.
    def tweak(c):
        c["A_log"][:] = -np.inf
        c["b"][:] = synth.to_bf16(np.full(c["b"].shape, 4.0, np.float32))
        Hk, dk = 4, 128
        x = synth.from_bf16(c["mixed_qkv"]).copy()
        base = x[0, Hk * dk:2 * Hk * dk].copy()
        x[:, Hk * dk:2 * Hk * dk] = base + 0.05 * x[:, Hk * dk:2 * Hk * dk]
        c["mixed_qkv"] = synth.to_bf16(x)
    case, slots = _prefill_case(42, [150], [1], Hk=4, Hv=8, tweak=tweak)
    _check_nonspec(case, slots)
