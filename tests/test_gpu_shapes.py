"""HIP path against the oracle on the shapes and layer options the other
parity tests leave out: spec rows of more than 4 tokens (up to 14, the most
a 16-column ring holds with width 4), rings longer than the rows need, a
conv bias, the identity activation and unnormalised q/k.

Each shape picks a different specialisation of the row kernel (register
gathers sized for rings of at most 6 or 8 columns and rows of at most 4
tokens, or the general one), so every one of them runs here."""
from __future__ import annotations

import numpy as np
import pytest

import synth
from tests import helpers
from tests.gpu_util import (Gpu, assert_out_close, assert_states_close, gpu_available, say)
from tests.test_gpu_parity import check_spec_case

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU and libgdn.so")]


@pytest.mark.parametrize("K", [6, 8, 14])
def test_spec_long_rows(K):
    # ring of W-1+K-1 columns (16 for K = 14), NULL slots, permuted tokens
    case = synth.make_case("small", seed=20 + K, K=K, Ns=6, Hv=32, num_slots=128, null_p=0.1,
                           permute_tokens=True)
    check_spec_case(case)


@pytest.mark.parametrize("K,L", [(4, 7), (4, 8), (3, 12)])
def test_spec_ring_longer_than_needed(K, L):
    # n_acc may then reach past K - 1 columns of history; the window offset
    # and the roll still follow n_acc
    case = synth.make_case("small", seed=30 + L, K=K, L=L, Ns=10, Hv=32, num_slots=128,
                           null_p=0.0, permute_tokens=True)
    check_spec_case(case)


def _options(case, bias, activation, l2norm, seed):
    rng = np.random.default_rng(seed)
    d = case["dims"]
    d["activation"] = activation
    d["use_qk_l2norm"] = l2norm
    C = synth.conv_dim(d["Hk"], d["Hv"], d["dk"], d["dv"])
    if bias:
        case["conv_bias"] = synth.to_bf16(0.5 * rng.standard_normal(C).astype(np.float32))
    if not l2norm:
        # unnormalised keys: keep |k|^2 below 1 so the recurrence stays stable
        w = synth.from_bf16(case["conv_weight"]) / 16.0
        case["conv_weight"] = synth.to_bf16(w)
        if bias:
            case["conv_bias"] = synth.to_bf16(synth.from_bf16(case["conv_bias"]) / 16.0)
    return case


OPTIONS = [(True, 1, 1), (False, 0, 1), (True, 0, 1), (True, 1, 0), (False, 0, 0)]


@pytest.mark.parametrize("bias,activation,l2norm", OPTIONS)
def test_spec_layer_options(bias, activation, l2norm):
    case = synth.make_case("small", seed=40, K=3, Ns=8, Hv=32, num_slots=64, null_p=0.2,
                           permute_tokens=True)
    check_spec_case(_options(case, bias, activation, l2norm, 41))


@pytest.mark.parametrize("bias,activation,l2norm", OPTIONS)
@pytest.mark.parametrize("dk", [16, 32, 64, 128])
def test_mixed_layer_options(bias, activation, l2norm, dk):
    # decodes, prefill rows (the token recurrence below dk = 64, the chunked
    # form from 64) and spec rows in one call, at every head size the row
    # kernel is built for
    case = synth.make_case("mixed", seed=50, Ns=6, K=3, Nd=5, prefill_lens=(70, 130),
                           Hk=4, Hv=8, dk=dk, dv=dk, num_slots=64)
    case = _options(case, bias, activation, l2norm, 51)
    o1, r1, s1, _ = helpers.run_nonspec(case)
    c = helpers.clone(case)
    c["conv_state"], c["ssm_state"] = r1, s1
    out_ref, conv_ref, ssm_ref, _ = helpers.run_spec(c, out=o1)
    g = Gpu(case)
    say(f"mixed dk={dk} bias={bias} act={activation} l2norm={l2norm}")
    g.attention()
    assert_out_close(g.host_out(), out_ref)
    slots = synth.referenced_slots(case)
    np.testing.assert_array_equal(g.host_conv(slots), conv_ref[slots])
    assert_states_close(g.host_ssm(slots), ssm_ref[slots])


@pytest.mark.parametrize("Hk,Hv", [(2, 8), (1, 8), (4, 4)])
def test_spec_head_groups(Hk, Hv):
    # 4 and 8 v-heads per k-head (the row kernel then takes its 512 or 1024
    # state rows in several passes) and one
    case = synth.make_case("small", seed=60 + Hv // Hk, K=3, Ns=6, Hk=Hk, Hv=Hv, num_slots=64,
                           null_p=0.15, permute_tokens=True)
    check_spec_case(case)


def test_mixed_four_v_heads_per_k_head():
    case = synth.make_case("mixed", seed=70, Ns=5, K=4, Nd=4, prefill_lens=(65, 140),
                           Hk=2, Hv=8, num_slots=64)
    o1, r1, s1, _ = helpers.run_nonspec(case)
    c = helpers.clone(case)
    c["conv_state"], c["ssm_state"] = r1, s1
    out_ref, conv_ref, ssm_ref, _ = helpers.run_spec(c, out=o1)
    g = Gpu(case)
    say("mixed, 4 v-heads per k-head")
    g.attention()
    assert_out_close(g.host_out(), out_ref)
    slots = synth.referenced_slots(case)
    np.testing.assert_array_equal(g.host_conv(slots), conv_ref[slots])
    assert_states_close(g.host_ssm(slots), ssm_ref[slots])


# (dk, Hk, Hv) whose conv channels end part-way into a wave: C/4 = 16, 96,
# 96 and 24 threads, so the last wave has 16, 32, 32 and 24 live lanes,
# fewer than the 35 lanes conv_prefill reads token rows from
@pytest.mark.parametrize("dk,Hk,Hv", [(16, 1, 2), (64, 2, 2), (128, 1, 1), (32, 1, 1)])
def test_mixed_partial_channel_wave(dk, Hk, Hv):
    case = synth.make_case("mixed", seed=80 + dk, Ns=4, K=3, Nd=3, prefill_lens=(64, 17),
                           Hk=Hk, Hv=Hv, dk=dk, dv=dk, num_slots=64)
    o1, r1, s1, _ = helpers.run_nonspec(case)
    c = helpers.clone(case)
    c["conv_state"], c["ssm_state"] = r1, s1
    out_ref, conv_ref, ssm_ref, _ = helpers.run_spec(c, out=o1)
    g = Gpu(case)
    say(f"mixed, partial channel wave dk={dk} Hk={Hk} Hv={Hv}")
    g.attention()
    assert_out_close(g.host_out(), out_ref)
    slots = synth.referenced_slots(case)
    np.testing.assert_array_equal(g.host_conv(slots), conv_ref[slots])
    assert_states_close(g.host_ssm(slots), ssm_ref[slots])


@pytest.mark.parametrize("shape", ["K16_ring16", "K16_per_token", "G8_dv1024"])
def test_spec_maximum_sizes(shape):
    # The largest shapes the header allows: 16 tokens per row (a width-2 conv
    # whose 16-column ring keeps the window at n_acc - 1 in range for every
    # n_acc), 16 tokens per row under the per-token conv contract, and eight
    # v-heads per k-head at dk = 128 ((Hv/Hk) * dv = 1024 state rows).
    if shape == "K16_ring16":
        case = synth.make_case("small", seed=90, K=16, W=2, Ns=5, Hk=2, Hv=4, num_slots=96,
                               null_p=0.1, permute_tokens=True)
        assert case["dims"]["L"] == 16
    elif shape == "K16_per_token":
        from tests.test_gpu_per_token import per_token_case
        case = per_token_case(91, Ns=6, K=16, Hk=2, Hv=4)
    else:
        case = synth.make_case("small", seed=92, K=4, Ns=6, Hk=1, Hv=8, num_slots=64,
                               null_p=0.1, permute_tokens=True)
    say(f"maximum size {shape}")
    check_spec_case(case)
