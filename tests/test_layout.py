"""The two channel orders of mixed_qkv ("[GDN] Spec-decoding-aware attention
kernel", "Test Plan": the reorder_input equivalence test).

Grouped order: all q heads, all k heads, all v heads.  Per-k-head order (the
projections as produced): for each k-head i its q, its k, then the v of its
G = Hv/Hk v-heads.  Only the reads of mixed_qkv change; outputs, the conv
ring and the SSM pool must be the same bits either way."""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest

import synth
from tests.gpu_util import Gpu, gpu_available, say


def per_k_head(qkv, Hk, Hv, dk, dv):
    """Rows of a grouped mixed_qkv [T, C] repacked in per-k-head order."""
    T = qkv.shape[0]
    G = Hv // Hk
    q = qkv[:, :Hk * dk].reshape(T, Hk, dk)
    k = qkv[:, Hk * dk:2 * Hk * dk].reshape(T, Hk, dk)
    v = qkv[:, 2 * Hk * dk:].reshape(T, Hk, G * dv)
    return np.ascontiguousarray(np.concatenate([q, k, v], axis=2).reshape(T, -1))


def test_per_k_head_repack_labels():
    # Hk=2, G=2, dk=2, dv=1: grouped [q0 q0 q1 q1 | k0 k0 k1 k1 | v0 v1 v2 v3]
    grouped = np.array([["q0a", "q0b", "q1a", "q1b", "k0a", "k0b", "k1a", "k1b",
                         "v0", "v1", "v2", "v3"]])
    assert per_k_head(grouped, 2, 4, 2, 1).tolist() == [
        ["q0a", "q0b", "k0a", "k0b", "v0", "v1", "q1a", "q1b", "k1a", "k1b", "v2", "v3"]]


def _pair(case):
    d = case["dims"]
    grouped = Gpu(case)
    inter = dict(case)
    inter["mixed_qkv"] = per_k_head(case["mixed_qkv"], d["Hk"], d["Hv"], d["dk"], d["dv"])
    per = Gpu(inter)
    per.cfg = dataclasses.replace(per.cfg, reorder_input=False)
    return grouped, per


def _same(a, b):
    np.testing.assert_array_equal(a.host_out(), b.host_out())
    np.testing.assert_array_equal(a.host_conv(), b.host_conv())
    np.testing.assert_array_equal(a.host_ssm(), b.host_ssm())


@pytest.mark.parametrize("name", ["small", "qwen3next_k3_b64"])
@pytest.mark.gpu
@pytest.mark.skipif(not gpu_available(), reason="needs a GPU and libgdn.so")
def test_per_k_head_layout_spec(name):
    case = synth.make_case(name, seed=21, permute_tokens=True)
    a, b = _pair(case)
    say(f"layout equivalence, spec {name}")
    a.spec()
    b.spec()
    _same(a, b)


@pytest.mark.gpu
@pytest.mark.skipif(not gpu_available(), reason="needs a GPU and libgdn.so")
def test_per_k_head_layout_mixed_batch():
    # decodes, two 1024-token prefills (conv_prefill + chunked form) and spec rows
    case = synth.make_case("mixed", seed=22)
    a, b = _pair(case)
    say("layout equivalence, mixed batch")
    a.attention()
    b.attention()
    _same(a, b)


@pytest.mark.gpu
@pytest.mark.skipif(not gpu_available(), reason="needs a GPU and libgdn.so")
def test_per_k_head_layout_conv_stage():
    import torch
    import speculative_decoding_causal_amd as gdn
    from tests.gpu_util import dev, i32
    case = synth.make_case("small", seed=23, permute_tokens=True)
    sp = case["spec"]
    a, b = _pair(case)
    T = sp["num_spec_tokens"]
    outs = []
    for g in (a, b):
        y = torch.zeros(T, g.cfg.conv_dim, dtype=torch.float32, device=dev())
        gdn.gdn_conv_only(g.cfg, g.qkv, g.w, g.bias, g.conv, y, kind=gdn.GDN_ROWS_SPEC,
                          query_start_loc=i32(sp["spec_query_start_loc"]), num_tokens=T,
                          max_row_tokens=sp["spec_state_indices"].shape[1],
                          state_indices=i32(sp["spec_state_indices"]),
                          num_accepted_tokens=i32(sp["num_accepted_tokens"]),
                          cache_indices=i32(sp.get("spec_cache_indices")),
                          token_indx=i32(sp.get("spec_token_indx")))
        outs.append(y.cpu().numpy())
    np.testing.assert_array_equal(outs[0], outs[1])
    np.testing.assert_array_equal(a.host_conv(), b.host_conv())
