"""Capture/replay format ("[GDN] Spec-decoding-aware attention kernel", "Test
Plan": regression on captured (metadata, inputs, outputs) tuples)."""
from __future__ import annotations

import numpy as np
import pytest

from speculative_decoding_causal_amd import capture
from tests.gpu_util import Gpu, gpu_available, i32, say, u8


def test_slot_remap():
    slots = np.array([3, 7, 9], np.int32)
    x = np.array([[7, 0, -1], [3, 9, 11]], np.int32)
    assert capture.remap_slots(x, slots).tolist() == [[2, 0, 0], [1, 3, 0]]
    assert capture.remap_slots(x, np.zeros(0, np.int32)).tolist() == [[0, 0, 0], [0, 0, 0]]
    meta = dict(spec_state_indices=np.array([[3, 0], [7, 12]]),
                non_spec_state_indices=np.array([9, -1]))
    assert capture.referenced_slots(meta, num_slots=10).tolist() == [3, 7, 9]


def test_file_round_trip(tmp_path):
    rec = dict(format=capture.FORMAT, call="gdn_spec_attention",
               cfg=dict(num_k_heads=1), state_len=3, num_slots=8,
               scalars=dict(num_spec_tokens=4),
               arrays=dict(slots=np.array([1, 2], np.int32),
                           mixed_qkv=np.arange(12, dtype=np.int16).reshape(3, 4),
                           conv_bias=None))
    p = str(tmp_path / "c.npz")
    capture.save(p, rec)
    back = capture.load(p)
    assert back["call"] == "gdn_spec_attention" and back["scalars"] == {"num_spec_tokens": 4}
    assert "conv_bias" not in back["arrays"]
    np.testing.assert_array_equal(back["arrays"]["mixed_qkv"], rec["arrays"]["mixed_qkv"])


def _record(g, tmp_path, name):
    import synth  # noqa: F401
    sp, ns = g.case.get("spec"), g.case.get("nonspec")
    kw = dict(mixed_qkv=g.qkv, a=g.a, b=g.b, conv_weight=g.w, conv_bias=g.bias, A_log=g.A_log,
              dt_bias=g.dt_bias)
    if sp is not None:
        kw.update(spec_query_start_loc=i32(sp["spec_query_start_loc"]),
                  spec_state_indices=i32(sp["spec_state_indices"]),
                  num_accepted_tokens=i32(sp["num_accepted_tokens"]),
                  spec_cache_indices=i32(sp.get("spec_cache_indices")),
                  spec_token_indx=i32(sp.get("spec_token_indx")),
                  num_spec_tokens=int(sp["num_spec_tokens"]))
    path = str(tmp_path / f"{name}.npz")
    if ns is None:
        capture.record_call(path, "gdn_spec_attention", g.cfg, g.conv, g.ssm, g.out, **kw)
        return path
    import speculative_decoding_causal_amd as gdn
    import torch
    d = g.case["dims"]
    ws = None
    if ns["num_prefills"] > 0:
        n = gdn.gdn_workspace_bytes(g.cfg, d["L"], d["num_slots"], ns["num_non_spec_tokens"],
                                    ns["num_prefills"])
        ws = torch.empty(n, dtype=torch.uint8, device=g.qkv.device)
    kw.update(num_decodes=ns["num_decodes"], num_prefills=ns["num_prefills"],
              num_non_spec_tokens=ns["num_non_spec_tokens"],
              query_start_loc=i32(ns["query_start_loc"]),
              non_spec_state_indices=i32(ns["cache_indices"]),
              has_initial_state=u8(ns.get("has_initial_state")),
              non_spec_token_indx=i32(ns.get("token_indx")), workspace=ws)
    capture.record_call(path, "gdn_attention", g.cfg, g.conv, g.ssm, g.out, **kw)
    return path


@pytest.mark.gpu
@pytest.mark.skipif(not gpu_available(), reason="needs a GPU and libgdn.so")
@pytest.mark.parametrize("name", ["small", "mixed"])
def test_record_then_replay_is_bit_exact(name, tmp_path):
    import synth
    g = Gpu(synth.make_case(name, seed=31, permute_tokens=(name == "small")))
    say(f"capture + replay {name}")
    path = _record(g, tmp_path, name)
    res = capture.replay(path)
    assert res["out_bit_equal"] and res["conv_bit_equal"] and res["ssm_bit_equal"], res
    assert res["within_tolerance"]


@pytest.mark.gpu
@pytest.mark.skipif(not gpu_available(), reason="needs a GPU and libgdn.so")
def test_replay_reports_a_wrong_capture(tmp_path):
    import synth
    g = Gpu(synth.make_case("small", seed=32))
    path = _record(g, tmp_path, "small")
    rec = capture.load(path)
    A = rec["arrays"]
    row = int(A["spec_token_indx"][0]) if "spec_token_indx" in A else 0
    A["core_attn_out"][row, 0, :4] ^= np.int16(0x4000)     # flip an exponent bit
    A["ssm_post"][0, 0, 0, 0] += 1.0
    capture.save(path, rec)
    res = capture.replay(path)
    assert not res["out_bit_equal"] and not res["ssm_bit_equal"]
    assert not res["within_tolerance"]
