"""Capture/replay format ("[GDN] Spec-decoding-aware attention kernel", "Test
Plan": regression on captured (metadata, inputs, outputs) tuples, each replay
diffed against an oracle at atol = rtol = 2e-2).  A replay is compared with
the bytes it recorded and, independently, with the CPU oracle run on the
capture's own inputs and compact pools."""
from __future__ import annotations

import numpy as np
import pytest

from speculative_decoding_causal_amd import capture
import synth
from tests import helpers
from tests.gpu_util import (Gpu, assert_out_close, assert_states_close, gpu_available, i32,
                            say, u8)


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


def oracle_of_capture(rec):
    """The oracle on a capture's inputs and compact pools (slot i+1 holds the
    capture's i-th slot, slot 0 is NULL): returns (out, conv, ssm), the pools
    without their NULL slot.  Only grouped mixed_qkv captures."""
    A, cfg, sc = rec["arrays"], rec["cfg"], rec["scalars"]
    assert cfg["reorder_input"], "the oracle reads the grouped channel order"
    n = len(A["slots"]) + 1
    d = synth.dims_of(cfg["num_k_heads"], cfg["num_v_heads"], cfg["head_k_dim"],
                      cfg["head_v_dim"], cfg["conv_width"], rec["state_len"], n,
                      cfg["activation"], cfg["use_qk_l2norm"], cfg["l2norm_eps"],
                      cfg["scale"] if cfg["scale"] is not None else cfg["head_k_dim"] ** -0.5)
    d["conv_layout"] = cfg["conv_layout"]
    u16 = lambda x: None if x is None else np.ascontiguousarray(x).view(np.uint16)
    conv = np.zeros((n,) + A["conv_pre"].shape[1:], np.uint16)
    ssm = np.zeros((n,) + A["ssm_pre"].shape[1:], np.float32)
    conv[1:], ssm[1:] = u16(A["conv_pre"]), A["ssm_pre"]
    case = dict(dims=d, mixed_qkv=u16(A["mixed_qkv"]), a=u16(A["a"]), b=u16(A["b"]),
                conv_weight=u16(A["conv_weight"]), conv_bias=u16(A.get("conv_bias")),
                A_log=A["A_log"], dt_bias=A["dt_bias"], conv_state=conv, ssm_state=ssm,
                num_actual_tokens=int(A["mixed_qkv"].shape[0]), spec=None, nonspec=None)
    m = capture.compact_metadata(rec)
    if "spec_state_indices" in m:
        case["spec"] = helpers.spec_meta(m["spec_query_start_loc"], m["spec_state_indices"],
                                         m["num_accepted_tokens"], m.get("spec_token_indx"),
                                         m.get("spec_cache_indices"))
    if "non_spec_state_indices" in m:
        case["nonspec"] = dict(num_decodes=sc["num_decodes"], num_prefills=sc["num_prefills"],
                               num_non_spec_tokens=sc["num_non_spec_tokens"],
                               query_start_loc=m["query_start_loc"],
                               cache_indices=m["non_spec_state_indices"],
                               has_initial_state=m.get("has_initial_state"),
                               token_indx=m.get("non_spec_token_indx"))
    out, conv, ssm = helpers.run_case(case, out=u16(A["core_attn_out_pre"]))
    return out, conv[1:], ssm[1:]


def _record(g, tmp_path, name):
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
    rec, out, conv, ssm = capture.rerun(path)
    res = capture.compare(rec["arrays"], out, conv, ssm)
    assert res["out_bit_equal"] and res["conv_bit_equal"] and res["ssm_bit_equal"], res
    assert res["within_tolerance"]
    # the replay against the oracle on the capture's own inputs and pools
    ref_out, ref_conv, ref_ssm = oracle_of_capture(rec)
    assert_out_close(out.view(np.uint16), ref_out)
    np.testing.assert_array_equal(conv.view(np.uint16), ref_conv)
    assert_states_close(ssm, ref_ssm)
    assert capture.replay(path)["within_tolerance"]


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


@pytest.mark.parametrize("name", ["small", "mixed"])
def test_compact_pools_keep_the_oracle_result(name):
    # A capture record built on the host (as record_call lays it out) from a
    # batch and its oracle result: rerunning the oracle on the compact pools
    # and remapped metadata gives the same outputs and the same bytes for the
    # named slots.  Checks the slot remap that replays rely on, no GPU.
    case = synth.make_case(name, seed=33, permute_tokens=(name == "small"))
    if name == "mixed":   # keep the prefill rows short: host-side oracle time
        case = synth.make_case(name, seed=33, prefill_lens=(70, 5))
    out0 = np.full(helpers.out_shape(case), 0x5A5A, np.uint16)
    out1, conv1, ssm1 = helpers.run_case(case, out=out0)
    sp, ns = case["spec"], case["nonspec"]
    meta = dict(spec_query_start_loc=sp["spec_query_start_loc"],
                spec_state_indices=sp["spec_state_indices"],
                num_accepted_tokens=sp["num_accepted_tokens"],
                spec_token_indx=sp["spec_token_indx"])
    scalars = dict(num_spec_tokens=sp["num_spec_tokens"])
    if ns is not None:
        meta.update(query_start_loc=ns["query_start_loc"],
                    non_spec_state_indices=ns["cache_indices"],
                    has_initial_state=ns["has_initial_state"],
                    non_spec_token_indx=ns["token_indx"])
        scalars.update(num_decodes=ns["num_decodes"], num_prefills=ns["num_prefills"],
                       num_non_spec_tokens=ns["num_non_spec_tokens"])
    meta = {k: v for k, v in meta.items() if v is not None}
    d = case["dims"]
    slots = capture.referenced_slots(meta, d["num_slots"])
    i16 = lambda x: np.ascontiguousarray(x).view(np.int16)
    arrays = dict(mixed_qkv=i16(case["mixed_qkv"]), a=i16(case["a"]), b=i16(case["b"]),
                  conv_weight=i16(case["conv_weight"]), A_log=case["A_log"],
                  dt_bias=case["dt_bias"], slots=slots,
                  conv_pre=i16(case["conv_state"][slots]), ssm_pre=case["ssm_state"][slots],
                  core_attn_out_pre=i16(out0), **meta)
    cfg = dict(num_k_heads=d["Hk"], num_v_heads=d["Hv"], head_k_dim=d["dk"],
               head_v_dim=d["dv"], conv_width=d["W"], activation=d["activation"],
               use_qk_l2norm=d["use_qk_l2norm"], l2norm_eps=d["eps"], scale=d["scale"],
               reorder_input=True, conv_layout=0)
    rec = dict(format=capture.FORMAT, call="gdn_attention", cfg=cfg, state_len=d["L"],
               num_slots=d["num_slots"], scalars=scalars, arrays=arrays)
    out, conv, ssm = oracle_of_capture(rec)
    np.testing.assert_array_equal(out, out1)
    np.testing.assert_array_equal(conv, conv1[slots])
    np.testing.assert_array_equal(ssm, ssm1[slots])
