"""Capture and replay of GDN step calls.

"[GDN] Spec-decoding-aware attention kernel" ("Test Plan") regression-tests
the kernel on (metadata, inputs, outputs) tuples captured from live model
runs and replayed through the kernel.  This module gives the library that
format: one ``.npz`` file per call holding

* the call (``gdn_spec_attention`` or ``gdn_attention``), the layer shape
  and the scalar arguments (JSON);
* the inputs (mixed_qkv, a, b, conv weight and bias, A_log, dt_bias) and
  every metadata array, as given;
* the pool slots the metadata names (0 < slot < num_slots), with their conv
  and SSM bytes before and after the call;
* core_attn_out before and after the call (rows the call does not name keep
  their bytes).

Replay rebuilds compact pools holding only those slots (slot ids remapped,
NULL stays NULL), reruns the call on the GPU and compares: bit equality,
and the tolerances of the equivalence tests (outputs |x-y| <= 2e-2 +
2e-2|y|, SSM tiles max|dS| <= 1e-3 max|S|, conv bytes equal) for captures
taken from another implementation.  Files are read with
``numpy.load(allow_pickle=False)``; nothing in them is executed.

Command line::

    python -m speculative_decoding_causal_amd.capture replay FILE...
"""
from __future__ import annotations

import json
import sys

import numpy as np
import torch

FORMAT = "gdn-step-capture/1"

_INPUTS = ("mixed_qkv", "a", "b", "conv_weight", "conv_bias", "A_log", "dt_bias")
_META = ("spec_query_start_loc", "spec_state_indices", "num_accepted_tokens",
         "spec_cache_indices", "spec_token_indx", "query_start_loc",
         "non_spec_state_indices", "has_initial_state", "non_spec_token_indx")
_SLOT_ARRAYS = ("spec_state_indices", "spec_cache_indices", "non_spec_state_indices")
_SCALARS = ("num_spec_tokens", "num_decodes", "num_prefills", "num_non_spec_tokens",
            "num_actual_tokens")
_CFG = ("num_k_heads", "num_v_heads", "head_k_dim", "head_v_dim", "conv_width",
        "activation", "use_qk_l2norm", "l2norm_eps", "scale", "reorder_input", "conv_layout")

OUT_ATOL = OUT_RTOL = 2e-2
STATE_RTOL = 1e-3


def _host(t):
    if t is None:
        return None
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return t.detach().cpu().numpy()


def referenced_slots(meta: dict, num_slots: int) -> np.ndarray:
    """Sorted valid slot ids (0 < s < num_slots) named by the metadata."""
    vals = [np.asarray(meta[k]).ravel() for k in _SLOT_ARRAYS if meta.get(k) is not None]
    if not vals:
        return np.zeros(0, np.int32)
    v = np.concatenate(vals)
    return np.unique(v[(v > 0) & (v < num_slots)]).astype(np.int32)


def remap_slots(x, slots: np.ndarray) -> np.ndarray:
    """Slot ids -> compact ids: the i-th referenced slot becomes i+1, every
    other value (NULL, pad or out of range) becomes 0."""
    x = np.asarray(x, np.int32)
    idx = np.searchsorted(slots, x)
    hit = (idx < len(slots)) & (slots[np.minimum(idx, max(len(slots) - 1, 0))] == x) \
        if len(slots) else np.zeros(x.shape, bool)
    return np.where(hit, idx + 1, 0).astype(np.int32)


def save(path: str, record: dict) -> None:
    """Write a capture record (see ``record_call``) as an uncompressed npz."""
    arrays = {k: v for k, v in record["arrays"].items() if v is not None}
    header = {k: record[k] for k in ("format", "call", "cfg", "state_len", "num_slots",
                                     "scalars")}
    np.savez(path, header=np.frombuffer(json.dumps(header).encode(), np.uint8), **arrays)


def load(path: str) -> dict:
    with np.load(path, allow_pickle=False) as z:
        header = json.loads(bytes(z["header"]).decode())
        if header.get("format") != FORMAT:
            raise ValueError(f"{path}: not a {FORMAT} file")
        arrays = {k: z[k] for k in z.files if k != "header"}
    header["arrays"] = arrays
    return header


def record_call(path: str, call: str, cfg, conv_state, ssm_state, core_attn_out,
                **kwargs) -> dict:
    """Run ``call`` ("gdn_spec_attention" or "gdn_attention") with the given
    tensors and keyword arguments, and write the capture to ``path``.  The
    pools and core_attn_out are updated in place, as by the call itself.
    Host copies are taken before and after, so this is for test captures,
    not for the serving path."""
    import speculative_decoding_causal_amd as gdn
    if call not in ("gdn_spec_attention", "gdn_attention"):
        raise ValueError(f"unknown call {call!r}")
    meta = {k: _host(kwargs.get(k)) for k in _META}
    num_slots = int(conv_state.shape[0])
    slots = referenced_slots(meta, num_slots)
    sl = torch.as_tensor(slots, dtype=torch.long, device=conv_state.device)
    conv_pre, ssm_pre = _host(conv_state[sl]), _host(ssm_state[sl])
    out_pre = _host(core_attn_out)
    args = dict(kwargs)
    inputs = {k: args.pop(k) for k in _INPUTS}
    for k in _META:
        args.pop(k, None)
    scalars = {k: args.pop(k) for k in _SCALARS if k in args}
    fn = getattr(gdn, call)
    if call == "gdn_spec_attention":
        fn(cfg, inputs["mixed_qkv"], inputs["a"], inputs["b"], inputs["conv_weight"],
           inputs["conv_bias"], inputs["A_log"], inputs["dt_bias"], conv_state, ssm_state,
           kwargs["spec_query_start_loc"], kwargs["spec_state_indices"],
           kwargs["num_accepted_tokens"], core_attn_out,
           spec_cache_indices=kwargs.get("spec_cache_indices"),
           spec_token_indx=kwargs.get("spec_token_indx"), **scalars, **args)
    else:
        fn(cfg, inputs["mixed_qkv"], inputs["a"], inputs["b"], inputs["conv_weight"],
           inputs["conv_bias"], inputs["A_log"], inputs["dt_bias"], conv_state, ssm_state,
           core_attn_out, **{k: kwargs.get(k) for k in _META}, **scalars, **args)
    torch.cuda.current_stream().synchronize()
    rec = dict(format=FORMAT, call=call,
               cfg={k: getattr(cfg, k) for k in _CFG},
               state_len=int(conv_state.shape[1]), num_slots=num_slots,
               scalars={k: (None if v is None else int(v)) for k, v in scalars.items()})
    arrays = {k: _host(v) for k, v in inputs.items()}
    arrays.update({k: v for k, v in meta.items()})
    arrays.update(slots=slots, conv_pre=conv_pre, ssm_pre=ssm_pre,
                  conv_post=_host(conv_state[sl]), ssm_post=_host(ssm_state[sl]),
                  core_attn_out_pre=out_pre, core_attn_out=_host(core_attn_out))
    rec["arrays"] = arrays
    save(path, rec)
    return rec


def _dev(x, device, bf16=False):
    if x is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(x)).to(device)
    return t.view(torch.bfloat16) if bf16 else t


def replay(path: str, device: str = "cuda:0") -> dict:
    """Rerun a captured call on compact pools and compare with the capture."""
    rec, out, conv, ssm = rerun(path, device)
    return compare(rec["arrays"], out, conv, ssm)


def compact_metadata(rec: dict) -> dict:
    """The capture's metadata arrays with slot ids remapped to the compact
    pools (slot ``slots[i]`` becomes i+1; NULL, pad and out-of-range ids
    become 0)."""
    A = rec["arrays"]
    return {k: (remap_slots(A[k], A["slots"]) if k in _SLOT_ARRAYS else A[k])
            for k in _META if k in A}


def rerun(path: str, device: str = "cuda:0"):
    """Rerun a captured call on compact pools (slot 0 is NULL, slot i+1 holds
    the capture's i-th slot).  Returns (record, core_attn_out, conv slots,
    SSM slots) as host arrays, the pools without their NULL slot."""
    import speculative_decoding_causal_amd as gdn
    rec = load(path)
    A = rec["arrays"]
    slots = A["slots"]
    n = len(slots) + 1
    cfg = gdn.GdnConfig(**rec["cfg"])
    conv = torch.zeros((n,) + A["conv_pre"].shape[1:], dtype=torch.int16, device=device)
    ssm = torch.zeros((n,) + A["ssm_pre"].shape[1:], dtype=torch.float32, device=device)
    if len(slots):
        conv[1:] = _dev(A["conv_pre"], device)
        ssm[1:] = _dev(A["ssm_pre"], device)
    conv = conv.view(torch.bfloat16)
    out = _dev(A["core_attn_out_pre"], device, bf16=True)
    kw = {k: _dev(v, device) for k, v in compact_metadata(rec).items()}
    inputs = {k: _dev(A.get(k), device, bf16=A.get(k) is not None and A[k].dtype == np.int16)
              for k in _INPUTS}
    sc = {k: v for k, v in rec["scalars"].items() if v is not None}
    # fresh turn counters for the compact pools (the results are the same
    # bits with or without them)
    turns = gdn.conv_turns(cfg, n, device)
    if rec["call"] == "gdn_spec_attention":
        gdn.gdn_spec_attention(cfg, inputs["mixed_qkv"], inputs["a"], inputs["b"],
                               inputs["conv_weight"], inputs["conv_bias"], inputs["A_log"],
                               inputs["dt_bias"], conv, ssm, kw["spec_query_start_loc"],
                               kw["spec_state_indices"], kw["num_accepted_tokens"], out,
                               spec_cache_indices=kw.get("spec_cache_indices"),
                               spec_token_indx=kw.get("spec_token_indx"), conv_turns=turns,
                               **sc)
    else:
        ws = None
        if sc.get("num_prefills", 0) > 0:
            nbytes = gdn.gdn_workspace_bytes(cfg, rec["state_len"], n,
                                             sc["num_non_spec_tokens"], sc["num_prefills"])
            ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        gdn.gdn_attention(cfg, inputs["mixed_qkv"], inputs["a"], inputs["b"],
                          inputs["conv_weight"], inputs["conv_bias"], inputs["A_log"],
                          inputs["dt_bias"], conv, ssm, out, workspace=ws, conv_turns=turns,
                          **kw, **sc)
    torch.cuda.synchronize()
    got_out = out.view(torch.int16).cpu().numpy()
    got_conv = conv.view(torch.int16)[1:].cpu().numpy()
    got_ssm = ssm[1:].cpu().numpy()
    return rec, got_out, got_conv, got_ssm


def _bf16_to_f64(x):
    return (np.asarray(x).astype(np.uint16).astype(np.uint32) << 16).view(np.float32) \
        .astype(np.float64)


def compare(A: dict, out, conv, ssm) -> dict:
    """Bit equality and tolerance checks of a replay against its capture."""
    ref_out, ref_conv, ref_ssm = A["core_attn_out"], A["conv_post"], A["ssm_post"]
    g, r = _bf16_to_f64(out), _bf16_to_f64(ref_out)
    err = np.abs(g - r)
    out_ok = bool(np.all(err <= OUT_ATOL + OUT_RTOL * np.abs(r)))
    if len(ref_ssm):
        d = np.abs(ssm.astype(np.float64) - ref_ssm).reshape(len(ref_ssm), -1,
                                                             *ref_ssm.shape[-2:])
        scale = np.abs(ref_ssm.astype(np.float64)).reshape(d.shape).max(axis=(-2, -1))
        rel = d.max(axis=(-2, -1)) / np.maximum(scale, 1e-30)
        ssm_rel = float(rel.max())
    else:
        ssm_rel = 0.0
    res = dict(out_bit_equal=bool(np.array_equal(out, ref_out)),
               out_max_abs=float(err.max()) if err.size else 0.0,
               conv_bit_equal=bool(np.array_equal(conv, ref_conv)),
               ssm_bit_equal=bool(np.array_equal(ssm, ref_ssm)),
               ssm_max_rel=ssm_rel)
    res["within_tolerance"] = out_ok and res["conv_bit_equal"] and ssm_rel <= STATE_RTOL
    return res


def main(argv=None) -> int:
    argv = sys.argv[1:] if argv is None else argv
    if len(argv) < 2 or argv[0] != "replay":
        print("usage: python -m speculative_decoding_causal_amd.capture replay FILE...",
              file=sys.stderr)
        return 2
    bad = 0
    for path in argv[1:]:
        res = replay(path)
        bad += not res["within_tolerance"]
        print(json.dumps(dict(file=path, **res)), flush=True)
    return 1 if bad else 0


if __name__ == "__main__":
    sys.exit(main())
