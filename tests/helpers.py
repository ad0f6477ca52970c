"""Shared helpers for the tests: running the oracle on copies of a case and
building small hand-made batches.  Pure host code, no GPU."""
from __future__ import annotations

import copy

import numpy as np

import oracle
import synth


def clone(case: dict) -> dict:
    c = dict(case)
    for k in ("conv_state", "ssm_state", "mixed_qkv", "a", "b", "conv_weight",
              "A_log", "dt_bias"):
        if c.get(k) is not None:
            c[k] = c[k].copy()
    c["spec"] = copy.deepcopy(case.get("spec"))
    c["nonspec"] = copy.deepcopy(case.get("nonspec"))
    c["dims"] = dict(case["dims"])
    return c


def out_shape(case):
    d = case["dims"]
    return (case["num_actual_tokens"], d["Hv"], d["dv"])


def run_spec(case, spec=None, with_conv=False, out=None):
    """Oracle spec call on a clone; returns (out, conv_state, ssm_state, y)."""
    c = clone(case)
    d = c["dims"]
    C = synth.conv_dim(d["Hk"], d["Hv"], d["dk"], d["dv"])
    o = np.zeros(out_shape(c), np.uint16) if out is None else out.copy()
    y = np.full((c["num_actual_tokens"], C), np.nan) if with_conv else None
    oracle.spec_step(d, c, spec if spec is not None else c["spec"], o, y)
    return o, c["conv_state"], c["ssm_state"], y


def run_nonspec(case, ns=None, with_conv=False, out=None):
    c = clone(case)
    d = c["dims"]
    C = synth.conv_dim(d["Hk"], d["Hv"], d["dk"], d["dv"])
    o = np.zeros(out_shape(c), np.uint16) if out is None else out.copy()
    y = np.full((c["num_actual_tokens"], C), np.nan) if with_conv else None
    oracle.nonspec_step(d, c, ns if ns is not None else c["nonspec"], o, y)
    return o, c["conv_state"], c["ssm_state"], y


def run_case(case, out=None):
    """Oracle on a clone of the whole batch: the non-spec rows, then the spec
    rows (rows of one call use disjoint slots, so the order does not matter).
    Either stream may be absent.  Returns (out, conv_state, ssm_state)."""
    c = clone(case)
    d = c["dims"]
    o = np.zeros(out_shape(c), np.uint16) if out is None else out.copy()
    if c.get("nonspec") is not None:
        oracle.nonspec_step(d, c, c["nonspec"], o)
    if c.get("spec") is not None:
        oracle.spec_step(d, c, c["spec"], o)
    return o, c["conv_state"], c["ssm_state"]


def spec_meta(sqsl, ssi, nacc, tix=None, cache=None):
    sqsl = np.asarray(sqsl, np.int32)
    ssi = np.asarray(ssi, np.int32)
    return dict(num_spec_decodes=len(sqsl) - 1, K=ssi.shape[1],
                num_spec_tokens=int(sqsl[-1]), spec_query_start_loc=sqsl,
                spec_cache_indices=None if cache is None else np.asarray(cache, np.int32),
                spec_state_indices=ssi, num_accepted_tokens=np.asarray(nacc, np.int32),
                spec_token_indx=None if tix is None else np.asarray(tix, np.int32))


def nonspec_meta(lens, slots, his=None, tix=None, num_decodes=None):
    lens = list(lens)
    qsl = np.zeros(len(lens) + 1, np.int32)
    qsl[1:] = np.cumsum(lens)
    nd = sum(1 for l in lens if l == 1) if num_decodes is None else num_decodes
    return dict(num_decodes=nd, num_prefills=len(lens) - nd,
                num_non_spec_tokens=int(qsl[-1]), query_start_loc=qsl,
                cache_indices=np.asarray(slots, np.int32),
                has_initial_state=None if his is None else np.asarray(his, np.uint8),
                token_indx=None if tix is None else np.asarray(tix, np.int32))


def small_case(seed=0, Hk=2, Hv=4, dk=16, dv=16, W=4, K=3, T=None, L=None,
               num_slots=16, activation=1, use_qk_l2norm=1, eps=1e-6,
               scale=None):
    """Random parameters, inputs and pools for hand-built metadata."""
    rng = np.random.default_rng(seed)
    L = W - 1 + K - 1 if L is None else L
    d = synth.dims_of(Hk, Hv, dk, dv, W, L, num_slots, activation,
                      use_qk_l2norm, eps, scale)
    T = K if T is None else T
    case = dict(dims=d)
    case.update(synth._params(rng, d, T))
    case.update(synth._pools(rng, d))
    return case
