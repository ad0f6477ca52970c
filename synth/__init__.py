"""Seeded synthetic inputs for the GDN spec-verify step.

This module only draws random inputs and builds batch metadata; it holds none
of the step's arithmetic, so both the oracle (``oracle/``) and the HIP path
(``speculative_decoding_causal_amd``) can be fed from it.

Shapes and value distributions (one record per workload):

=========  ===================================================================
``tiny``   2 spec rows, K=2, 2 k-heads / 4 v-heads, dk=dv=16, W=4, C=128, L=4,
           8 slots
``small``  8 spec rows, K=3, 16/16 heads, dk=dv=128, C=6144, L=5, 64 slots,
           each state index NULL (0) with p=0.25, at least one NULL load and
           one NULL store
``qwen3next_k3_b64``  64 spec rows, K=3, 16 k-heads / 32 v-heads, dk=dv=128,
           C=8192, L=5, 512 slots, 192 distinct slots from [1, 512)
``qwen3next_k3_b64_tp2``  the same batch on one GPU's share of a two-way
           head split: 8 k-heads / 16 v-heads, C=4096
``deep_k4_b256``  256 spec rows, K=4, same heads, L=6, 2048 slots, at least
           one row with n_acc=1
``mixed``  32 spec rows (K=4) + 32 one-token decodes + 2 prefills of 1024
           tokens, rows shuffled (each row's tokens contiguous, at least one
           non-spec row ahead of a spec row), spec slots in [1, 513),
           non-spec slots in [513, 1024), L=6
=========  ===================================================================

Common to all: mixed_qkv, a, b ~ N(0, 1) rounded to bf16; conv weight
~ N(0, 0.5) bf16; no conv bias; A_log ~ U(ln 1, ln 16) and dt_bias ~ N(0, 0.1)
in fp32; SSM pool ~ N(0, 0.1) fp32 and conv pool ~ N(0, 1) bf16 on the
slots the batch references (other slots hold the constant 0.5, a canary that
must survive the step); SiLU; q/k
L2-normalised with eps 1e-6; scale = dk^-1/2; n_acc ~ U{1..K}.  L is the
smallest ring that keeps the window n_acc-1 in range: W-1 + K-1.  Slot 0 is
always the NULL block.  Random numbers come from numpy's PCG64 seeded per
workload.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["CONFIGS", "make_case", "to_bf16", "from_bf16", "dims_of",
           "conv_dim", "compose_rows"]


def to_bf16(x) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def from_bf16(h) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


def conv_dim(Hk, Hv, dk, dv) -> int:
    return 2 * Hk * dk + Hv * dv


def dims_of(Hk, Hv, dk, dv, W, L, num_slots, activation=1, use_qk_l2norm=1,
            eps=1e-6, scale=None) -> dict:
    return dict(Hk=Hk, Hv=Hv, dk=dk, dv=dv, W=W, L=L, num_slots=num_slots,
                activation=activation, use_qk_l2norm=use_qk_l2norm, eps=eps,
                scale=(dk ** -0.5) if scale is None else scale)


CONFIGS = {
    "tiny": dict(kind="spec", Ns=2, K=2, Hk=2, Hv=4, dk=16, dv=16, W=4,
                 num_slots=8, null_p=0.0),
    "small": dict(kind="spec", Ns=8, K=3, Hk=16, Hv=16, dk=128, dv=128, W=4,
                  num_slots=64, null_p=0.25),
    "qwen3next_k3_b64": dict(kind="spec", Ns=64, K=3, Hk=16, Hv=32, dk=128,
                             dv=128, W=4, num_slots=512, null_p=0.0),
    "qwen3next_k3_b64_tp2": dict(kind="spec", Ns=64, K=3, Hk=8, Hv=16, dk=128,
                                 dv=128, W=4, num_slots=512, null_p=0.0),
    "deep_k4_b256": dict(kind="spec", Ns=256, K=4, Hk=16, Hv=32, dk=128,
                         dv=128, W=4, num_slots=2048, null_p=0.0,
                         force_nacc1=True),
    "mixed": dict(kind="mixed", Ns=32, K=4, Nd=32, prefill_lens=(1024, 1024),
                  Hk=16, Hv=32, dk=128, dv=128, W=4, num_slots=1024),
}


def _params(rng, d, T):
    C = conv_dim(d["Hk"], d["Hv"], d["dk"], d["dv"])
    Hv, W = d["Hv"], d["W"]
    return dict(
        mixed_qkv=to_bf16(rng.standard_normal((T, C), dtype=np.float32)),
        a=to_bf16(rng.standard_normal((T, Hv), dtype=np.float32)),
        b=to_bf16(rng.standard_normal((T, Hv), dtype=np.float32)),
        conv_weight=to_bf16(0.5 * rng.standard_normal((C, W), dtype=np.float32)),
        conv_bias=None,
        A_log=rng.uniform(math.log(1.0), math.log(16.0), Hv).astype(np.float32),
        dt_bias=(0.1 * rng.standard_normal(Hv)).astype(np.float32),
        num_actual_tokens=T,
    )


CANARY_SSM = np.float32(0.5)       # value of pool slots no row references
CANARY_CONV = np.uint16(0x3F00)     # bf16 0.5


def _pools(rng, d, slots=None):
    """SSM pool ~ N(0, 0.1) fp32 and conv pool ~ N(0, 1) bf16 on ``slots``
    (all slots when None); every other slot holds the canary value."""
    S, L, C = d["num_slots"], d["L"], conv_dim(d["Hk"], d["Hv"], d["dk"], d["dv"])
    shape = (S, d["Hv"], d["dv"], d["dk"])
    if slots is None:
        ssm = rng.standard_normal(shape, dtype=np.float32)
        ssm *= np.float32(0.1)
        conv = to_bf16(rng.standard_normal((S, L, C), dtype=np.float32))
        return dict(ssm_state=ssm, conv_state=conv)
    slots = np.unique(np.asarray(list(slots), np.int64))
    slots = slots[(slots >= 0) & (slots < S)]
    ssm = np.full(shape, CANARY_SSM, np.float32)
    conv = np.full((S, L, C), CANARY_CONV, np.uint16)
    n = len(slots)
    if n:
        v = rng.standard_normal((n,) + shape[1:], dtype=np.float32)
        v *= np.float32(0.1)
        ssm[slots] = v
        conv[slots] = to_bf16(rng.standard_normal((n, L, C), dtype=np.float32))
    return dict(ssm_state=ssm, conv_state=conv)


def referenced_slots(case, rows=None) -> np.ndarray:
    """Slots the batch's rows read or write (spec rows ``rows`` only, when
    given); slot 0 (NULL) excluded."""
    out = []
    sp = case.get("spec")
    if sp is not None:
        ssi = sp["spec_state_indices"]
        sel = range(sp["num_spec_decodes"]) if rows is None else rows
        for b in sel:
            out.extend(ssi[b].tolist())
            if sp.get("spec_cache_indices") is not None:
                out.append(int(sp["spec_cache_indices"][b]))
    ns = case.get("nonspec")
    if ns is not None and rows is None:
        out.extend(ns["cache_indices"].tolist())
    return np.array(sorted(set(s for s in out if s > 0)), np.int64)


def _spec_meta(rng, Ns, K, slot_lo, slot_hi, null_p=0.0, force_nacc1=False,
               lens=None):
    """Spec rows with K state slots each, distinct slots from [lo, hi)."""
    lens = np.full(Ns, K, np.int32) if lens is None else np.asarray(lens, np.int32)
    sqsl = np.zeros(Ns + 1, np.int32)
    sqsl[1:] = np.cumsum(lens)
    nacc = np.array([rng.integers(1, int(l) + 1) for l in lens], np.int32)
    if force_nacc1 and Ns > 0:
        nacc[rng.integers(0, Ns)] = 1
    slots = rng.choice(np.arange(slot_lo, slot_hi), size=Ns * K, replace=False)
    ssi = slots.reshape(Ns, K).astype(np.int32)
    if null_p > 0.0:
        ssi[rng.random((Ns, K)) < null_p] = 0
        # at least one NULL load and one NULL store that is not also the load
        b0 = 0
        ssi[b0, nacc[b0] - 1] = 0
        if Ns > 1:
            b1 = 1
            j = (nacc[b1]) % lens[b1]
            ssi[b1, j] = 0
    return dict(num_spec_decodes=Ns, K=K, num_spec_tokens=int(sqsl[-1]),
                spec_query_start_loc=sqsl, spec_cache_indices=None,
                spec_state_indices=ssi, num_accepted_tokens=nacc,
                spec_token_indx=None)


def compose_rows(rng, row_kinds, row_lens, keep_first_nonspec=True):
    """Shuffle rows (tokens of a row stay contiguous) and return, per row, its
    global token rows.  ``row_kinds`` holds 's' (spec) or 'n' (non-spec).
    With ``keep_first_nonspec`` the order puts at least one non-spec row
    ahead of a spec row (the layout the gate-gather fix is about)."""
    n = len(row_kinds)
    order = rng.permutation(n)
    if keep_first_nonspec and "n" in row_kinds and "s" in row_kinds:
        kinds = [row_kinds[i] for i in order]
        first_s = kinds.index("s")
        if "n" not in kinds[:first_s]:
            # move the first non-spec row in front
            k = kinds.index("n")
            order = np.concatenate([[order[k]], np.delete(order, k)])
    starts = {}
    pos = 0
    for i in order:
        starts[int(i)] = pos
        pos += int(row_lens[i])
    return [np.arange(starts[i], starts[i] + row_lens[i], dtype=np.int32)
            for i in range(n)]


def make_case(name: str, seed: int = 0, permute_tokens: bool = False,
              with_pools: bool = True, fill="touched", **over) -> dict:
    """Build one workload.  Returns a dict with ``dims``, the parameter and
    input arrays, the pools, and ``spec`` / ``nonspec`` metadata (either may
    be None).  ``fill`` picks the pool slots that get random values:
    "touched" (every slot the batch references), "all", or a list of spec
    row indices whose slots (plus every non-spec slot) are filled."""
    cfg = dict(CONFIGS[name])
    cfg.update(over)
    rng = np.random.default_rng(seed)
    Hk, Hv, dk, dv, W = cfg["Hk"], cfg["Hv"], cfg["dk"], cfg["dv"], cfg["W"]
    K = cfg["K"]
    L = cfg.get("L", W - 1 + K - 1)
    d = dims_of(Hk, Hv, dk, dv, W, L, cfg["num_slots"])
    case = dict(name=name, seed=seed, dims=d)
    if cfg["kind"] == "spec":
        Ns = cfg["Ns"]
        spec = _spec_meta(rng, Ns, K, 1, cfg["num_slots"], cfg.get("null_p", 0.0),
                          cfg.get("force_nacc1", False), cfg.get("lens"))
        T = spec["num_spec_tokens"]
        if permute_tokens:
            spec["spec_token_indx"] = rng.permutation(T).astype(np.int32)
        case.update(_params(rng, d, T))
        case["spec"] = spec
        case["nonspec"] = None
    else:
        Ns, Nd = cfg["Ns"], cfg["Nd"]
        plens = list(cfg["prefill_lens"])
        Np = len(plens)
        half = cfg["num_slots"] // 2 + 1
        spec = _spec_meta(rng, Ns, K, 1, half)
        ns_lens = [1] * Nd + plens
        ns_slots = rng.choice(np.arange(half, cfg["num_slots"]), size=Nd + Np,
                              replace=False).astype(np.int32)
        kinds = ["s"] * Ns + ["n"] * (Nd + Np)
        lens = [K] * Ns + ns_lens
        per_row = compose_rows(rng, kinds, lens)
        T = int(sum(lens))
        spec["spec_token_indx"] = (np.concatenate(per_row[:Ns]).astype(np.int32) if Ns
                                   else np.zeros(0, np.int32))
        qsl = np.zeros(Nd + Np + 1, np.int32)
        qsl[1:] = np.cumsum(ns_lens)
        his = np.ones(Nd + Np, np.uint8)
        if Np >= 2:
            his[Nd + 1] = 0  # second prefill starts fresh
        nonspec = dict(num_decodes=Nd, num_prefills=Np,
                       num_non_spec_tokens=int(qsl[-1]), query_start_loc=qsl,
                       cache_indices=ns_slots, has_initial_state=his,
                       token_indx=(np.concatenate(per_row[Ns:]).astype(np.int32)
                                   if Nd + Np else np.zeros(0, np.int32)))
        case.update(_params(rng, d, T))
        case["spec"] = spec
        case["nonspec"] = nonspec
    if with_pools:
        if isinstance(fill, str) and fill == "all":
            slots = None
        elif isinstance(fill, str) and fill == "touched":
            slots = referenced_slots(case)
        else:
            slots = np.union1d(referenced_slots(case, rows=list(fill)),
                               referenced_slots(dict(nonspec=case["nonspec"])))
        case.update(_pools(rng, d, slots))
    return case
