"""GPU-side helpers for the parity tests: upload a synthetic case, call the
HIP library through the C-ABI binding, download what to compare, and the
comparison rules:

  * conv-state ring and slot bookkeeping: bit-exact;
  * core_attn_out (bf16): |gpu - ref| <= 2e-2 + 2e-2 |ref| (the allclose form
    of the bf16 tolerance of the replay harness on the spec-decoding kernel
    page, "Test Plan");
  * SSM state: per (slot, v-head) tile, max |gpu - ref| <= 1e-3 max |ref|;
  * slots and output rows the batch does not name keep their canary bytes.
"""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

import synth

OUT_ATOL = 2e-2
OUT_RTOL = 2e-2
STATE_RTOL = 1e-3
OUT_CANARY = np.uint16(0x5A5A)


def say(msg):
    """Name the GPU step before it runs (flushed, so a fault still shows it)."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def cfg_of(case):
    import speculative_decoding_causal_amd as gdn
    d = case["dims"]
    return gdn.GdnConfig(d["Hk"], d["Hv"], d["dk"], d["dv"], d["W"], d["activation"],
                         d["use_qk_l2norm"], d["eps"], d["scale"],
                         conv_layout=int(d.get("conv_layout", 0)))


def bf(x, device=None):
    x = np.ascontiguousarray(x, np.uint16)
    return torch.from_numpy(x.view(np.int16)).to(device or dev()).view(torch.bfloat16)


def i32(x, device=None):
    if x is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(x, np.int32)).to(device or dev())


def u8(x, device=None):
    if x is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(x, np.uint8)).to(device or dev())


def f32(x, device=None):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(device or dev())


def to_np_bf16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


class Gpu:
    """A case resident on the GPU.  With ``turns`` (the default) the calls
    pass the pool's turn counters, so batches large enough run the
    (row, v-head) form of the row kernel; ``turns=False`` keeps the
    (row, k-head) form everywhere."""

    def __init__(self, case, out=None, turns=True):
        import speculative_decoding_causal_amd as gdn
        self.case = case
        self.cfg = cfg_of(case)
        d = case["dims"]
        self.qkv = bf(case["mixed_qkv"])
        self.a = bf(case["a"])
        self.b = bf(case["b"])
        self.w = bf(case["conv_weight"])
        self.bias = None if case.get("conv_bias") is None else bf(case["conv_bias"])
        self.A_log = f32(case["A_log"])
        self.dt_bias = f32(case["dt_bias"])
        self.conv = bf(case["conv_state"])
        self.ssm = f32(case["ssm_state"])
        T = case["num_actual_tokens"]
        if out is None:
            out = np.full((T, d["Hv"], d["dv"]), OUT_CANARY, np.uint16)
        self.out = bf(out)
        self.turns = gdn.conv_turns(self.cfg, d["num_slots"], dev()) if turns else None

    def spec(self, spec=None, stream=None):
        import speculative_decoding_causal_amd as gdn
        sp = self.case["spec"] if spec is None else spec
        gdn.gdn_spec_attention(
            self.cfg, self.qkv, self.a, self.b, self.w, self.bias, self.A_log, self.dt_bias,
            self.conv, self.ssm, i32(sp["spec_query_start_loc"]),
            i32(sp["spec_state_indices"]), i32(sp["num_accepted_tokens"]), self.out,
            spec_cache_indices=i32(sp.get("spec_cache_indices")),
            spec_token_indx=i32(sp.get("spec_token_indx")),
            num_spec_tokens=int(sp["num_spec_tokens"]), conv_turns=self.turns, stream=stream)

    def decode_row(self, r, slot, his=1):
        """One non-spec one-token decode of global row r on ``slot`` (tensors
        sliced to that row, so the call's batch is exactly one token)."""
        import speculative_decoding_causal_amd as gdn
        sl = slice(r, r + 1)
        gdn.gdn_attention(self.cfg, self.qkv[sl], self.a[sl], self.b[sl], self.w, self.bias,
                          self.A_log, self.dt_bias, self.conv, self.ssm, self.out[sl],
                          num_decodes=1, num_non_spec_tokens=1,
                          query_start_loc=i32([0, 1]), non_spec_state_indices=i32([slot]),
                          has_initial_state=u8([his]), conv_turns=self.turns)

    def attention(self, ns="case", spec="case", workspace=None):
        import speculative_decoding_causal_amd as gdn
        ns = self.case.get("nonspec") if isinstance(ns, str) else ns
        sp = self.case.get("spec") if isinstance(spec, str) else spec
        kw = {}
        if ns is not None:
            kw.update(num_decodes=ns["num_decodes"], num_prefills=ns["num_prefills"],
                      num_non_spec_tokens=ns["num_non_spec_tokens"],
                      query_start_loc=i32(ns["query_start_loc"]),
                      non_spec_state_indices=i32(ns["cache_indices"]),
                      has_initial_state=u8(ns.get("has_initial_state")),
                      non_spec_token_indx=i32(ns.get("token_indx")))
        if sp is not None:
            kw.update(spec_query_start_loc=i32(sp["spec_query_start_loc"]),
                      spec_state_indices=i32(sp["spec_state_indices"]),
                      num_accepted_tokens=i32(sp["num_accepted_tokens"]),
                      spec_cache_indices=i32(sp.get("spec_cache_indices")),
                      spec_token_indx=i32(sp.get("spec_token_indx")),
                      num_spec_tokens=int(sp["num_spec_tokens"]))
        if workspace is None and ns is not None and ns["num_prefills"] > 0:
            d = self.case["dims"]
            nbytes = gdn.gdn_workspace_bytes(self.cfg, d["L"], d["num_slots"],
                                             ns["num_non_spec_tokens"], ns["num_prefills"])
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev())
        gdn.gdn_attention(self.cfg, self.qkv, self.a, self.b, self.w, self.bias, self.A_log,
                          self.dt_bias, self.conv, self.ssm, self.out, workspace=workspace,
                          conv_turns=self.turns, **kw)

    def host_out(self):
        return to_np_bf16(self.out)

    def host_conv(self, slots=None):
        c = self.conv if slots is None else self.conv[torch.as_tensor(np.asarray(slots), device=dev())]
        return to_np_bf16(c)

    def host_ssm(self, slots=None):
        s = self.ssm if slots is None else self.ssm[torch.as_tensor(np.asarray(slots), device=dev())]
        return s.cpu().numpy()


def assert_out_close(gpu, ref, rows=None, what="core_attn_out"):
    g = synth.from_bf16(gpu if rows is None else gpu[rows]).astype(np.float64)
    r = synth.from_bf16(ref if rows is None else ref[rows]).astype(np.float64)
    err = np.abs(g - r)
    # written so that a NaN or an infinity on either side is a failure
    bad = ~(err <= OUT_ATOL + OUT_RTOL * np.abs(r))
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; "
                             f"max err {err.max():.4g}; first at {idx.tolist()}")


def assert_states_close(gpu, ref, what="ssm_state"):
    """gpu/ref: [..., dv, dk] tiles; per-tile relative max-norm check."""
    g = gpu.reshape(-1, gpu.shape[-2] * gpu.shape[-1]).astype(np.float64)
    r = ref.reshape(-1, ref.shape[-2] * ref.shape[-1]).astype(np.float64)
    err = np.abs(g - r).max(axis=1)
    scale = np.abs(r).max(axis=1)
    bad = ~(err <= STATE_RTOL * scale + 1e-30)  # NaN anywhere in a tile fails it
    if bad.any():
        i = int(np.argmax(bad))
        raise AssertionError(f"{what}: {bad.sum()} of {len(bad)} tiles outside 1e-3 relative; "
                             f"tile {i}: err {err[i]:.4g} vs max {scale[i]:.4g}")


def sub_spec(spec, rows):
    """The spec metadata restricted to rows ``rows`` (their tokens keep their
    global rows through spec_token_indx)."""
    sq = spec["spec_query_start_loc"]
    tix = spec["spec_token_indx"]
    lens, glob, ssi, nacc, cache = [], [], [], [], []
    for b in rows:
        j0, j1 = int(sq[b]), int(sq[b + 1])
        lens.append(j1 - j0)
        glob.extend(tix[j0:j1] if tix is not None else range(j0, j1))
        ssi.append(spec["spec_state_indices"][b])
        nacc.append(spec["num_accepted_tokens"][b])
        if spec.get("spec_cache_indices") is not None:
            cache.append(spec["spec_cache_indices"][b])
    sqsl = np.zeros(len(rows) + 1, np.int32)
    sqsl[1:] = np.cumsum(lens)
    return dict(num_spec_decodes=len(rows), K=spec["K"], num_spec_tokens=int(sqsl[-1]),
                spec_query_start_loc=sqsl,
                spec_cache_indices=np.array(cache, np.int32) if cache else None,
                spec_state_indices=np.array(ssi, np.int32).reshape(len(rows), spec["K"]),
                num_accepted_tokens=np.array(nacc, np.int32),
                spec_token_indx=np.array(glob, np.int32))


def spec_rows_of(spec, rows):
    """Global token rows and touched slots of spec rows ``rows``."""
    sq = spec["spec_query_start_loc"]
    tix = spec["spec_token_indx"]
    glob, slots = [], set()
    for b in rows:
        j0, j1 = int(sq[b]), int(sq[b + 1])
        glob.extend(tix[j0:j1] if tix is not None else range(j0, j1))
        slots.update(int(s) for s in spec["spec_state_indices"][b] if s > 0)
        if spec.get("spec_cache_indices") is not None and spec["spec_cache_indices"][b] > 0:
            slots.add(int(spec["spec_cache_indices"][b]))
    return np.array(glob, np.int64), np.array(sorted(slots), np.int64)


def gpu_available():
    return torch.cuda.is_available() and os.path.exists(
        os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                     "speculative_decoding_causal_amd", "libgdn.so"))
