"""CPU oracle for the speculative-decoding-aware Gated DeltaNet step.

TEST INFRASTRUCTURE ONLY: ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
path (``speculative_decoding_causal_amd``) never does, and this package never
imports the product path: the two share no code.

The arithmetic lives in ``gdn_oracle.c`` (plain C, double precision); this
module only builds it with gcc, loads it with ctypes and marshals numpy
arrays.  bf16 tensors are carried as ``numpy.uint16`` bit patterns.

Function map (see the C file for the citations of each step):
  * ``gates``        - decay alpha and write strength beta per (token, head)
  * ``spec_step``    - one spec-verify call (conv window at n_acc-1, rolled
                        ring, per-token SSM snapshots, NULL slots, token_indx)
  * ``nonspec_step`` - non-spec rows (decodes and prefills, sequential
                        recurrence, tail window, final-state store)
  * ``bf16_round``   - the oracle's own double -> bf16 rounding
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

# No fast-math and no FMA contraction: the double-precision sums are formed
# exactly as written in the source.
CFLAGS = ["-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(force: bool = True) -> str:
    """Compile ``liboracle.so`` with gcc (always, when ``force``)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class Dims(ctypes.Structure):
    _fields_ = [
        ("num_k_heads", ctypes.c_int32),
        ("num_v_heads", ctypes.c_int32),
        ("head_k_dim", ctypes.c_int32),
        ("head_v_dim", ctypes.c_int32),
        ("conv_width", ctypes.c_int32),
        ("state_len", ctypes.c_int32),
        ("num_slots", ctypes.c_int32),
        ("activation", ctypes.c_int32),
        ("use_qk_l2norm", ctypes.c_int32),
        ("conv_layout", ctypes.c_int32),
        ("l2norm_eps", ctypes.c_double),
        ("scale", ctypes.c_double),
    ]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i32 = ctypes.c_int32
        lib.oracle_gates.argtypes = [i32, i32, P, P, P, P, P, P]
        lib.oracle_gates.restype = ctypes.c_int
        lib.oracle_spec_step.argtypes = [ctypes.POINTER(Dims)] + [P] * 9 + [
            i32, i32, i32, P, P, P, P, P, P, P]
        lib.oracle_spec_step.restype = ctypes.c_int
        lib.oracle_nonspec_step.argtypes = [ctypes.POINTER(Dims)] + [P] * 9 + [
            i32, i32, P, P, P, P, P, P]
        lib.oracle_nonspec_step.restype = ctypes.c_int
        lib.oracle_bf16_round.argtypes = [ctypes.c_double]
        lib.oracle_bf16_round.restype = ctypes.c_uint16
        _lib = lib
    return _lib


def _ptr(arr, dtype=None):
    if arr is None:
        return None
    if dtype is not None and arr.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {arr.dtype}")
    if not arr.flags.c_contiguous:
        raise ValueError("arrays passed to the oracle must be C-contiguous")
    return arr.ctypes.data


def make_dims(d: dict) -> Dims:
    return Dims(int(d["Hk"]), int(d["Hv"]), int(d["dk"]), int(d["dv"]),
                int(d["W"]), int(d["L"]), int(d["num_slots"]),
                int(d.get("activation", 1)), int(d.get("use_qk_l2norm", 1)),
                int(d.get("conv_layout", 0)),
                float(d.get("eps", 1e-6)), float(d["scale"]))


def gates(a, b, A_log, dt_bias):
    """alpha, beta (float64) for bf16 gate rows ``a``/``b`` of shape [n, Hv]."""
    a = np.ascontiguousarray(a, dtype=np.uint16)
    b = np.ascontiguousarray(b, dtype=np.uint16)
    Hv = a.shape[-1]
    n = a.size
    alpha = np.empty(a.shape, np.float64)
    beta = np.empty(a.shape, np.float64)
    A_log = np.ascontiguousarray(A_log, dtype=np.float32)
    dt_bias = np.ascontiguousarray(dt_bias, dtype=np.float32)
    rc = _load().oracle_gates(n, Hv, _ptr(a), _ptr(b), _ptr(A_log),
                              _ptr(dt_bias), _ptr(alpha), _ptr(beta))
    if rc != 0:
        raise ValueError(f"oracle_gates failed ({rc})")
    return alpha, beta


def bf16_round(x: float) -> int:
    return int(_load().oracle_bf16_round(float(x)))


def _i32(x):
    return None if x is None else np.ascontiguousarray(x, dtype=np.int32)


def spec_step(dims: dict, t: dict, spec: dict, out: np.ndarray,
              conv_out: np.ndarray | None = None) -> None:
    """Run one spec-verify call in place on ``t['conv_state']``,
    ``t['ssm_state']`` and ``out`` (uint16 [T, Hv, dv])."""
    d = make_dims(dims)
    sqsl = _i32(spec["spec_query_start_loc"])
    ci = _i32(spec.get("spec_cache_indices"))
    ssi = _i32(spec["spec_state_indices"])
    nacc = _i32(spec["num_accepted_tokens"])
    tix = _i32(spec.get("spec_token_indx"))
    rc = _load().oracle_spec_step(
        ctypes.byref(d), _ptr(t["mixed_qkv"], np.uint16), _ptr(t["a"], np.uint16),
        _ptr(t["b"], np.uint16), _ptr(t["conv_weight"], np.uint16),
        _ptr(t.get("conv_bias"), np.uint16), _ptr(t["A_log"], np.float32),
        _ptr(t["dt_bias"], np.float32), _ptr(t["conv_state"], np.uint16),
        _ptr(t["ssm_state"], np.float32), int(t["num_actual_tokens"]),
        int(spec["num_spec_decodes"]), int(spec["K"]), _ptr(sqsl), _ptr(ci),
        _ptr(ssi), _ptr(nacc), _ptr(tix), _ptr(out, np.uint16),
        _ptr(conv_out, np.float64))
    if rc != 0:
        raise ValueError(f"oracle_spec_step rejected the metadata ({rc})")


def nonspec_step(dims: dict, t: dict, ns: dict, out: np.ndarray,
                 conv_out: np.ndarray | None = None) -> None:
    """Run the non-spec rows (decodes then prefills) in place."""
    d = make_dims(dims)
    qsl = _i32(ns["query_start_loc"])
    ci = _i32(ns["cache_indices"])
    his = ns.get("has_initial_state")
    his = None if his is None else np.ascontiguousarray(his, dtype=np.uint8)
    tix = _i32(ns.get("token_indx"))
    nrows = int(ns["num_decodes"]) + int(ns["num_prefills"])
    rc = _load().oracle_nonspec_step(
        ctypes.byref(d), _ptr(t["mixed_qkv"], np.uint16), _ptr(t["a"], np.uint16),
        _ptr(t["b"], np.uint16), _ptr(t["conv_weight"], np.uint16),
        _ptr(t.get("conv_bias"), np.uint16), _ptr(t["A_log"], np.float32),
        _ptr(t["dt_bias"], np.float32), _ptr(t["conv_state"], np.uint16),
        _ptr(t["ssm_state"], np.float32), int(t["num_actual_tokens"]), nrows,
        _ptr(qsl), _ptr(ci), _ptr(his), _ptr(tix), _ptr(out, np.uint16),
        _ptr(conv_out, np.float64))
    if rc != 0:
        raise ValueError(f"oracle_nonspec_step rejected the metadata ({rc})")
