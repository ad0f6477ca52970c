"""MI355X-native Gated DeltaNet attention step with speculative decoding.

Thin ctypes binding over ``libgdn.so`` (HIP kernels for gfx950 behind a C
ABI declared in ``include/gdn.h``).  This module only marshals arguments:
dtype / contiguity / device checks, size checks of every tensor the kernels
index (plain pointers carry no size), sizes derived from tensor shapes, the
current HIP stream.  Every step of the computation runs in the library's
kernels; there is no CPU fallback, and importing fails loudly when the
library has not been built.

Entry points (same names as the C ABI):
  gdn_spec_attention, gdn_attention, gdn_attention_static, gdn_workspace_bytes, gdn_conv_only,
  gdn_delta_rule_only, gdn_check_metadata_host, gdn_status_string,
  gdn_last_error.
Capture and replay of step calls: ``speculative_decoding_causal_amd.capture``.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# GDN_LIBRARY names another build of the library (e.g. one with the host
# code under AddressSanitizer, from `build.py --asan`); default: in-tree.
LIB_PATH = os.environ.get("GDN_LIBRARY") or os.path.join(_HERE, "libgdn.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with "
        "`python speculative_decoding_causal_amd/build.py` (hipcc, gfx950)")

_lib = ctypes.CDLL(LIB_PATH)

GDN_OK = 0
GDN_ERR_NULL = -1
GDN_ERR_DIMS = -2
GDN_ERR_SPEC_PAIR = -3
GDN_ERR_MISSING_OPTIONAL = -4
GDN_ERR_CONSERVATION = -5
GDN_ERR_WORKSPACE = -6
GDN_ERR_HIP = -7
GDN_ERR_UNSUPPORTED = -8
GDN_ERR_METADATA = -9
GDN_QKV_GROUPED = 0
GDN_QKV_PER_K_HEAD = 1
GDN_CONV_ROLLED_HISTORY = 0
GDN_CONV_PER_TOKEN_SLOTS = 1
GDN_ROWS_NON_SPEC = 0
GDN_ROWS_SPEC = 1
MAX_ROW_TOKENS = 16

EXPORTED_SYMBOLS = (
    "gdn_spec_attention", "gdn_attention", "gdn_attention_static", "gdn_workspace_bytes",
    "gdn_conv_turns_count",
    "gdn_conv_only", "gdn_delta_rule_only", "gdn_check_metadata_host",
    "gdn_status_string", "gdn_last_error",
)


class GdnDims(ctypes.Structure):
    _fields_ = [
        ("num_k_heads", ctypes.c_int32), ("num_v_heads", ctypes.c_int32),
        ("head_k_dim", ctypes.c_int32), ("head_v_dim", ctypes.c_int32),
        ("conv_width", ctypes.c_int32), ("state_len", ctypes.c_int32),
        ("num_slots", ctypes.c_int32), ("activation", ctypes.c_int32),
        ("use_qk_l2norm", ctypes.c_int32), ("l2norm_eps", ctypes.c_float),
        ("scale", ctypes.c_float), ("qkv_layout", ctypes.c_int32),
        ("conv_layout", ctypes.c_int32),
    ]


class GdnRows(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32), ("num_rows", ctypes.c_int32),
        ("num_tokens", ctypes.c_int32), ("max_row_tokens", ctypes.c_int32),
        ("query_start_loc", ctypes.c_void_p), ("cache_indices", ctypes.c_void_p),
        ("state_indices", ctypes.c_void_p), ("num_accepted_tokens", ctypes.c_void_p),
        ("has_initial_state", ctypes.c_void_p), ("token_indx", ctypes.c_void_p),
    ]


_P = ctypes.c_void_p
_I = ctypes.c_int32
_lib.gdn_spec_attention.argtypes = ([ctypes.POINTER(GdnDims)] + [_P] * 9 + [_I] * 4 + [_P] * 6 +
                                    [_P, _P])
_lib.gdn_spec_attention.restype = ctypes.c_int
_lib.gdn_attention.argtypes = ([ctypes.POINTER(GdnDims)] + [_P] * 9 + [_I] * 4 + [_P] * 4 +
                               [_I] * 3 + [_P] * 5 + [_P, _P, _P, ctypes.c_size_t, _P])
_lib.gdn_attention.restype = ctypes.c_int
_lib.gdn_attention_static.argtypes = ([ctypes.POINTER(GdnDims)] + [_P] * 9 + [_I] * 4 + [_P] * 4 +
                                      [_I] * 3 + [_P] * 5 + [_P, _P, _P])
_lib.gdn_attention_static.restype = ctypes.c_int
STATIC_SCRATCH_BYTES = 64 << 20   # GDN_STATIC_SCRATCH_BYTES
_lib.gdn_workspace_bytes.argtypes = [ctypes.POINTER(GdnDims), _I, _I]
_lib.gdn_workspace_bytes.restype = ctypes.c_size_t
_lib.gdn_conv_turns_count.argtypes = [ctypes.POINTER(GdnDims)]
_lib.gdn_conv_turns_count.restype = ctypes.c_size_t
_lib.gdn_conv_only.argtypes = [ctypes.POINTER(GdnDims), _P, _P, _P, _P, _I,
                               ctypes.POINTER(GdnRows), _P, _P]
_lib.gdn_conv_only.restype = ctypes.c_int
_lib.gdn_delta_rule_only.argtypes = [ctypes.POINTER(GdnDims), _P, _P, _P, _P, _P, _P, _I,
                                     ctypes.POINTER(GdnRows), _P, _P]
_lib.gdn_delta_rule_only.restype = ctypes.c_int
class GdnHostI32(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("len", ctypes.c_int64)]


_lib.gdn_check_metadata_host.argtypes = ([ctypes.POINTER(GdnDims), _I, _I, _I, _I] +
                                         [GdnHostI32] * 3 + [_I, _I, _I] + [GdnHostI32] * 5)
_lib.gdn_check_metadata_host.restype = ctypes.c_int
_lib.gdn_status_string.argtypes = [ctypes.c_int]
_lib.gdn_status_string.restype = ctypes.c_char_p
_lib.gdn_last_error.argtypes = []
_lib.gdn_last_error.restype = ctypes.c_char_p


class GdnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = gdn_last_error()
        super().__init__(f"{where}: {gdn_status_string(status)} ({status}): {msg}")


def gdn_status_string(status: int) -> str:
    return _lib.gdn_status_string(int(status)).decode()


def gdn_last_error() -> str:
    return _lib.gdn_last_error().decode()


@dataclass
class GdnConfig:
    """Layer shape; ``state_len`` and ``num_slots`` come from the pools."""
    num_k_heads: int
    num_v_heads: int
    head_k_dim: int
    head_v_dim: int
    conv_width: int = 4
    activation: int = 1          # 0 identity, 1 SiLU
    use_qk_l2norm: int = 1
    l2norm_eps: float = 1e-6
    scale: float | None = None   # default head_k_dim ** -0.5
    # mixed_qkv channel order: True = grouped [q | k | v] (GDN_QKV_GROUPED),
    # False = per k-head [q_i k_i v_i ...] as projected (GDN_QKV_PER_K_HEAD)
    reorder_input: bool = True
    # conv state of spec rows: GDN_CONV_ROLLED_HISTORY (one rolled ring per
    # row) or GDN_CONV_PER_TOKEN_SLOTS (a window per token slot, L = W-1)
    conv_layout: int = GDN_CONV_ROLLED_HISTORY

    @property
    def conv_dim(self) -> int:
        return 2 * self.num_k_heads * self.head_k_dim + self.num_v_heads * self.head_v_dim

    def dims(self, conv_state: torch.Tensor | None = None,
             state_len: int | None = None, num_slots: int | None = None) -> GdnDims:
        if conv_state is not None:
            num_slots, state_len = int(conv_state.shape[0]), int(conv_state.shape[1])
        scale = self.head_k_dim ** -0.5 if self.scale is None else self.scale
        return GdnDims(self.num_k_heads, self.num_v_heads, self.head_k_dim,
                       self.head_v_dim, self.conv_width, int(state_len),
                       int(num_slots), self.activation, self.use_qk_l2norm,
                       float(self.l2norm_eps), float(scale),
                       GDN_QKV_GROUPED if self.reorder_input else GDN_QKV_PER_K_HEAD,
                       int(self.conv_layout))


def _ptr(t, dtype=None, name="tensor", device=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (the kernels read device memory)")
    return t.data_ptr()


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_I32 = torch.int32


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _check_pools(cfg: GdnConfig, conv_state, ssm_state):
    if conv_state.dim() != 3 or conv_state.shape[2] != cfg.conv_dim:
        raise ValueError(f"conv_state must be [num_slots, state_len, {cfg.conv_dim}]")
    want = (conv_state.shape[0], cfg.num_v_heads, cfg.head_v_dim, cfg.head_k_dim)
    if tuple(ssm_state.shape) != want:
        raise ValueError(f"ssm_state must be {list(want)}, got {list(ssm_state.shape)}")


def _need(t, name, shape=None, at_least=None):
    """Size check of a tensor the kernels index (plain pointers carry no
    size, so a short tensor would be read or written past its end)."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be {list(shape)}, got {list(t.shape)}")
    if at_least is not None and t.numel() < at_least:
        raise ValueError(f"{name} holds {t.numel()} values; the call needs {at_least}")


def _check_layer(cfg: GdnConfig, nat, mixed_qkv, a, b, conv_weight, conv_bias, A_log, dt_bias,
                 core_attn_out):
    C, Hv = cfg.conv_dim, cfg.num_v_heads
    if mixed_qkv.dim() != 2 or mixed_qkv.shape[1] != C or mixed_qkv.shape[0] < nat:
        raise ValueError(f"mixed_qkv must be [>= {nat}, {C}], got {list(mixed_qkv.shape)}")
    _need(a, "a", at_least=nat * Hv)
    _need(b, "b", at_least=nat * Hv)
    _need(conv_weight, "conv_weight", shape=(C, cfg.conv_width))
    _need(conv_bias, "conv_bias", shape=(C,))
    _need(A_log, "A_log", shape=(Hv,))
    _need(dt_bias, "dt_bias", shape=(Hv,))
    _need(core_attn_out, "core_attn_out", at_least=nat * Hv * cfg.head_v_dim)


def _check_spec_meta(Ns, K, Ts, ssi, nacc, scache, stix):
    if Ns <= 0:
        return
    _need(ssi, "spec_state_indices", at_least=Ns * K)
    _need(nacc, "num_accepted_tokens", at_least=Ns)
    _need(scache, "spec_cache_indices", at_least=Ns)
    _need(stix, "spec_token_indx", at_least=Ts)


def _check_nonspec_meta(rows, tokens, qsl, nsi, his, ntix):
    if rows <= 0:
        return
    _need(qsl, "query_start_loc", at_least=rows + 1)
    _need(nsi, "non_spec_state_indices", at_least=rows)
    _need(his, "has_initial_state", at_least=rows)
    _need(ntix, "non_spec_token_indx", at_least=tokens)


def _host_count(x, given):
    if given is not None:
        return int(given)
    return int(x[-1].item())  # synchronises; pass the count to avoid it


def gdn_spec_attention(cfg: GdnConfig, mixed_qkv, a, b, conv_weight, conv_bias,
                       A_log, dt_bias, conv_state, ssm_state,
                       spec_query_start_loc, spec_state_indices,
                       num_accepted_tokens, core_attn_out,
                       spec_cache_indices=None, spec_token_indx=None,
                       num_spec_tokens: int | None = None, num_actual_tokens: int | None = None,
                       conv_turns=None, stream=None) -> None:
    """One spec-verify step (see ``include/gdn.h``); pools are updated in
    place and ``core_attn_out`` [num_actual_tokens, Hv, dv] is written at the
    rows named by ``spec_token_indx``.  ``num_actual_tokens`` defaults to the
    rows of ``mixed_qkv``; pass ``num_spec_tokens`` too when capturing the
    call in a graph (it is read back from the device otherwise).
    ``conv_turns``: None, or the pool's turn counters from ``conv_turns``."""
    dev = mixed_qkv.device
    _check_pools(cfg, conv_state, ssm_state)
    dims = cfg.dims(conv_state)
    nat = int(mixed_qkv.shape[0] if num_actual_tokens is None else num_actual_tokens)
    _check_layer(cfg, nat, mixed_qkv, a, b, conv_weight, conv_bias, A_log, dt_bias,
                 core_attn_out)
    Ns = int(spec_query_start_loc.shape[0]) - 1 if spec_query_start_loc is not None else 0
    K = int(spec_state_indices.shape[1]) if spec_state_indices is not None else 1
    T = _host_count(spec_query_start_loc, num_spec_tokens) if Ns > 0 else 0
    _check_spec_meta(Ns, K, T, spec_state_indices, num_accepted_tokens, spec_cache_indices,
                     spec_token_indx)
    rc = _lib.gdn_spec_attention(
        ctypes.byref(dims), _ptr(mixed_qkv, _BF16, "mixed_qkv", dev), _ptr(a, _BF16, "a", dev),
        _ptr(b, _BF16, "b", dev), _ptr(conv_weight, _BF16, "conv_weight", dev),
        _ptr(conv_bias, _BF16, "conv_bias", dev), _ptr(A_log, torch.float32, "A_log", dev),
        _ptr(dt_bias, torch.float32, "dt_bias", dev), _ptr(conv_state, _BF16, "conv_state", dev),
        _ptr(ssm_state, torch.float32, "ssm_state", dev), nat, Ns, T, K,
        _ptr(spec_query_start_loc, _I32, "spec_query_start_loc", dev),
        _ptr(spec_cache_indices, _I32, "spec_cache_indices", dev),
        _ptr(spec_state_indices, _I32, "spec_state_indices", dev),
        _ptr(num_accepted_tokens, _I32, "num_accepted_tokens", dev),
        _ptr(spec_token_indx, _I32, "spec_token_indx", dev),
        _ptr(core_attn_out, _BF16, "core_attn_out", dev),
        _turns_ptr(cfg, conv_state, conv_turns, dev), _stream(stream))
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_spec_attention")


def conv_turns(cfg: GdnConfig, num_slots: int, device=None):
    """Zeroed turn counters for a conv pool of ``num_slots`` slots (four per
    (slot, k-head)); keep them with the pool and pass them to every call on
    it (see ``gdn_spec_attention`` in ``include/gdn.h``)."""
    dims = cfg.dims(state_len=cfg.conv_width - 1, num_slots=num_slots)
    n = int(_lib.gdn_conv_turns_count(ctypes.byref(dims)))
    return torch.zeros(n, dtype=torch.int32, device=device)


def _turns_ptr(cfg, conv_state, turns, dev):
    if turns is None:
        return None
    n = 4 * int(conv_state.shape[0]) * cfg.num_k_heads
    if turns.dtype != torch.int32 or turns.numel() != n:
        raise ValueError(f"conv_turns must be int32 with {n} entries (4 * num_slots * "
                         "num_k_heads)")
    return _ptr(turns, torch.int32, "conv_turns", dev)


def gdn_workspace_bytes(cfg: GdnConfig, state_len: int, num_slots: int,
                        max_non_spec_tokens: int, max_prefill_rows: int) -> int:
    dims = cfg.dims(state_len=state_len, num_slots=num_slots)
    return int(_lib.gdn_workspace_bytes(ctypes.byref(dims), int(max_non_spec_tokens),
                                        int(max_prefill_rows)))


def gdn_attention(cfg: GdnConfig, mixed_qkv, a, b, conv_weight, conv_bias, A_log,
                  dt_bias, conv_state, ssm_state, core_attn_out, *,
                  num_decodes=0, num_prefills=0, num_non_spec_tokens=0,
                  query_start_loc=None, non_spec_state_indices=None,
                  has_initial_state=None, non_spec_token_indx=None,
                  spec_query_start_loc=None, spec_state_indices=None,
                  num_accepted_tokens=None, spec_cache_indices=None,
                  spec_token_indx=None, num_spec_tokens=None, workspace=None,
                  num_actual_tokens=None, conv_turns=None, stream=None) -> None:
    """A layer step over a batch of non-spec rows (decodes, then prefills)
    and spec rows.  ``workspace`` (uint8 device tensor) is needed when
    ``num_prefills > 0``; size it with ``gdn_workspace_bytes``.
    ``conv_turns``: None, or the pool's turn counters."""
    _attention(False, cfg, mixed_qkv, a, b, conv_weight, conv_bias, A_log, dt_bias, conv_state,
               ssm_state, core_attn_out, num_decodes, num_prefills, num_non_spec_tokens,
               query_start_loc, non_spec_state_indices, has_initial_state, non_spec_token_indx,
               spec_query_start_loc, spec_state_indices, num_accepted_tokens, spec_cache_indices,
               spec_token_indx, num_spec_tokens, workspace, num_actual_tokens, conv_turns,
               stream)


def gdn_attention_static(cfg: GdnConfig, mixed_qkv, a, b, conv_weight, conv_bias, A_log,
                         dt_bias, conv_state, ssm_state, core_attn_out, *,
                         num_decodes=0, num_prefills=0, num_non_spec_tokens=0,
                         query_start_loc=None, non_spec_state_indices=None,
                         has_initial_state=None, non_spec_token_indx=None,
                         spec_query_start_loc=None, spec_state_indices=None,
                         num_accepted_tokens=None, spec_cache_indices=None,
                         spec_token_indx=None, num_spec_tokens=None,
                         num_actual_tokens=None, conv_turns=None, stream=None) -> None:
    """``gdn_attention`` without a workspace: prefill rows use the library's
    static per-GPU scratch (STATIC_SCRATCH_BYTES); nothing is allocated.
    Calls that overlap on one GPU share that scratch and race."""
    _attention(True, cfg, mixed_qkv, a, b, conv_weight, conv_bias, A_log, dt_bias, conv_state,
               ssm_state, core_attn_out, num_decodes, num_prefills, num_non_spec_tokens,
               query_start_loc, non_spec_state_indices, has_initial_state, non_spec_token_indx,
               spec_query_start_loc, spec_state_indices, num_accepted_tokens, spec_cache_indices,
               spec_token_indx, num_spec_tokens, None, num_actual_tokens, conv_turns, stream)


def _attention(static, cfg, mixed_qkv, a, b, conv_weight, conv_bias, A_log, dt_bias, conv_state,
               ssm_state, core_attn_out, num_decodes, num_prefills, num_non_spec_tokens,
               query_start_loc, non_spec_state_indices, has_initial_state, non_spec_token_indx,
               spec_query_start_loc, spec_state_indices, num_accepted_tokens, spec_cache_indices,
               spec_token_indx, num_spec_tokens, workspace, num_actual_tokens, turns, stream):
    dev = mixed_qkv.device
    _check_pools(cfg, conv_state, ssm_state)
    dims = cfg.dims(conv_state)
    nat = int(mixed_qkv.shape[0] if num_actual_tokens is None else num_actual_tokens)
    _check_layer(cfg, nat, mixed_qkv, a, b, conv_weight, conv_bias, A_log, dt_bias,
                 core_attn_out)
    Ns = int(spec_query_start_loc.shape[0]) - 1 if spec_query_start_loc is not None else 0
    K = int(spec_state_indices.shape[1]) if spec_state_indices is not None else 1
    Ts = _host_count(spec_query_start_loc, num_spec_tokens) if Ns > 0 else 0
    _check_spec_meta(Ns, K, Ts, spec_state_indices, num_accepted_tokens, spec_cache_indices,
                     spec_token_indx)
    _check_nonspec_meta(int(num_decodes) + int(num_prefills), int(num_non_spec_tokens),
                        query_start_loc, non_spec_state_indices, has_initial_state,
                        non_spec_token_indx)
    args = [
        ctypes.byref(dims), _ptr(mixed_qkv, _BF16, "mixed_qkv", dev), _ptr(a, _BF16, "a", dev),
        _ptr(b, _BF16, "b", dev), _ptr(conv_weight, _BF16, "conv_weight", dev),
        _ptr(conv_bias, _BF16, "conv_bias", dev), _ptr(A_log, torch.float32, "A_log", dev),
        _ptr(dt_bias, torch.float32, "dt_bias", dev), _ptr(conv_state, _BF16, "conv_state", dev),
        _ptr(ssm_state, torch.float32, "ssm_state", dev), nat,
        int(num_decodes), int(num_prefills), int(num_non_spec_tokens),
        _ptr(query_start_loc, _I32, "query_start_loc", dev),
        _ptr(non_spec_state_indices, _I32, "non_spec_state_indices", dev),
        _ptr(has_initial_state, (torch.uint8, torch.bool), "has_initial_state", dev),
        _ptr(non_spec_token_indx, _I32, "non_spec_token_indx", dev),
        Ns, Ts, K,
        _ptr(spec_query_start_loc, _I32, "spec_query_start_loc", dev),
        _ptr(spec_cache_indices, _I32, "spec_cache_indices", dev),
        _ptr(spec_state_indices, _I32, "spec_state_indices", dev),
        _ptr(num_accepted_tokens, _I32, "num_accepted_tokens", dev),
        _ptr(spec_token_indx, _I32, "spec_token_indx", dev),
        _ptr(core_attn_out, _BF16, "core_attn_out", dev),
        _turns_ptr(cfg, conv_state, turns, dev)]
    if static:
        rc = _lib.gdn_attention_static(*args, _stream(stream))
    else:
        ws_ptr = _ptr(workspace, None, "workspace", dev)
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        rc = _lib.gdn_attention(*args, ws_ptr, ctypes.c_size_t(ws_bytes), _stream(stream))
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_attention_static" if static else "gdn_attention")


def _rows(kind, query_start_loc, num_tokens, max_row_tokens, cache_indices=None,
          state_indices=None, num_accepted_tokens=None, has_initial_state=None,
          token_indx=None, dev=None) -> GdnRows:
    n = int(query_start_loc.shape[0]) - 1
    if n > 0:
        per_row = int(max_row_tokens) if int(kind) == GDN_ROWS_SPEC else 1
        _need(cache_indices, "cache_indices", at_least=n)
        _need(state_indices, "state_indices", at_least=n * per_row)
        _need(num_accepted_tokens, "num_accepted_tokens", at_least=n)
        _need(has_initial_state, "has_initial_state", at_least=n)
        _need(token_indx, "token_indx", at_least=int(num_tokens))
    return GdnRows(int(kind), n, int(num_tokens), int(max_row_tokens),
                   _ptr(query_start_loc, _I32, "query_start_loc", dev),
                   _ptr(cache_indices, _I32, "cache_indices", dev),
                   _ptr(state_indices, _I32, "state_indices", dev),
                   _ptr(num_accepted_tokens, _I32, "num_accepted_tokens", dev),
                   _ptr(has_initial_state, (torch.uint8, torch.bool), "has_initial_state", dev),
                   _ptr(token_indx, _I32, "token_indx", dev))


def gdn_conv_only(cfg: GdnConfig, mixed_qkv, conv_weight, conv_bias, conv_state,
                  conv_out, kind, query_start_loc, num_tokens, max_row_tokens,
                  cache_indices=None, state_indices=None, num_accepted_tokens=None,
                  has_initial_state=None, token_indx=None, stream=None) -> None:
    dev = mixed_qkv.device
    dims = cfg.dims(conv_state)
    C, nat = cfg.conv_dim, int(mixed_qkv.shape[0])
    if mixed_qkv.dim() != 2 or mixed_qkv.shape[1] != C:
        raise ValueError(f"mixed_qkv must be [num_tokens, {C}], got {list(mixed_qkv.shape)}")
    if conv_state.dim() != 3 or conv_state.shape[2] != C:
        raise ValueError(f"conv_state must be [num_slots, state_len, {C}]")
    _need(conv_weight, "conv_weight", shape=(C, cfg.conv_width))
    _need(conv_bias, "conv_bias", shape=(C,))
    _need(conv_out, "conv_out", at_least=nat * C)
    rows = _rows(kind, query_start_loc, num_tokens, max_row_tokens, cache_indices,
                 state_indices, num_accepted_tokens, has_initial_state, token_indx, dev)
    rc = _lib.gdn_conv_only(ctypes.byref(dims), _ptr(mixed_qkv, _BF16, "mixed_qkv", dev),
                            _ptr(conv_weight, _BF16, "conv_weight", dev),
                            _ptr(conv_bias, _BF16, "conv_bias", dev),
                            _ptr(conv_state, _BF16, "conv_state", dev), int(mixed_qkv.shape[0]),
                            ctypes.byref(rows), _ptr(conv_out, torch.float32, "conv_out", dev),
                            _stream(stream))
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_conv_only")


def gdn_delta_rule_only(cfg: GdnConfig, conv_out, a, b, A_log, dt_bias, ssm_state,
                        core_attn_out, kind, query_start_loc, num_tokens, max_row_tokens,
                        cache_indices=None, state_indices=None, num_accepted_tokens=None,
                        has_initial_state=None, token_indx=None, state_len=None,
                        stream=None) -> None:
    dev = conv_out.device
    dims = cfg.dims(state_len=state_len if state_len is not None else cfg.conv_width - 1,
                    num_slots=int(ssm_state.shape[0]))
    C, Hv, nat = cfg.conv_dim, cfg.num_v_heads, int(conv_out.shape[0])
    if conv_out.dim() != 2 or conv_out.shape[1] != C:
        raise ValueError(f"conv_out must be [num_tokens, {C}], got {list(conv_out.shape)}")
    want = (ssm_state.shape[0], Hv, cfg.head_v_dim, cfg.head_k_dim)
    if tuple(ssm_state.shape) != want:
        raise ValueError(f"ssm_state must be {list(want)}, got {list(ssm_state.shape)}")
    _need(a, "a", at_least=nat * Hv)
    _need(b, "b", at_least=nat * Hv)
    _need(A_log, "A_log", shape=(Hv,))
    _need(dt_bias, "dt_bias", shape=(Hv,))
    _need(core_attn_out, "core_attn_out", at_least=nat * Hv * cfg.head_v_dim)
    rows = _rows(kind, query_start_loc, num_tokens, max_row_tokens, cache_indices,
                 state_indices, num_accepted_tokens, has_initial_state, token_indx, dev)
    rc = _lib.gdn_delta_rule_only(
        ctypes.byref(dims), _ptr(conv_out, torch.float32, "conv_out", dev),
        _ptr(a, _BF16, "a", dev), _ptr(b, _BF16, "b", dev),
        _ptr(A_log, torch.float32, "A_log", dev), _ptr(dt_bias, torch.float32, "dt_bias", dev),
        _ptr(ssm_state, torch.float32, "ssm_state", dev), int(conv_out.shape[0]),
        ctypes.byref(rows), _ptr(core_attn_out, _BF16, "core_attn_out", dev), _stream(stream))
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_delta_rule_only")


def gdn_check_metadata_host(cfg: GdnConfig, state_len: int, num_slots: int,
                            num_actual_tokens: int, *, num_decodes=0, num_prefills=0,
                            num_non_spec_tokens=None, query_start_loc=None,
                            non_spec_state_indices=None, non_spec_token_indx=None,
                            num_spec_decodes=None, num_spec_tokens=None, max_spec_len=None,
                            spec_query_start_loc=None, spec_cache_indices=None,
                            spec_state_indices=None, num_accepted_tokens=None,
                            spec_token_indx=None) -> int:
    """Check metadata values on host (numpy) copies; returns the status and
    raises nothing (``gdn_last_error()`` explains a failure).  Each array is
    passed with its length.  ``num_spec_decodes`` defaults to the length of
    ``spec_query_start_loc`` less one, the token counts to the last entry of
    the query_start_loc arrays, ``max_spec_len`` to the row length of
    ``spec_state_indices`` (a flat array needs it given)."""
    dims = cfg.dims(state_len=state_len, num_slots=num_slots)
    keep = []

    def arr(x):
        if x is None:
            return GdnHostI32(None, 0)
        a = np.ascontiguousarray(x, dtype=np.int32).ravel()
        keep.append(a)
        return GdnHostI32(a.ctypes.data if a.size else None, a.size)

    ns_rows = int(num_decodes) + int(num_prefills)
    if num_spec_decodes is not None:
        Ns = int(num_spec_decodes)
    else:
        Ns = 0 if spec_query_start_loc is None else max(len(spec_query_start_loc) - 1, 0)
    if num_non_spec_tokens is None:
        num_non_spec_tokens = (int(query_start_loc[-1]) if ns_rows and query_start_loc is not None
                               and len(query_start_loc) else 0)
    if num_spec_tokens is None:
        num_spec_tokens = int(spec_query_start_loc[-1]) if Ns else 0
    if max_spec_len is None:
        ssi = None if spec_state_indices is None else np.asarray(spec_state_indices)
        max_spec_len = ssi.shape[1] if ssi is not None and ssi.ndim == 2 else 1
    return int(_lib.gdn_check_metadata_host(
        ctypes.byref(dims), int(num_actual_tokens), int(num_decodes), int(num_prefills),
        int(num_non_spec_tokens), arr(query_start_loc), arr(non_spec_state_indices),
        arr(non_spec_token_indx), int(Ns), int(num_spec_tokens), int(max_spec_len),
        arr(spec_query_start_loc), arr(spec_cache_indices), arr(spec_state_indices),
        arr(num_accepted_tokens), arr(spec_token_indx)))
