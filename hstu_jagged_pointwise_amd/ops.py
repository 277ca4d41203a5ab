"""ctypes binding to libhstu.so (C ABI in include/hstu.h).

This layer only marshals arguments. It turns torch tensors into device
pointers, builds the descriptor structs, allocates the workspace with torch
(PyTorch is used for device memory and streams) and raises on a non-OK status.
Every step of the computation runs in libhstu's HIP kernels. There is no
fallback: if the library is missing, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# HSTU_LIB selects another build of the same library (the host-sanitizer build that the
# CPU tests use); by default the in-tree libhstu.so
LIB_PATH = os.environ.get("HSTU_LIB") or os.path.join(_HERE, "libhstu.so")

HSTU_OK, HSTU_INVALID_ARGUMENT, HSTU_UNSUPPORTED, HSTU_WORKSPACE_TOO_SMALL, HSTU_DEVICE_ERROR = range(5)
HSTU_F32, HSTU_BF16 = 0, 1

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -m hstu_jagged_pointwise_amd.build` "
        "(hipcc, gfx950). There is no non-HIP fallback.")
lib = ctypes.CDLL(LIB_PATH)


class hstu_attn_desc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_heads", ctypes.c_int32), ("d_qk", ctypes.c_int32),
                ("d_v", ctypes.c_int32), ("max_seq_len", ctypes.c_int32),
                ("num_pos_buckets", ctypes.c_int32), ("num_time_buckets", ctypes.c_int32),
                ("dtype", ctypes.c_int), ("ln_eps", ctypes.c_float)]


class hstu_layer_desc(ctypes.Structure):
    _fields_ = [("attn", hstu_attn_desc), ("d_model", ctypes.c_int32), ("residual", ctypes.c_int32),
                ("num_layers", ctypes.c_int32)]


class hstu_layer_weights(ctypes.Structure):
    _fields_ = [("w1", ctypes.c_void_p), ("b1", ctypes.c_void_p), ("rab_pos", ctypes.c_void_p),
                ("rab_time", ctypes.c_void_p), ("ln_gamma", ctypes.c_void_p),
                ("ln_beta", ctypes.c_void_p), ("w2", ctypes.c_void_p), ("b2", ctypes.c_void_p)]


class mfalcon_desc(ctypes.Structure):
    _fields_ = [("layer", hstu_layer_desc), ("microbatch", ctypes.c_int32)]


class hstu_layer_grads(ctypes.Structure):
    _fields_ = [("dw1", ctypes.c_void_p), ("db1", ctypes.c_void_p), ("d_rab_pos", ctypes.c_void_p),
                ("d_rab_time", ctypes.c_void_p), ("d_ln_gamma", ctypes.c_void_p),
                ("d_ln_beta", ctypes.c_void_p), ("dw2", ctypes.c_void_p), ("db2", ctypes.c_void_p)]


class hstu_sl_desc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("max_seq_len", ctypes.c_int32),
                ("alpha", ctypes.c_float)]


_P = ctypes.c_void_p
_I64P = ctypes.POINTER(ctypes.c_int64)
_SZP = ctypes.POINTER(ctypes.c_size_t)
_sig = {
    "hstu_version": ([], ctypes.c_int),
    "hstu_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "hstu_last_error": ([], ctypes.c_char_p),
    "hstu_attn_workspace_size": ([ctypes.POINTER(hstu_attn_desc), _I64P, _SZP], ctypes.c_int),
    "hstu_attn_fwd": ([ctypes.POINTER(hstu_attn_desc), _I64P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                       _P, _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "hstu_attn_noalloc_scratch_bytes": ([], ctypes.c_size_t),
    "hstu_attn_fwd_noalloc": ([ctypes.POINTER(hstu_attn_desc), _I64P, _P, _P, _P, _P, _P, _P, _P,
                               _P, _P, _P, _P, _P], ctypes.c_int),
    "hstu_layer_workspace_size": ([ctypes.POINTER(hstu_layer_desc), _I64P, _SZP], ctypes.c_int),
    "hstu_layer_fwd": ([ctypes.POINTER(hstu_layer_desc), _I64P, _P, _P, _P,
                        ctypes.POINTER(hstu_layer_weights), _P, _P, ctypes.c_size_t, _P],
                       ctypes.c_int),
    "mfalcon_workspace_size": ([ctypes.POINTER(mfalcon_desc), _I64P, _I64P, _SZP], ctypes.c_int),
    "mfalcon_score": ([ctypes.POINTER(mfalcon_desc), _I64P, _P, _P, _P, _I64P, _P, _P, _P,
                       ctypes.POINTER(hstu_layer_weights), _P, _P, _P, _P, ctypes.c_size_t, _P],
                      ctypes.c_int),
    "mfalcon_cache_size": ([ctypes.POINTER(mfalcon_desc), _I64P, _SZP], ctypes.c_int),
    "mfalcon_history_workspace_size": ([ctypes.POINTER(mfalcon_desc), _I64P, _SZP], ctypes.c_int),
    "mfalcon_history": ([ctypes.POINTER(mfalcon_desc), _I64P, _P, _P, _P,
                         ctypes.POINTER(hstu_layer_weights), _P, ctypes.c_size_t, _P,
                         ctypes.c_size_t, _P], ctypes.c_int),
    "mfalcon_cached_workspace_size": ([ctypes.POINTER(mfalcon_desc), _I64P, _I64P, _SZP],
                                      ctypes.c_int),
    "mfalcon_score_cached": ([ctypes.POINTER(mfalcon_desc), _I64P, _P, _P, _P, ctypes.c_size_t,
                              _I64P, _P, _P, _P, ctypes.POINTER(hstu_layer_weights), _P, _P, _P,
                              _P, ctypes.c_size_t, _P], ctypes.c_int),
    "hstu_attn_bwd_workspace_size": ([ctypes.POINTER(hstu_attn_desc), _I64P, _SZP], ctypes.c_int),
    "hstu_attn_bwd": ([ctypes.POINTER(hstu_attn_desc), _I64P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                       _P, _P, _P, _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "hstu_layer_bwd_workspace_size": ([ctypes.POINTER(hstu_layer_desc), _I64P, _SZP], ctypes.c_int),
    "hstu_layer_bwd": ([ctypes.POINTER(hstu_layer_desc), _I64P, _P, _P, _P,
                        ctypes.POINTER(hstu_layer_weights), _P, _P, ctypes.POINTER(hstu_layer_grads),
                        _P, ctypes.c_size_t, _P], ctypes.c_int),
    "hstu_softmax_attn_workspace_size": ([ctypes.POINTER(hstu_attn_desc), _I64P, _SZP],
                                         ctypes.c_int),
    "hstu_softmax_attn_fwd": ([ctypes.POINTER(hstu_attn_desc), _I64P, _P, _P, _P, _P, _P, _P, _P, _P,
                               _P, ctypes.c_size_t, _P], ctypes.c_int),
    "hstu_sl_lengths": ([ctypes.POINTER(hstu_sl_desc), _I64P, ctypes.POINTER(ctypes.c_float), _I64P,
                         _I64P], ctypes.c_int),
    "hstu_sl_sample": ([ctypes.c_int32, _I64P, _I64P, _P, _P, _P, _P, _P, ctypes.c_int64, _P, _P,
                        _P, _P], ctypes.c_int),
    "hstu_debug_buckets": ([ctypes.POINTER(hstu_attn_desc), _I64P, _P, _P, ctypes.c_int32, _P, _P,
                            _P], ctypes.c_int),
}
for _name, (_args, _res) in _sig.items():
    _f = getattr(lib, _name)
    _f.argtypes = _args
    _f.restype = _res

EXPORTED = tuple(_sig)


class HstuError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{lib.hstu_status_string(status).decode()}: {message}")
        self.status = status


def _check(status: int):
    if status != HSTU_OK:
        raise HstuError(status, lib.hstu_last_error().decode())


def hstu_version() -> int:
    return lib.hstu_version()


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------
def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libhstu must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _host_offsets(dev: torch.Tensor, host) -> np.ndarray:
    if host is None:
        host = dev.detach().to("cpu")
    if isinstance(host, torch.Tensor):
        host = host.numpy()
    return np.ascontiguousarray(host, dtype=np.int64)


def _i64p(a: np.ndarray):
    return a.ctypes.data_as(_I64P)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return HSTU_F32
    if t.dtype == torch.bfloat16:
        return HSTU_BF16
    raise ValueError(f"unsupported dtype {t.dtype}")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]):
    if workspace is not None:
        return workspace, workspace.numel() * workspace.element_size()
    if nbytes == 0:
        return None, 0
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


def attn_desc(batch, num_heads, d_qk, d_v, max_seq_len, num_pos_buckets, num_time_buckets,
              dtype_code, ln_eps=1e-5) -> hstu_attn_desc:
    return hstu_attn_desc(int(batch), int(num_heads), int(d_qk), int(d_v), int(max_seq_len),
                          int(num_pos_buckets), int(num_time_buckets), int(dtype_code),
                          float(ln_eps))


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------
def hstu_attn_workspace_size(desc: hstu_attn_desc, seq_offsets_host: np.ndarray) -> int:
    n = ctypes.c_size_t(0)
    _check(lib.hstu_attn_workspace_size(ctypes.byref(desc), _i64p(seq_offsets_host), ctypes.byref(n)))
    return n.value


def hstu_attn_fwd(seq_offsets: torch.Tensor, timestamps: Optional[torch.Tensor], q, k, v,
                  rab_pos=None, rab_time=None, *, max_seq_len: int, num_pos_buckets=None,
                  num_time_buckets=None, u=None, ln_gamma=None, ln_beta=None, ln_eps=1e-5,
                  out=None, workspace=None, seq_offsets_host=None, stream=None) -> torch.Tensor:
    """Jagged causal HSTU attention; with u, the gated LayerNorm output. See include/hstu.h."""
    host = _host_offsets(seq_offsets, seq_offsets_host)
    T_tot, H, d_qk = q.shape
    d_v = v.shape[2]
    P = rab_pos.shape[1] if rab_pos is not None else (num_pos_buckets or 1)
    T = rab_time.shape[1] if rab_time is not None else (num_time_buckets or 1)
    desc = attn_desc(len(host) - 1, H, d_qk, d_v, max_seq_len, P, T, _dtype_code(q), ln_eps)
    if out is None:
        out = torch.empty((T_tot, H, d_v), dtype=q.dtype, device=q.device)
    ws, nbytes = _workspace(hstu_attn_workspace_size(desc, host), q.device, workspace)
    _check(lib.hstu_attn_fwd(ctypes.byref(desc), _i64p(host), _ptr(seq_offsets), _ptr(timestamps),
                             _ptr(q), _ptr(k), _ptr(v), _ptr(rab_pos), _ptr(rab_time), _ptr(u),
                             _ptr(ln_gamma), _ptr(ln_beta), _ptr(out), _ptr(ws), nbytes,
                             _stream(stream)))
    return out


def hstu_attn_fwd_noalloc(seq_offsets: torch.Tensor, timestamps: Optional[torch.Tensor], q, k,
                          v, rab_pos=None, rab_time=None, *, max_seq_len: int,
                          num_pos_buckets=None, num_time_buckets=None, u=None, ln_gamma=None,
                          ln_beta=None, ln_eps=1e-5, out=None, seq_offsets_host=None,
                          stream=None) -> torch.Tensor:
    """hstu_attn_fwd with the library's own device scratch instead of a workspace (nothing
    is allocated by the call; `out` may be passed in to allocate nothing here either)."""
    host = _host_offsets(seq_offsets, seq_offsets_host)
    T_tot, H, d_qk = q.shape
    d_v = v.shape[2]
    P = rab_pos.shape[1] if rab_pos is not None else (num_pos_buckets or 1)
    T = rab_time.shape[1] if rab_time is not None else (num_time_buckets or 1)
    desc = attn_desc(len(host) - 1, H, d_qk, d_v, max_seq_len, P, T, _dtype_code(q), ln_eps)
    if out is None:
        out = torch.empty((T_tot, H, d_v), dtype=q.dtype, device=q.device)
    _check(lib.hstu_attn_fwd_noalloc(ctypes.byref(desc), _i64p(host), _ptr(seq_offsets),
                                     _ptr(timestamps), _ptr(q), _ptr(k), _ptr(v), _ptr(rab_pos),
                                     _ptr(rab_time), _ptr(u), _ptr(ln_gamma), _ptr(ln_beta),
                                     _ptr(out), _stream(stream)))
    return out


@dataclass
class LayerWeights:
    """Device tensors of one HSTU layer. w1 [2H(d_v+d_qk), d_model] and
    w2 [d_model, H*d_v] are stored [out, in] in the activation dtype; everything
    else is fp32 or None."""
    w1: torch.Tensor
    w2: torch.Tensor
    b1: Optional[torch.Tensor] = None
    b2: Optional[torch.Tensor] = None
    rab_pos: Optional[torch.Tensor] = None
    rab_time: Optional[torch.Tensor] = None
    ln_gamma: Optional[torch.Tensor] = None
    ln_beta: Optional[torch.Tensor] = None

    def c_struct(self) -> hstu_layer_weights:
        return hstu_layer_weights(_ptr(self.w1), _ptr(self.b1), _ptr(self.rab_pos),
                                  _ptr(self.rab_time), _ptr(self.ln_gamma), _ptr(self.ln_beta),
                                  _ptr(self.w2), _ptr(self.b2))


def _weights_array(layers: Sequence[LayerWeights]):
    arr = (hstu_layer_weights * len(layers))()
    for i, w in enumerate(layers):
        arr[i] = w.c_struct()
    return arr


def layer_desc(layers: Sequence[LayerWeights], batch, num_heads, d_qk, d_v, d_model, max_seq_len,
               dtype_code, ln_eps=1e-5, residual=0, num_pos_buckets=None, num_time_buckets=None):
    w0 = layers[0]
    P = w0.rab_pos.shape[1] if w0.rab_pos is not None else (num_pos_buckets or 1)
    T = w0.rab_time.shape[1] if w0.rab_time is not None else (num_time_buckets or 1)
    a = attn_desc(batch, num_heads, d_qk, d_v, max_seq_len, P, T, dtype_code, ln_eps)
    return hstu_layer_desc(a, int(d_model), int(residual), len(layers))


def hstu_layer_workspace_size(desc: hstu_layer_desc, seq_offsets_host: np.ndarray) -> int:
    n = ctypes.c_size_t(0)
    _check(lib.hstu_layer_workspace_size(ctypes.byref(desc), _i64p(seq_offsets_host), ctypes.byref(n)))
    return n.value


def hstu_layer_fwd(seq_offsets, timestamps, x, layers: Sequence[LayerWeights], *, num_heads, d_qk,
                   d_v, max_seq_len, ln_eps=1e-5, residual=0, out=None, workspace=None,
                   seq_offsets_host=None, stream=None) -> torch.Tensor:
    """A stack of len(layers) HSTU layers over a jagged batch (eqs. 1-3)."""
    host = _host_offsets(seq_offsets, seq_offsets_host)
    desc = layer_desc(layers, len(host) - 1, num_heads, d_qk, d_v, x.shape[1], max_seq_len,
                      _dtype_code(x), ln_eps, residual)
    if out is None:
        out = torch.empty_like(x)
    ws, nbytes = _workspace(hstu_layer_workspace_size(desc, host), x.device, workspace)
    arr = _weights_array(layers)
    _check(lib.hstu_layer_fwd(ctypes.byref(desc), _i64p(host), _ptr(seq_offsets), _ptr(timestamps),
                              _ptr(x), arr, _ptr(out), _ptr(ws), nbytes, _stream(stream)))
    return out


def mfalcon_workspace_size(desc: mfalcon_desc, hist_offsets_host, cand_offsets_host) -> int:
    n = ctypes.c_size_t(0)
    _check(lib.mfalcon_workspace_size(ctypes.byref(desc), _i64p(hist_offsets_host),
                                      _i64p(cand_offsets_host), ctypes.byref(n)))
    return n.value


def mfalcon_score(hist_offsets, hist_ts, hist_x, cand_offsets, cand_ts, cand_x,
                  layers: Sequence[LayerWeights], *, num_heads, d_qk, d_v, max_seq_len, microbatch,
                  w_head=None, ln_eps=1e-5, residual=0, out=None, logit=None, workspace=None,
                  hist_offsets_host=None, cand_offsets_host=None, stream=None):
    """M-FALCON: history once, candidates in microbatches. Returns (cand_out, logits or None)."""
    hh = _host_offsets(hist_offsets, hist_offsets_host)
    ch = _host_offsets(cand_offsets, cand_offsets_host)
    ld = layer_desc(layers, len(hh) - 1, num_heads, d_qk, d_v, cand_x.shape[1], max_seq_len,
                    _dtype_code(cand_x), ln_eps, residual)
    desc = mfalcon_desc(ld, int(microbatch))
    if out is None:
        out = torch.empty_like(cand_x)
    if logit is None and w_head is not None:
        logit = torch.empty(cand_x.shape[0], dtype=torch.float32, device=cand_x.device)
    ws, nbytes = _workspace(mfalcon_workspace_size(desc, hh, ch), cand_x.device, workspace)
    arr = _weights_array(layers)
    _check(lib.mfalcon_score(ctypes.byref(desc), _i64p(hh), _ptr(hist_offsets), _ptr(hist_ts),
                             _ptr(hist_x), _i64p(ch), _ptr(cand_offsets), _ptr(cand_ts),
                             _ptr(cand_x), arr, _ptr(w_head), _ptr(out), _ptr(logit), _ptr(ws),
                             nbytes, _stream(stream)))
    return out, logit


def _mf_desc(layers, n_users, cand_or_hist_x, *, num_heads, d_qk, d_v, max_seq_len, microbatch,
             ln_eps, residual):
    ld = layer_desc(layers, n_users, num_heads, d_qk, d_v, cand_or_hist_x.shape[1], max_seq_len,
                    _dtype_code(cand_or_hist_x), ln_eps, residual)
    return mfalcon_desc(ld, int(microbatch))


def mfalcon_cache_size(desc, hist_offsets_host) -> int:
    n = ctypes.c_size_t(0)
    _check(lib.mfalcon_cache_size(ctypes.byref(desc), _i64p(hist_offsets_host), ctypes.byref(n)))
    return n.value


def mfalcon_cached_workspace_size(desc, hist_offsets_host, cand_offsets_host) -> int:
    n = ctypes.c_size_t(0)
    _check(lib.mfalcon_cached_workspace_size(ctypes.byref(desc), _i64p(hist_offsets_host),
                                             _i64p(cand_offsets_host), ctypes.byref(n)))
    return n.value


def mfalcon_history(hist_offsets, hist_ts, hist_x, layers: Sequence[LayerWeights], *, num_heads,
                    d_qk, d_v, max_seq_len, microbatch=1, ln_eps=1e-5, residual=0, cache=None,
                    workspace=None, hist_offsets_host=None, stream=None):
    """History pass of M-FALCON into a reusable cache (a uint8 device tensor, returned)."""
    hh = _host_offsets(hist_offsets, hist_offsets_host)
    desc = _mf_desc(layers, len(hh) - 1, hist_x, num_heads=num_heads, d_qk=d_qk, d_v=d_v,
                    max_seq_len=max_seq_len, microbatch=microbatch, ln_eps=ln_eps,
                    residual=residual)
    need = mfalcon_cache_size(desc, hh)
    if cache is None:
        cache = torch.empty(max(need, 1), dtype=torch.uint8, device=hist_x.device)
    n = ctypes.c_size_t(0)
    _check(lib.mfalcon_history_workspace_size(ctypes.byref(desc), _i64p(hh), ctypes.byref(n)))
    ws, nbytes = _workspace(n.value, hist_x.device, workspace)
    arr = _weights_array(layers)
    _check(lib.mfalcon_history(ctypes.byref(desc), _i64p(hh), _ptr(hist_offsets), _ptr(hist_ts),
                               _ptr(hist_x), arr, _ptr(cache), cache.numel(), _ptr(ws), nbytes,
                               _stream(stream)))
    return cache


def mfalcon_score_cached(cache, hist_offsets, hist_ts, cand_offsets, cand_ts, cand_x,
                         layers: Sequence[LayerWeights], *, num_heads, d_qk, d_v, max_seq_len,
                         microbatch, w_head=None, ln_eps=1e-5, residual=0, out=None, logit=None,
                         workspace=None, hist_offsets_host=None, cand_offsets_host=None,
                         stream=None):
    """Candidate pass of M-FALCON against a cache from mfalcon_history. Returns (out, logit)."""
    hh = _host_offsets(hist_offsets, hist_offsets_host)
    ch = _host_offsets(cand_offsets, cand_offsets_host)
    desc = _mf_desc(layers, len(hh) - 1, cand_x, num_heads=num_heads, d_qk=d_qk, d_v=d_v,
                    max_seq_len=max_seq_len, microbatch=microbatch, ln_eps=ln_eps,
                    residual=residual)
    if out is None:
        out = torch.empty_like(cand_x)
    if logit is None and w_head is not None:
        logit = torch.empty(cand_x.shape[0], dtype=torch.float32, device=cand_x.device)
    n = ctypes.c_size_t(0)
    _check(lib.mfalcon_cached_workspace_size(ctypes.byref(desc), _i64p(hh), _i64p(ch),
                                             ctypes.byref(n)))
    ws, nbytes = _workspace(n.value, cand_x.device, workspace)
    arr = _weights_array(layers)
    _check(lib.mfalcon_score_cached(ctypes.byref(desc), _i64p(hh), _ptr(hist_offsets),
                                    _ptr(hist_ts), _ptr(cache), cache.numel(), _i64p(ch),
                                    _ptr(cand_offsets), _ptr(cand_ts), _ptr(cand_x), arr,
                                    _ptr(w_head), _ptr(out), _ptr(logit), _ptr(ws), nbytes,
                                    _stream(stream)))
    return out, logit


def hstu_attn_bwd(seq_offsets, timestamps, q, k, v, d_out, rab_pos=None, rab_time=None, *,
                  max_seq_len: int, num_pos_buckets=None, num_time_buckets=None,
                  rab_grads=True, workspace=None, seq_offsets_host=None, stream=None):
    """Gradients of hstu_attn_fwd (no gate). Returns (dq, dk, dv, d_rab_pos, d_rab_time);
    the table gradients are fp32 [H, P] / [H, T], or None when rab_grads is False."""
    host = _host_offsets(seq_offsets, seq_offsets_host)
    T_tot, H, d_qk = q.shape
    d_v = v.shape[2]
    P = rab_pos.shape[1] if rab_pos is not None else (num_pos_buckets or 1)
    T = rab_time.shape[1] if rab_time is not None else (num_time_buckets or 1)
    desc = attn_desc(len(host) - 1, H, d_qk, d_v, max_seq_len, P, T, _dtype_code(q))
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    drp = drt = None
    if rab_grads:
        drp = torch.empty((H, P), dtype=torch.float32, device=q.device)
        drt = torch.empty((H, T), dtype=torch.float32, device=q.device)
    n = ctypes.c_size_t(0)
    _check(lib.hstu_attn_bwd_workspace_size(ctypes.byref(desc), _i64p(host), ctypes.byref(n)))
    ws, nbytes = _workspace(n.value, q.device, workspace)
    _check(lib.hstu_attn_bwd(ctypes.byref(desc), _i64p(host), _ptr(seq_offsets), _ptr(timestamps),
                             _ptr(q), _ptr(k), _ptr(v), _ptr(rab_pos), _ptr(rab_time),
                             _ptr(d_out), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(drp), _ptr(drt),
                             _ptr(ws), nbytes, _stream(stream)))
    return dq, dk, dv, drp, drt


def hstu_attn_bwd_workspace_size(desc: hstu_attn_desc, seq_offsets_host) -> int:
    n = ctypes.c_size_t(0)
    _check(lib.hstu_attn_bwd_workspace_size(ctypes.byref(desc), _i64p(seq_offsets_host),
                                            ctypes.byref(n)))
    return n.value


def hstu_layer_bwd_workspace_size(desc: hstu_layer_desc, seq_offsets_host) -> int:
    n = ctypes.c_size_t(0)
    _check(lib.hstu_layer_bwd_workspace_size(ctypes.byref(desc), _i64p(seq_offsets_host),
                                             ctypes.byref(n)))
    return n.value


_GRAD_FIELDS = ("dw1", "db1", "d_rab_pos", "d_rab_time", "d_ln_gamma", "d_ln_beta", "dw2", "db2")


def hstu_layer_bwd(seq_offsets, timestamps, x, layers: Sequence[LayerWeights], d_y, *, num_heads,
                   d_qk, d_v, max_seq_len, ln_eps=1e-5, residual=0, want_dx=True, workspace=None,
                   seq_offsets_host=None, stream=None):
    """Gradients of hstu_layer_fwd over the stack `layers`. Returns (d_x or None, grads) where
    grads[l] is a dict of fp32 tensors named like the C struct hstu_layer_grads."""
    host = _host_offsets(seq_offsets, seq_offsets_host)
    desc = layer_desc(layers, len(host) - 1, num_heads, d_qk, d_v, x.shape[1], max_seq_len,
                      _dtype_code(x), ln_eps, residual)
    dev_ = x.device
    f1 = 2 * num_heads * (d_v + d_qk)
    hv = num_heads * d_v
    a = desc.attn
    shapes = {"dw1": (f1, x.shape[1]), "db1": (f1,), "d_rab_pos": (num_heads, a.num_pos_buckets),
              "d_rab_time": (num_heads, a.num_time_buckets), "d_ln_gamma": (hv,),
              "d_ln_beta": (hv,), "dw2": (x.shape[1], hv), "db2": (x.shape[1],)}
    grads = [{k: torch.empty(shapes[k], dtype=torch.float32, device=dev_) for k in _GRAD_FIELDS}
             for _ in layers]
    garr = (hstu_layer_grads * len(layers))()
    for i, gd in enumerate(grads):
        garr[i] = hstu_layer_grads(*[_ptr(gd[k]) for k in _GRAD_FIELDS])
    dx = torch.empty_like(x) if want_dx else None
    n = ctypes.c_size_t(0)
    _check(lib.hstu_layer_bwd_workspace_size(ctypes.byref(desc), _i64p(host), ctypes.byref(n)))
    ws, nbytes = _workspace(n.value, dev_, workspace)
    arr = _weights_array(layers)
    _check(lib.hstu_layer_bwd(ctypes.byref(desc), _i64p(host), _ptr(seq_offsets), _ptr(timestamps),
                              _ptr(x), arr, _ptr(d_y), _ptr(dx), garr, _ptr(ws), nbytes,
                              _stream(stream)))
    return dx, grads


def hstu_softmax_attn_fwd(seq_offsets, timestamps, q, k, v, rab_pos=None, rab_time=None, *,
                          max_seq_len: int, num_pos_buckets=None, num_time_buckets=None, out=None,
                          workspace=None, seq_offsets_host=None, stream=None) -> torch.Tensor:
    """Causal softmax attention over the same scores as hstu_attn_fwd (bf16 only)."""
    host = _host_offsets(seq_offsets, seq_offsets_host)
    T_tot, H, d_qk = q.shape
    d_v = v.shape[2]
    P = rab_pos.shape[1] if rab_pos is not None else (num_pos_buckets or 1)
    T = rab_time.shape[1] if rab_time is not None else (num_time_buckets or 1)
    desc = attn_desc(len(host) - 1, H, d_qk, d_v, max_seq_len, P, T, _dtype_code(q))
    if out is None:
        out = torch.empty((T_tot, H, d_v), dtype=q.dtype, device=q.device)
    n = ctypes.c_size_t(0)
    _check(lib.hstu_softmax_attn_workspace_size(ctypes.byref(desc), _i64p(host), ctypes.byref(n)))
    ws, nbytes = _workspace(n.value, q.device, workspace)
    _check(lib.hstu_softmax_attn_fwd(ctypes.byref(desc), _i64p(host), _ptr(seq_offsets),
                                     _ptr(timestamps), _ptr(q), _ptr(k), _ptr(v), _ptr(rab_pos),
                                     _ptr(rab_time), _ptr(out), _ptr(ws), nbytes, _stream(stream)))
    return out


def hstu_sl_lengths(offsets_host, max_seq_len: int, alpha: float, u_keep_host):
    """New offsets after Stochastic Length, on the host: (new_offsets int64 [B+1], L)."""
    off = np.ascontiguousarray(offsets_host, dtype=np.int64)
    u = np.ascontiguousarray(u_keep_host, dtype=np.float32)
    B = len(off) - 1
    if len(u) != B:
        raise ValueError(f"u_keep has {len(u)} entries for {B} sequences")
    desc = hstu_sl_desc(B, int(max_seq_len), float(alpha))
    new = np.zeros(B + 1, np.int64)
    L = ctypes.c_int64(0)
    _check(lib.hstu_sl_lengths(ctypes.byref(desc), _i64p(off),
                               u.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), _i64p(new),
                               ctypes.byref(L)))
    return new, L.value


def hstu_sl_sample(offsets, new_offsets, keys, x=None, timestamps=None, *, offsets_host=None,
                   new_offsets_host=None, stream=None):
    """Kept rows of each sequence on the device. keys: int32 or uint32 device tensor, one
    random 32-bit key per input row (compared as unsigned). Returns (src_index, x[src_index]
    or None, timestamps[src_index] or None)."""
    oh = _host_offsets(offsets, offsets_host)
    nh = _host_offsets(new_offsets, new_offsets_host)
    B = len(oh) - 1
    rows = int(nh[-1]) if B > 0 else 0
    dev = offsets.device
    src = torch.empty(rows, dtype=torch.int64, device=dev)
    out_x = out_ts = None
    row_bytes = 0
    if x is not None:
        out_x = torch.empty((rows,) + tuple(x.shape[1:]), dtype=x.dtype, device=dev)
        row_bytes = x[0].numel() * x.element_size() if x.shape[0] else 0
    if timestamps is not None:
        out_ts = torch.empty(rows, dtype=torch.int64, device=dev)
    if keys is not None and keys.element_size() != 4:
        raise ValueError("keys must be 32-bit")
    _check(lib.hstu_sl_sample(int(B), _i64p(oh), _i64p(nh), _ptr(offsets), _ptr(new_offsets),
                              _ptr(keys), _ptr(src), _ptr(x), int(row_bytes), _ptr(out_x),
                              _ptr(timestamps), _ptr(out_ts), _stream(stream)))
    return src, out_x, out_ts


def hstu_debug_buckets(seq_offsets, timestamps, seq: int, *, max_seq_len, num_pos_buckets,
                       num_time_buckets, num_heads=1, seq_offsets_host=None, stream=None):
    """(pos_bucket, time_bucket) int32 [n, n] for sequence `seq`, from the kernels' bucket code."""
    host = _host_offsets(seq_offsets, seq_offsets_host)
    n = int(host[seq + 1] - host[seq])
    desc = attn_desc(len(host) - 1, num_heads, 32, 32, max_seq_len, num_pos_buckets,
                     num_time_buckets, HSTU_F32)
    pb = torch.empty((n, n), dtype=torch.int32, device=seq_offsets.device)
    tb = torch.empty((n, n), dtype=torch.int32, device=seq_offsets.device)
    _check(lib.hstu_debug_buckets(ctypes.byref(desc), _i64p(host), _ptr(seq_offsets),
                                  _ptr(timestamps), int(seq), _ptr(pb), _ptr(tb), _stream(stream)))
    return pb, tb
