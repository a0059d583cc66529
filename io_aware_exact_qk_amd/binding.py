"""Thin ctypes binding of libfa.so.

Argument marshalling only: tensors are checked for device, dtype, layout and
shape, outputs are allocated with torch when the caller passes none, and the
raw device pointers plus the current HIP stream go to the C entry points of
the same names.  Every step of the computation runs in the library's HIP
kernels; if the library is missing the import of this module's functions
fails loudly — there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")
_lib = None

FA_DTYPE = {torch.float16: 0, torch.bfloat16: 1}
KERNEL_KINDS = ("fwd", "bwd_preprocess", "bwd_dkdv", "bwd_dq", "decode_split", "decode_combine")

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_Z = ctypes.c_size_t


class FAError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {lib().fa_status_string(status).decode()} (status {status})")


def lib():
    """Load libfa.so once (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                           "`python -m io_aware_exact_qk_amd.build` (or __graft_entry__.build())")
    L = ctypes.CDLL(_LIB_PATH)
    L.fa_status_string.restype = ctypes.c_char_p
    L.fa_status_string.argtypes = [_I]
    L.fa_kernel_name.restype = ctypes.c_char_p
    L.fa_kernel_name.argtypes = [_I]
    L.fa_fwd.restype = _I
    L.fa_fwd.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _I, _I, _F, _P, _P]
    L.fa_bwd.restype = _I
    L.fa_bwd.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _I,
                         _I, _F, _P, _I, _P, _Z, _P]
    L.fa_bwd_workspace_size.restype = _Z
    L.fa_bwd_workspace_size.argtypes = [_I] * 7
    L.fa_fwd_varlen.restype = _I
    L.fa_fwd_varlen.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _F, _I,
                                _I, _I, _F, _P, _P, _Z, _P]
    L.fa_fwd_varlen_workspace_size.restype = _Z
    L.fa_fwd_varlen_workspace_size.argtypes = [_I] * 4
    L.fa_bwd_varlen.restype = _I
    L.fa_bwd_varlen.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I,
                                _I, _I, _F, _I, _I, _I, _F, _P, _I, _P, _Z, _P]
    L.fa_bwd_varlen_workspace_size.restype = _Z
    L.fa_bwd_varlen_workspace_size.argtypes = [_I] * 6
    # dropout variants: the plain argument list with (p, seed, offset) in
    # front of the stream (forward) or of `deterministic` (backward)
    _D = [_F, ctypes.c_ulonglong, ctypes.c_ulonglong]
    L.fa_fwd_dropout.restype = _I
    L.fa_fwd_dropout.argtypes = L.fa_fwd.argtypes[:-1] + _D + [_P]
    L.fa_bwd_dropout.restype = _I
    L.fa_bwd_dropout.argtypes = L.fa_bwd.argtypes[:22] + _D + L.fa_bwd.argtypes[22:]
    L.fa_fwd_varlen_dropout.restype = _I
    L.fa_fwd_varlen_dropout.argtypes = L.fa_fwd_varlen.argtypes[:-3] + _D + [_P, _Z, _P]
    L.fa_fwd_qkvpacked.restype = _I
    L.fa_fwd_qkvpacked.argtypes = [_P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I, _I, _F, _P, _P]
    L.fa_bwd_qkvpacked.restype = _I
    L.fa_bwd_qkvpacked.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I, _I, _F, _P, _I,
                                   _P, _Z, _P]
    L.fa_fwd_kvpacked.restype = _I
    L.fa_fwd_kvpacked.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _I, _I, _F, _P, _P]
    L.fa_bwd_kvpacked.restype = _I
    L.fa_bwd_kvpacked.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _I, _I,
                                  _F, _P, _I, _P, _Z, _P]
    L.fa_fwd_fp8.restype = _I
    L.fa_fwd_fp8.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _I, _F, _P, _P, _P, _P,
                             _P, _Z, _P]
    L.fa_fwd_fp8_workspace_size.restype = _Z
    L.fa_fwd_fp8_workspace_size.argtypes = [_I] * 4
    L.fa_bwd_varlen_dropout.restype = _I
    L.fa_bwd_varlen_dropout.argtypes = L.fa_bwd_varlen.argtypes[:26] + _D + L.fa_bwd_varlen.argtypes[26:]
    L.fa_fwd_kvcache.restype = _I
    L.fa_fwd_kvcache.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _I, _P, _P, _I, _P, _P, _I, _I, _I, _I,
                                 _I, _I, _F, _I, _I, _I, _F, _P, _I, _P, _Z, _P]
    L.fa_kvcache_workspace_size.restype = _Z
    L.fa_kvcache_workspace_size.argtypes = [_I] * 5
    # the same arguments without (workspace, workspace_bytes)
    L.fa_fwd_kvcache_noalloc.restype = _I
    L.fa_fwd_kvcache_noalloc.argtypes = L.fa_fwd_kvcache.argtypes[:27] + [_P]
    L.fa_kvcache_noalloc_max_bytes.restype = _Z
    L.fa_kvcache_noalloc_max_bytes.argtypes = []
    L.fa_profiler_enable.restype = _I
    L.fa_profiler_enable.argtypes = [_I, _I]
    L.fa_profiler_reset.restype = _I
    L.fa_profiler_read.restype = _I
    L.fa_profiler_read.argtypes = [_I, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_long)]
    _lib = L
    return L


# ------------------------------------------------------------------ utils --
def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(t, name, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    return t


def _dt(q):
    if q.dtype not in FA_DTYPE:
        raise ValueError(f"dtype {q.dtype} not supported (float16 / bfloat16)")
    return FA_DTYPE[q.dtype]


def _raise(fn, st):
    if st != 0:
        raise FAError(fn, st)


def _drop(dropout_p, seed, offset):
    """(p, seed, offset) as the dropout entry points take them."""
    return [float(dropout_p), int(seed) & (2 ** 64 - 1), int(offset) & (2 ** 64 - 1)]


def _opts(D, scale, window, softcap, alibi_slopes):
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    wl, wr = (int(window[0]), int(window[1]))
    if alibi_slopes is not None:
        _check(alibi_slopes, "alibi_slopes", torch.float32, 1)
    return scale, wl, wr, float(softcap)


# -------------------------------------------------------------- forward ----
def fa_fwd(q, k, v, out=None, lse=None, scale=None, causal=False, window=(-1, -1), softcap=0.0,
           alibi_slopes=None, stream=None, _dropout=None):
    """q (B,Sq,Hq,D), k/v (B,Sk,Hkv,D) -> (out (B,Sq,Hq,D), lse (B,Hq,Sq) float32)."""
    _check(q, "q", ndim=4)
    _check(k, "k", q.dtype, 4)
    _check(v, "v", q.dtype, 4)
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    if k.shape != (B, Sk, Hkv, D) or v.shape != k.shape:
        raise ValueError("k/v shape mismatch")
    out = torch.empty_like(q) if out is None else _check(out, "out", q.dtype)
    lse = torch.empty(B, Hq, Sq, device=q.device, dtype=torch.float32) if lse is None else _check(lse, "lse", torch.float32)
    scale, wl, wr, sc = _opts(D, scale, window, softcap, alibi_slopes)
    args = [_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Sq, Sk, Hq, Hkv, D, _dt(q),
            scale, int(bool(causal)), wl, wr, sc, _ptr(alibi_slopes)]
    if _dropout is None:
        _raise("fa_fwd", lib().fa_fwd(*args, _stream(stream)))
    else:
        _raise("fa_fwd_dropout", lib().fa_fwd_dropout(*args, *_dropout, _stream(stream)))
    return out, lse


def fa_fwd_dropout(q, k, v, dropout_p, seed, offset=0, **kw):
    """fa_fwd with dropout on the attention weights (probability dropout_p,
    Philox4x32-10 keyed by seed, counter word 3 = offset)."""
    return fa_fwd(q, k, v, _dropout=_drop(dropout_p, seed, offset), **kw)


def fa_bwd(q, k, v, out, dout, lse, dq=None, dk=None, dv=None, scale=None, causal=False,
           window=(-1, -1), softcap=0.0, alibi_slopes=None, deterministic=False, workspace=None,
           stream=None, _dropout=None):
    """Gradients (dq, dk, dv) of attention given the forward's out and lse."""
    for n, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
        _check(t, n, q.dtype, 4)
    _check(lse, "lse", torch.float32, 3)
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    dq = torch.empty_like(q) if dq is None else _check(dq, "dq", q.dtype)
    dk = torch.empty_like(k) if dk is None else _check(dk, "dk", q.dtype)
    dv = torch.empty_like(v) if dv is None else _check(dv, "dv", q.dtype)
    L = lib()
    ws_bytes = L.fa_bwd_workspace_size(B, Sq, Sk, Hq, Hkv, D, int(bool(deterministic)))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), device=q.device, dtype=torch.uint8)
    scale, wl, wr, sc = _opts(D, scale, window, softcap, alibi_slopes)
    head = [_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
            _ptr(dv), B, Sq, Sk, Hq, Hkv, D, _dt(q), scale, int(bool(causal)), wl, wr, sc,
            _ptr(alibi_slopes)]
    tail = [int(bool(deterministic)), _ptr(workspace), workspace.numel() * workspace.element_size(),
            _stream(stream)]
    if _dropout is None:
        _raise("fa_bwd", L.fa_bwd(*head, *tail))
    else:
        _raise("fa_bwd_dropout", L.fa_bwd_dropout(*head, *_dropout, *tail))
    return dq, dk, dv


def fa_bwd_dropout(q, k, v, out, dout, lse, dropout_p, seed, offset=0, **kw):
    """fa_bwd of fa_fwd_dropout: the same dropout_p, seed and offset."""
    return fa_bwd(q, k, v, out, dout, lse, _dropout=_drop(dropout_p, seed, offset), **kw)


# --------------------------------------------------------------- packed ----
def fa_fwd_qkvpacked(qkv, out=None, lse=None, scale=None, causal=False, window=(-1, -1), softcap=0.0,
                     alibi_slopes=None, stream=None):
    """qkv (B,S,3,H,D) -> (out (B,S,H,D), lse (B,H,S) float32)."""
    _check(qkv, "qkv", ndim=5)
    B, S, three, H, D = qkv.shape
    if three != 3:
        raise ValueError("qkv must be (B, S, 3, H, D)")
    out = torch.empty(B, S, H, D, device=qkv.device, dtype=qkv.dtype) if out is None else _check(out, "out", qkv.dtype)
    lse = torch.empty(B, H, S, device=qkv.device, dtype=torch.float32) if lse is None else _check(lse, "lse", torch.float32)
    scale, wl, wr, sc = _opts(D, scale, window, softcap, alibi_slopes)
    st = lib().fa_fwd_qkvpacked(_ptr(qkv), _ptr(out), _ptr(lse), B, S, H, D, _dt(qkv), scale,
                                int(bool(causal)), wl, wr, sc, _ptr(alibi_slopes), _stream(stream))
    _raise("fa_fwd_qkvpacked", st)
    return out, lse


def fa_bwd_qkvpacked(qkv, out, dout, lse, dqkv=None, scale=None, causal=False, window=(-1, -1),
                     softcap=0.0, alibi_slopes=None, deterministic=False, workspace=None, stream=None):
    """Gradient dqkv (B,S,3,H,D) of fa_fwd_qkvpacked."""
    _check(qkv, "qkv", ndim=5)
    B, S, _, H, D = qkv.shape
    _check(out, "out", qkv.dtype, 4)
    _check(dout, "dout", qkv.dtype, 4)
    _check(lse, "lse", torch.float32, 3)
    dqkv = torch.empty_like(qkv) if dqkv is None else _check(dqkv, "dqkv", qkv.dtype)
    L = lib()
    ws_bytes = L.fa_bwd_workspace_size(B, S, S, H, H, D, int(bool(deterministic)))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), device=qkv.device, dtype=torch.uint8)
    scale, wl, wr, sc = _opts(D, scale, window, softcap, alibi_slopes)
    st = L.fa_bwd_qkvpacked(_ptr(qkv), _ptr(out), _ptr(dout), _ptr(lse), _ptr(dqkv), B, S, H, D, _dt(qkv),
                            scale, int(bool(causal)), wl, wr, sc, _ptr(alibi_slopes), int(bool(deterministic)),
                            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    _raise("fa_bwd_qkvpacked", st)
    return dqkv


def fa_fwd_kvpacked(q, kv, out=None, lse=None, scale=None, causal=False, window=(-1, -1), softcap=0.0,
                    alibi_slopes=None, stream=None):
    """q (B,Sq,Hq,D), kv (B,Sk,2,Hkv,D) -> (out, lse)."""
    _check(q, "q", ndim=4)
    _check(kv, "kv", q.dtype, 5)
    B, Sq, Hq, D = q.shape
    Sk, two, Hkv = kv.shape[1], kv.shape[2], kv.shape[3]
    if two != 2 or kv.shape[4] != D or kv.shape[0] != B:
        raise ValueError("kv must be (B, Sk, 2, Hkv, D)")
    out = torch.empty_like(q) if out is None else _check(out, "out", q.dtype)
    lse = torch.empty(B, Hq, Sq, device=q.device, dtype=torch.float32) if lse is None else _check(lse, "lse", torch.float32)
    scale, wl, wr, sc = _opts(D, scale, window, softcap, alibi_slopes)
    st = lib().fa_fwd_kvpacked(_ptr(q), _ptr(kv), _ptr(out), _ptr(lse), B, Sq, Sk, Hq, Hkv, D, _dt(q), scale,
                               int(bool(causal)), wl, wr, sc, _ptr(alibi_slopes), _stream(stream))
    _raise("fa_fwd_kvpacked", st)
    return out, lse


def fa_bwd_kvpacked(q, kv, out, dout, lse, dq=None, dkv=None, scale=None, causal=False, window=(-1, -1),
                    softcap=0.0, alibi_slopes=None, deterministic=False, workspace=None, stream=None):
    """Gradients (dq, dkv (B,Sk,2,Hkv,D)) of fa_fwd_kvpacked."""
    _check(q, "q", ndim=4)
    _check(kv, "kv", q.dtype, 5)
    for n, t in (("out", out), ("dout", dout)):
        _check(t, n, q.dtype, 4)
    _check(lse, "lse", torch.float32, 3)
    B, Sq, Hq, D = q.shape
    Sk, Hkv = kv.shape[1], kv.shape[3]
    dq = torch.empty_like(q) if dq is None else _check(dq, "dq", q.dtype)
    dkv = torch.empty_like(kv) if dkv is None else _check(dkv, "dkv", q.dtype)
    L = lib()
    ws_bytes = L.fa_bwd_workspace_size(B, Sq, Sk, Hq, Hkv, D, int(bool(deterministic)))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), device=q.device, dtype=torch.uint8)
    scale, wl, wr, sc = _opts(D, scale, window, softcap, alibi_slopes)
    st = L.fa_bwd_kvpacked(_ptr(q), _ptr(kv), _ptr(out), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dkv), B, Sq,
                           Sk, Hq, Hkv, D, _dt(q), scale, int(bool(causal)), wl, wr, sc, _ptr(alibi_slopes),
                           int(bool(deterministic)), _ptr(workspace),
                           workspace.numel() * workspace.element_size(), _stream(stream))
    _raise("fa_bwd_kvpacked", st)
    return dq, dkv


# ------------------------------------------------------------------ fp8 ----
def fa_fwd_fp8(q, k, v, descale_q=None, descale_k=None, descale_v=None, out=None, lse=None, scale=None,
               causal=False, window=(-1, -1), softcap=0.0, alibi_slopes=None, workspace=None, stream=None):
    """fp8 (torch.float8_e4m3fn) q (B,Sq,Hq,D), k/v (B,Sk,Hkv,D) with float32
    dequantisation factors (B, Hkv) each (None = 1) -> (out bf16, lse)."""
    f8 = torch.float8_e4m3fn
    _check(q, "q", f8, 4)
    _check(k, "k", f8, 4)
    _check(v, "v", f8, 4)
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    for n, d in (("descale_q", descale_q), ("descale_k", descale_k), ("descale_v", descale_v)):
        if d is not None:
            _check(d, n, torch.float32, 2)
            if tuple(d.shape) != (B, Hkv):
                raise ValueError(f"{n} must be (B, Hkv)")
    out = torch.empty(B, Sq, Hq, D, device=q.device, dtype=torch.bfloat16) if out is None else _check(out, "out", torch.bfloat16)
    lse = torch.empty(B, Hq, Sq, device=q.device, dtype=torch.float32) if lse is None else _check(lse, "lse", torch.float32)
    L = lib()
    ws_bytes = L.fa_fwd_fp8_workspace_size(B, Sk, Hkv, D)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), device=q.device, dtype=torch.uint8)
    scale, wl, wr, sc = _opts(D, scale, window, softcap, alibi_slopes)
    st = L.fa_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Sq, Sk, Hq, Hkv, D, scale,
                      int(bool(causal)), wl, wr, sc, _ptr(alibi_slopes), _ptr(descale_q), _ptr(descale_k),
                      _ptr(descale_v), _ptr(workspace), workspace.numel() * workspace.element_size(),
                      _stream(stream))
    _raise("fa_fwd_fp8", st)
    return out, lse


# --------------------------------------------------------------- varlen ----
def fa_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, out=None,
                  lse=None, scale=None, causal=False, window=(-1, -1), softcap=0.0,
                  alibi_slopes=None, workspace=None, stream=None, _dropout=None):
    """Packed q (total_q,Hq,D), k/v (total_k,Hkv,D) -> (out, lse (Hq,total_q))."""
    _check(q, "q", ndim=3)
    _check(k, "k", q.dtype, 3)
    _check(v, "v", q.dtype, 3)
    _check(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1)
    _check(cu_seqlens_k, "cu_seqlens_k", torch.int32, 1)
    tq, Hq, D = q.shape
    tk, Hkv = k.shape[0], k.shape[1]
    nseq = cu_seqlens_q.numel() - 1
    if cu_seqlens_k.numel() != nseq + 1:
        raise ValueError("cu_seqlens_q/k sizes differ")
    out = torch.empty_like(q) if out is None else _check(out, "out", q.dtype)
    lse = torch.empty(Hq, tq, device=q.device, dtype=torch.float32) if lse is None else _check(lse, "lse", torch.float32)
    scale, wl, wr, sc = _opts(D, scale, window, softcap, alibi_slopes)
    ws_bytes = lib().fa_fwd_varlen_workspace_size(nseq, tq, Hq, D)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), device=q.device, dtype=torch.uint8)
    args = [_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens_q),
            _ptr(cu_seqlens_k), nseq, int(max_seqlen_q), int(max_seqlen_k), tq, tk,
            Hq, Hkv, D, _dt(q), scale, int(bool(causal)), wl, wr, sc, _ptr(alibi_slopes)]
    ws = [_ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)]
    if _dropout is None:
        _raise("fa_fwd_varlen", lib().fa_fwd_varlen(*args, *ws))
    else:
        _raise("fa_fwd_varlen_dropout", lib().fa_fwd_varlen_dropout(*args, *_dropout, *ws))
    return out, lse


def fa_fwd_varlen_dropout(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                          dropout_p, seed, offset=0, **kw):
    """fa_fwd_varlen with dropout; sequence s plays the mask's batch entry."""
    return fa_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                         _dropout=_drop(dropout_p, seed, offset), **kw)


def fa_bwd_varlen(q, k, v, out, dout, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                  dq=None, dk=None, dv=None, scale=None, causal=False, window=(-1, -1), softcap=0.0,
                  alibi_slopes=None, deterministic=False, workspace=None, stream=None, _dropout=None):
    for n, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
        _check(t, n, q.dtype, 3)
    _check(lse, "lse", torch.float32, 2)
    tq, Hq, D = q.shape
    tk, Hkv = k.shape[0], k.shape[1]
    nseq = cu_seqlens_q.numel() - 1
    dq = torch.empty_like(q) if dq is None else _check(dq, "dq", q.dtype)
    dk = torch.zeros_like(k) if dk is None else _check(dk, "dk", q.dtype)
    dv = torch.zeros_like(v) if dv is None else _check(dv, "dv", q.dtype)
    L = lib()
    ws_bytes = L.fa_bwd_varlen_workspace_size(nseq, tq, tk, Hq, D, int(bool(deterministic)))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), device=q.device, dtype=torch.uint8)
    scale, wl, wr, sc = _opts(D, scale, window, softcap, alibi_slopes)
    head = [_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(dq),
            _ptr(dk), _ptr(dv), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), nseq,
            int(max_seqlen_q), int(max_seqlen_k), tq, tk, Hq, Hkv, D, _dt(q), scale,
            int(bool(causal)), wl, wr, sc, _ptr(alibi_slopes)]
    tail = [int(bool(deterministic)), _ptr(workspace), workspace.numel() * workspace.element_size(),
            _stream(stream)]
    if _dropout is None:
        _raise("fa_bwd_varlen", L.fa_bwd_varlen(*head, *tail))
    else:
        _raise("fa_bwd_varlen_dropout", L.fa_bwd_varlen_dropout(*head, *_dropout, *tail))
    return dq, dk, dv


def fa_bwd_varlen_dropout(q, k, v, out, dout, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                          max_seqlen_k, dropout_p, seed, offset=0, **kw):
    """fa_bwd_varlen of fa_fwd_varlen_dropout (same dropout_p, seed, offset)."""
    return fa_bwd_varlen(q, k, v, out, dout, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                         max_seqlen_k, _dropout=_drop(dropout_p, seed, offset), **kw)


# -------------------------------------------------------------- kvcache ----
def fa_fwd_kvcache(q, k_cache, v_cache, cache_seqlens, k_new=None, v_new=None, block_table=None,
                   rotary_cos=None, rotary_sin=None, rotary_dim=None, num_splits=1, out=None,
                   lse=None, scale=None, causal=True, window=(-1, -1), softcap=0.0,
                   alibi_slopes=None, workspace=None, stream=None, _noalloc=False):
    """Decode step: appends k_new/v_new in place, returns (out (B,Sq,Hq,D), lse (B,Hq,Sq))."""
    _check(q, "q", ndim=4)
    _check(k_cache, "k_cache", q.dtype, 4)
    _check(v_cache, "v_cache", q.dtype, 4)
    _check(cache_seqlens, "cache_seqlens", torch.int32, 1)
    B, Sq, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    if (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new go together")
    if k_new is not None:
        _check(k_new, "k_new", q.dtype, 4)
        _check(v_new, "v_new", q.dtype, 4)
    if block_table is not None:
        _check(block_table, "block_table", torch.int32, 2)
        page, max_blocks = k_cache.shape[1], block_table.shape[1]
    else:
        page = 64 if k_cache.shape[1] % 64 == 0 else k_cache.shape[1]
        max_blocks = k_cache.shape[1] // page
    if rotary_cos is not None:
        _check(rotary_cos, "rotary_cos", torch.float32, 2)
        _check(rotary_sin, "rotary_sin", torch.float32, 2)
        rd = 2 * rotary_cos.shape[1] if rotary_dim is None else int(rotary_dim)
    else:
        rd = 0
    out = torch.empty_like(q) if out is None else _check(out, "out", q.dtype)
    lse = torch.empty(B, Hq, Sq, device=q.device, dtype=torch.float32) if lse is None else _check(lse, "lse", torch.float32)
    L = lib()
    scale, wl, wr, sc = _opts(D, scale, window, softcap, alibi_slopes)
    args = [_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(cache_seqlens),
            _ptr(block_table), max_blocks, page, _ptr(rotary_cos), _ptr(rotary_sin), rd, _ptr(out), _ptr(lse),
            B, Sq, Hq, Hkv, D, _dt(q), scale, int(bool(causal)), wl, wr, sc, _ptr(alibi_slopes),
            int(num_splits)]
    if _noalloc:
        _raise("fa_fwd_kvcache_noalloc", L.fa_fwd_kvcache_noalloc(*args, _stream(stream)))
        return out, lse
    ws_bytes = L.fa_kvcache_workspace_size(B, Sq, Hq, D, int(num_splits))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), device=q.device, dtype=torch.uint8)
    st = L.fa_fwd_kvcache(*args, _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    _raise("fa_fwd_kvcache", st)
    return out, lse


def fa_fwd_kvcache_noalloc(*args, **kw):
    """fa_fwd_kvcache (same arguments, no workspace) through the entry point
    without a workspace: the library's static per-GPU scratch holds the split
    partials.  Pass `out` and `lse` to keep the call free of any allocation."""
    if "workspace" in kw:
        raise TypeError("fa_fwd_kvcache_noalloc takes no workspace")
    return fa_fwd_kvcache(*args, _noalloc=True, **kw)


# ------------------------------------------------------------- profiler ----
def profiler_enable(capacity=4096):
    _raise("fa_profiler_enable", lib().fa_profiler_enable(1, int(capacity)))


def profiler_disable():
    _raise("fa_profiler_enable", lib().fa_profiler_enable(0, 0))


def profiler_reset():
    _raise("fa_profiler_reset", lib().fa_profiler_reset())


def profiler_read():
    """{kernel name: (total_ms, launches)} since the last reset (synchronises)."""
    res = {}
    for i, name in enumerate(KERNEL_KINDS):
        ms, n = ctypes.c_double(0), ctypes.c_long(0)
        _raise("fa_profiler_read", lib().fa_profiler_read(i, ctypes.byref(ms), ctypes.byref(n)))
        res[name] = (ms.value, n.value)
    return res
