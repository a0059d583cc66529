"""Packed variable-length attention oracle — test infrastructure only.

Page "FlashAttention 实战指南：如何把训练内存省 20 倍、速度提 4 倍", section
"上手 FlashAttention 的三步走": batches whose sequences have different lengths
use the varlen interface.  Reading: the packed tensors (total, H, D) hold the
sequences back to back, ``cu_seqlens`` (int32, nseq + 1, starting at 0) gives
their boundaries, and each sequence s is plain attention on the slice
[cu_q[s], cu_q[s+1]) x [cu_k[s], cu_k[s+1]), independent of all others.
LSE is laid out (Hq, total_q).
"""
from __future__ import annotations

import numpy as np

from .attention import attention_fwd, attention_bwd, _f64


def _cu(x):
    return [int(t) for t in (x.tolist() if hasattr(x, "tolist") else x)]


def varlen_fwd(q, k, v, cu_q, cu_k, scale, causal=False, window=(-1, -1), softcap=0.0,
               alibi_slopes=None, seqs=None, dropout=None):
    """Returns (out (total_q, Hq, D), lse (Hq, total_q)) in float64.  With
    ``dropout`` the sequence index plays the batch entry of the mask."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    cq, ck = _cu(cu_q), _cu(cu_k)
    tq, Hq, D = q.shape
    out = np.full((tq, Hq, D), np.nan)
    lse = np.full((Hq, tq), np.nan)
    for s in (range(len(cq) - 1) if seqs is None else seqs):
        a, b2, c, d = cq[s], cq[s + 1], ck[s], ck[s + 1]
        if b2 == a:
            continue
        o, L = attention_fwd(q[None, a:b2], k[None, c:d], v[None, c:d], scale, causal, window,
                             softcap, alibi_slopes, dropout=dropout, batch0=s)
        out[a:b2] = o[0]
        lse[:, a:b2] = L[0]
    return out, lse


def varlen_bwd(q, k, v, dout, cu_q, cu_k, scale, causal=False, window=(-1, -1), softcap=0.0,
               alibi_slopes=None, seqs=None, dropout=None):
    """Returns (dq, dk, dv) packed like the inputs, float64."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(dout)
    cq, ck = _cu(cu_q), _cu(cu_k)
    dq = np.full(q.shape, np.nan)
    dk = np.full(k.shape, np.nan)
    dv = np.full(v.shape, np.nan)
    for s in (range(len(cq) - 1) if seqs is None else seqs):
        a, b2, c, d = cq[s], cq[s + 1], ck[s], ck[s + 1]
        if d > c:
            dk[c:d] = 0.0
            dv[c:d] = 0.0
        if b2 == a:
            continue
        gq, gk, gv = attention_bwd(q[None, a:b2], k[None, c:d], v[None, c:d], do[None, a:b2],
                                   scale, causal, window, softcap, alibi_slopes,
                                   dropout=dropout, batch0=s)
        dq[a:b2], dk[c:d], dv[c:d] = gq[0], gk[0], gv[0]
    return dq, dk, dv
