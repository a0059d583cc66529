"""Incremental-decode (KV-cache) oracle — test infrastructure only.

Page "FlashAttention 实战指南：如何把训练内存省 20 倍、速度提 4 倍", section
"增量解码场景flash_attn_with_kvcache": each step appends the new K and V to the
existing cache and attends in place; ``rotary_cos``/``rotary_sin`` apply a
built-in rotary position embedding; ``cache_seqlens`` marks each sample's valid
length; ``block_table`` turns on a paged cache stored in blocks; ``num_splits``
sets how many pieces the keys are split into (a scheduling choice with no
effect on the result, so the oracle has no splits).  Page
"终极指南：如何通过FlashAttention实现Transformer模型的4倍加速与20倍内存优化",
section "推理优化", shows the same call with ``causal=True``.

Readings taken where the pages are silent:

* ``cache_seqlens[b]`` is the length *before* the append; the new tokens go
  to logical positions L_b + t and the library does not change the lengths;
* logical key j of sequence b lives at page ``block_table[b][j // page]``,
  slot ``j % page``; with no block table the cache is (B, capacity, Hkv, D);
* rotary is the half-split form: for i < r/2 the pair (x_i, x_{i+r/2}) turns
  by the angle whose cosine/sine the caller's tables hold at row ``pos``;
  dims >= r are untouched, v is not rotated, cached keys are already rotated;
* the appended key is the rotated k_new rounded once (round-to-nearest-even)
  to the cache dtype; the appended value is v_new unchanged;
* attention then runs over the L_b + Sq_new logical keys with bottom-right
  causal alignment (a single new query sees the whole cache).
"""
from __future__ import annotations

import numpy as np

from .attention import attention_fwd, _f64


def _round_binary(x, p, emin, emax):
    """Round float64 values once to the nearest value of a binary floating
    format with ``p`` significant bits, smallest normal 2^emin and largest
    exponent emax (ties to even, subnormals below 2^emin, overflow to inf);
    returns float64.  Division and multiplication by the power-of-two
    quantum are exact, and ``np.rint`` rounds half to even."""
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    _, e = np.frexp(ax)                     # ax = m * 2^e, 0.5 <= m < 1
    lead = np.maximum(e - 1, emin)          # exponent of the leading bit (subnormals: emin)
    quantum = np.ldexp(1.0, lead - (p - 1))
    with np.errstate(invalid="ignore"):
        y = np.rint(ax / quantum) * quantum
    top = np.ldexp(2.0 - np.ldexp(1.0, 1 - p), emax)  # largest finite value
    y = np.where(y > top, np.inf, y)
    y = np.where(np.isinf(ax), np.inf, y)
    return np.copysign(y, x)


def round_bf16(x):
    """Round float64 values once to the nearest bfloat16 (8 significant bits,
    the exponent range of float32), ties to even; returns float64."""
    return _round_binary(x, 8, -126, 127)


def round_fp16(x):
    """Round float64 values once to the nearest IEEE binary16 (11 significant
    bits, smallest normal 2^-14, largest 65504), ties to even; returns float64."""
    return _round_binary(x, 11, -14, 15)


def rotary_apply(x, cos_row, sin_row, rotary_dim):
    """Half-split rotary on the last axis of x (float64).

    x: (..., D); cos_row, sin_row: (..., rotary_dim // 2) broadcastable."""
    x = np.array(x, dtype=np.float64, copy=True)
    if rotary_dim == 0:
        return x
    h = rotary_dim // 2
    a = x[..., :h].copy()
    b = x[..., h:rotary_dim].copy()
    c = np.asarray(cos_row, dtype=np.float64)
    s = np.asarray(sin_row, dtype=np.float64)
    x[..., :h] = a * c - b * s
    x[..., h:rotary_dim] = b * c + a * s
    return x


def gather_logical_cache(cache, b, L, block_table=None, page_size=None):
    """Rows 0..L-1 of sequence b's logical cache, shape (L, Hkv, D) float64.
    Rows are gathered first and converted afterwards, so only live rows are
    ever widened to float64."""
    if block_table is None:
        return _f64(cache[b, :L])
    bt = np.asarray(block_table.cpu().numpy() if hasattr(block_table, "cpu") else block_table)
    j = np.arange(L)
    pages = bt[b, j // page_size]
    assert (pages >= 0).all(), "block_table entry missing for a live position"
    if hasattr(cache, "detach"):
        import torch
        return _f64(cache[torch.from_numpy(pages).long(), torch.from_numpy(j % page_size).long()])
    return _f64(np.asarray(cache)[pages, j % page_size])


def kvcache_fwd(q, k_new, v_new, k_cache, v_cache, cache_seqlens, block_table=None,
                page_size=None, rotary_cos=None, rotary_sin=None, rotary_dim=0, scale=1.0,
                causal=True, window=(-1, -1), softcap=0.0, alibi_slopes=None,
                cache_dtype="bf16", heads=None):
    """Decode attention with in-place append.

    q (B, Sq_new, Hq, D); k_new/v_new (B, Sq_new, Hkv, D) or None.
    Returns dict with ``out`` (B, Sq_new, Hq, D), ``lse`` (B, Hq, Sq_new),
    ``k_app``/``v_app`` (B, Sq_new, Hkv, D): the values the append writes
    (already rounded to the cache dtype), and ``slots``: list of
    (b, t, physical_index) where they land (physical_index is (page, slot) or
    (b, position) for a contiguous cache)."""
    qd = _f64(q)
    B, Sq, Hq, D = qd.shape
    Ls = [int(x) for x in (cache_seqlens.tolist() if hasattr(cache_seqlens, "tolist") else cache_seqlens)]
    rnd = round_bf16 if cache_dtype == "bf16" else round_fp16
    cos = None if rotary_cos is None else _f64(rotary_cos)
    sin = None if rotary_sin is None else _f64(rotary_sin)
    Hkv = k_cache.shape[2]
    out = np.zeros((B, Sq, Hq, D))
    lse = np.zeros((B, Hq, Sq))
    k_app = np.zeros((B, Sq, Hkv, D))
    v_app = np.zeros((B, Sq, Hkv, D))
    slots = []
    bt = None
    if block_table is not None:
        bt = np.asarray(block_table.cpu().numpy() if hasattr(block_table, "cpu") else block_table)
    for b in range(B):
        L = Ls[b]
        pos = L + np.arange(Sq)
        qb = qd[b]
        if k_new is not None:
            kb = _f64(k_new)[b]
            vb = _f64(v_new)[b]
        if rotary_dim and cos is not None:
            cr = cos[pos][:, None, :]
            sr = sin[pos][:, None, :]
            qb = rotary_apply(qb, cr, sr, rotary_dim)
            if k_new is not None:
                kb = rotary_apply(kb, cr, sr, rotary_dim)
        Kc = gather_logical_cache(k_cache, b, L, bt, page_size)
        Vc = gather_logical_cache(v_cache, b, L, bt, page_size)
        if k_new is not None:
            ka, va = rnd(kb), vb.copy()
            k_app[b], v_app[b] = ka, va
            Kc = np.concatenate([Kc, ka], axis=0)
            Vc = np.concatenate([Vc, va], axis=0)
            for t in range(Sq):
                p = L + t
                phys = (int(bt[b, p // page_size]), p % page_size) if bt is not None else (b, p)
                slots.append((b, t, phys))
        o, l = attention_fwd(qb[None], Kc[None], Vc[None], scale, causal, window, softcap,
                             alibi_slopes, heads=heads)
        out[b], lse[b] = o[0], l[0]
    return {"out": out, "lse": lse, "k_app": k_app, "v_app": v_app, "slots": slots}
