"""Dense attention oracle (float64 numpy) — test infrastructure only.

Sources (titles and sections of the pages this follows):

* Page "FlashAttention 实战指南：如何把训练内存省 20 倍、速度提 4 倍":
  - section "长序列注意力为什么会爆内存": standard attention is QK^T, a
    softmax, then a product with V, with an n x n matrix in between;
  - section "进阶参数如何配置causal、window_size 与 MQA/GQA": the options
    ``window_size=(left, right)`` (-1 means unbounded), ``alibi_slopes``
    (a position bias that decays scores of distant keys), ``softcap``
    (logits capped to [-softcap, softcap]), and MQA/GQA (fewer K/V heads than
    Q heads, Q heads an integer multiple of K/V heads);
  - section "上手 FlashAttention 的三步走": inputs are laid out
    (batch, seqlen, nheads, headdim); autoregressive training passes causal.
* Page "终极指南：如何通过FlashAttention实现Transformer模型的4倍加速与20倍内存优化",
  section "精确性与效率的平衡": the result is exact, not an approximation.

Readings taken where the pages are silent (each is listed with its reason in
the design notes of this repository):

* causal alignment is bottom-right: query row i may see key j <= i + Sk - Sq;
* window bounds are inclusive: keys in [i' - left, i' + right] with
  i' = i + Sk - Sq, and causal forces right = 0;
* softcap is the smooth cap  c * tanh(s / c)  applied to the scaled logit s;
  0 disables it;
* order of the score transform: scale -> softcap -> ALiBi -> mask;
* ALiBi adds  -slope[h] * |i' - j|  with one float32 slope per query head;
* LSE is the natural-log log-sum-exp of the final logits z over allowed keys;
* a query row with no allowed key returns O = 0 and LSE = +inf;
* GQA maps query head h to K/V head  h // (Hq // Hkv).
"""
from __future__ import annotations

import numpy as np

from .dropout import keep_mask, keep_scale

ROW_CHUNK = 1024  # query rows materialised at once (full rows, no tiling of keys)


def _f64(x):
    """Exact conversion of a 16/32-bit tensor or array to float64 numpy."""
    if hasattr(x, "detach"):
        x = x.detach().cpu().float().numpy()
    return np.asarray(x, dtype=np.float64)


def allowed_mask(rows, Sq, Sk, causal=False, window=(-1, -1)):
    """Boolean (len(rows), Sk) mask of the keys each query row may attend.

    Follows the ``window_size`` / ``causal`` options of the section
    "进阶参数如何配置causal、window_size 与 MQA/GQA" (page "FlashAttention 实战指南…")
    with the bottom-right alignment and inclusive bounds read above."""
    rows = np.asarray(rows, dtype=np.int64)
    left, right = int(window[0]), int(window[1])
    if causal:
        right = 0
    ip = rows[:, None] + (Sk - Sq)           # aligned query position i'
    j = np.arange(Sk, dtype=np.int64)[None, :]
    ok = np.ones((len(rows), Sk), dtype=bool)
    if left >= 0:
        ok &= j >= ip - left
    if right >= 0:
        ok &= j <= ip + right
    return ok


def score_transform(s, rows, Sq, Sk, softcap=0.0, slope=None):
    """Map scaled logits s (rows x Sk) to final logits z.

    softcap: z = c * tanh(s / c) (section "进阶参数如何配置…", ``softcap``);
    ALiBi:   z -= slope * |i' - j| (same section, ``alibi_slopes``).
    Returns (z, t) where t = tanh(s / c) (or None) for the backward."""
    t = None
    if softcap and softcap > 0.0:
        t = np.tanh(s / softcap)
        z = softcap * t
    else:
        z = s.copy()
    if slope is not None:
        ip = np.asarray(rows, dtype=np.int64)[:, None] + (Sk - Sq)
        j = np.arange(Sk, dtype=np.int64)[None, :]
        z = z - float(slope) * np.abs(ip - j).astype(np.float64)
    return z, t


def _row_block(qh, kh, rows, Sq, Sk, scale, causal, window, softcap, slope):
    """Full score rows for a block of query rows: returns (z, t, allowed)."""
    s = scale * (qh[rows] @ kh.T)
    z, t = score_transform(s, rows, Sq, Sk, softcap, slope)
    ok = allowed_mask(rows, Sq, Sk, causal, window)
    return z, t, ok


def _softmax_rows(z, ok):
    """Row softmax over allowed entries: returns (P, LSE); empty rows give
    P = 0 and LSE = +inf."""
    zm = np.where(ok, z, -np.inf)
    m = zm.max(axis=1, initial=-np.inf)  # no keys at all (Sk = 0) is an empty row too
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.where(ok, np.exp(zm - m_safe[:, None]), 0.0)
    l = e.sum(axis=1)
    with np.errstate(divide="ignore"):
        lse = np.where(empty, np.inf, m_safe + np.log(np.where(empty, 1.0, l)))
    P = np.where(empty[:, None], 0.0, e / np.where(empty, 1.0, l)[:, None])
    return P, lse


def _dropped(P, dropout, bh, rows, cols):
    """(P * K * scale, K * scale) for dropout = (p, seed, offset), else (P, None)."""
    if dropout is None:
        return P, None
    p, seed, offset = dropout
    km = keep_mask(p, seed, offset, bh, rows, cols) * keep_scale(p)
    return P * km, km


def attention_fwd(q, k, v, scale, causal=False, window=(-1, -1), softcap=0.0,
                  alibi_slopes=None, heads=None, q_rows=None, dropout=None, batch0=0):
    """Standard attention forward in float64.

    q (B, Sq, Hq, D); k, v (B, Sk, Hkv, D) — any float dtype, converted exactly.
    Returns (out, lse): out (B, Sq, Hq, D) float64, lse (B, Hq, Sq) float64.
    ``heads`` / ``q_rows`` restrict the work to a subset (other entries are
    NaN) so that single rows of very long sequences can be checked.
    ``dropout`` = (p, seed, offset) drops attention weights as defined in
    ``oracle.dropout`` (batch entry b counts as b + batch0); LSE is that of
    the undropped weights.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    assert Hq % Hkv == 0, "query heads must be a multiple of K/V heads"
    g = Hq // Hkv
    slopes = None if alibi_slopes is None else _f64(alibi_slopes)
    heads = range(Hq) if heads is None else heads
    rows_all = np.arange(Sq) if q_rows is None else np.asarray(q_rows, dtype=np.int64)
    out = np.full((B, Sq, Hq, D), np.nan)
    lse = np.full((B, Hq, Sq), np.nan)
    for b in range(B):
        for h in heads:
            kh = k[b, :, h // g, :]
            vh = v[b, :, h // g, :]
            qh = q[b, :, h, :]
            slope = None if slopes is None else slopes[h]
            for c0 in range(0, len(rows_all), ROW_CHUNK):
                rows = rows_all[c0:c0 + ROW_CHUNK]
                z, _, ok = _row_block(qh, kh, rows, Sq, Sk, scale, causal, window, softcap, slope)
                P, L = _softmax_rows(z, ok)
                Pd, _ = _dropped(P, dropout, (b + batch0) * Hq + h, rows, np.arange(Sk))
                out[b, rows, h, :] = Pd @ vh
                lse[b, h, rows] = L
    return out, lse


def attention_bwd(q, k, v, dout, scale, causal=False, window=(-1, -1), softcap=0.0,
                  alibi_slopes=None, heads=None, k_rows=None, q_rows=None, check_delta=True,
                  dropout=None, batch0=0):
    """Analytic backward of standard attention in float64.

    The pages' method recomputes the attention matrix in the backward pass
    instead of storing it (page "FlashAttention 实战指南…", section
    "FlashAttention 的做法是三个手段配合"); the values it must reproduce are
    the gradients of the forward above:

      dP_ij = dO_i . v_j ;  delta_i = sum_j P_ij dP_ij
      dZ_ij = P_ij (dP_ij - delta_i)
      dS_ij = dZ_ij (1 - tanh^2(s_ij / c))   if softcap c > 0, else dZ_ij
      dq_i  = scale * sum_j dS_ij k_j
      dk_j  = scale * sum_{h in group} sum_i dS_ij q_i
      dv_j  = sum_{h in group} sum_i P_ij dO_i

    ALiBi and masks carry no gradient.  Returns (dq, dk, dv) float64.

    With ``dropout`` (see ``attention_fwd``) the forward multiplies P by
    M = K * scale before V, so dV uses P * M and dP_ij = M_ij (dO_i . v_j);
    delta_i = sum_j P_ij dP_ij is still dO_i . O_i.

    ``heads`` restricts dq to those query heads and accumulates dk/dv only
    from them; ``k_rows`` restricts dk/dv to a subset of key rows (dq is then
    not computed).  With ``k_rows`` the row term delta_i is taken as
    dO_i . O_i, the same quantity (sum_j P_ij dP_ij = dO_i . sum_j P_ij v_j),
    so that full rows of dP are not needed.  ``q_rows`` restricts the work to
    dq of those query rows (dk/dv are then not computed); each dq row needs
    only its own row of P and dP.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    g = Hq // Hkv
    slopes = None if alibi_slopes is None else _f64(alibi_slopes)
    heads = list(range(Hq)) if heads is None else list(heads)
    dq = np.full(q.shape, np.nan)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    cols = np.arange(Sk) if k_rows is None else np.asarray(k_rows, dtype=np.int64)
    for b in range(B):
        for h in heads:
            kh, vh, qh, doh = k[b, :, h // g, :], v[b, :, h // g, :], q[b, :, h, :], do[b, :, h, :]
            slope = None if slopes is None else slopes[h]
            dq_h = np.full((Sq, D), np.nan) if q_rows is not None else np.zeros((Sq, D))
            row_list = np.arange(Sq) if q_rows is None else np.asarray(q_rows, dtype=np.int64)
            for c0 in range(0, len(row_list), ROW_CHUNK):
                rows = row_list[c0:c0 + ROW_CHUNK]
                z, t, ok = _row_block(qh, kh, rows, Sq, Sk, scale, causal, window, softcap, slope)
                P, _ = _softmax_rows(z, ok)
                Pd, km = _dropped(P, dropout, (b + batch0) * Hq + h, rows, np.arange(Sk))
                if q_rows is not None:
                    dP = doh[rows] @ vh.T
                    if km is not None:
                        dP = dP * km
                    delta = (P * dP).sum(axis=1)
                    dZ = P * (dP - delta[:, None])
                    dS = dZ * (1.0 - t * t) if t is not None else dZ
                    dq_h[rows] = scale * (dS @ kh)
                elif k_rows is None:
                    dP = doh[rows] @ vh.T
                    if km is not None:
                        dP = dP * km
                    delta = (P * dP).sum(axis=1)
                    if check_delta:
                        alt = (doh[rows] * (Pd @ vh)).sum(axis=1)
                        assert np.allclose(delta, alt, rtol=1e-10, atol=1e-10)
                    dZ = P * (dP - delta[:, None])
                    dS = dZ * (1.0 - t * t) if t is not None else dZ
                    dq_h[rows] = scale * (dS @ kh)
                    dk[b, :, h // g, :] += scale * (dS.T @ qh[rows])
                    dv[b, :, h // g, :] += Pd.T @ doh[rows]
                else:
                    o_rows = Pd @ vh
                    delta = (doh[rows] * o_rows).sum(axis=1)
                    Pc = P[:, cols]
                    dPc = doh[rows] @ vh[cols].T
                    if km is not None:
                        dPc = dPc * km[:, cols]
                    dZ = Pc * (dPc - delta[:, None])
                    dS = dZ * (1.0 - t[:, cols] ** 2) if t is not None else dZ
                    dk[b, cols, h // g, :] += scale * (dS.T @ qh[rows])
                    dv[b, cols, h // g, :] += Pd[:, cols].T @ doh[rows]
            if k_rows is None:
                dq[b, :, h, :] = dq_h
    if q_rows is not None:
        dk[:] = np.nan
        dv[:] = np.nan
    return dq, dk, dv
