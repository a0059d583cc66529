"""GPU parity of the packed varlen forward / backward (runs on an MI355X)."""
import numpy as np
import pytest
import torch

import io_aware_exact_qk_amd as fa
from oracle import varlen_fwd, varlen_bwd, attention_fwd, attention_bwd
from workloads import varlen_case, cfg4
from _helpers import DEV, assert_out, assert_lse, assert_grad, say, np64, tile_rows

pytestmark = pytest.mark.gpu


def _run(c, bwd=True):
    q, k, v = (t.to(DEV) for t in (c.q, c.k, c.v))
    cq, ck = c.cu_seqlens_q.to(DEV), c.cu_seqlens_k.to(DEV)
    al = None if c.alibi_slopes is None else c.alibi_slopes.to(DEV)
    kw = dict(scale=c.scale, causal=c.causal, window=c.window, softcap=c.softcap, alibi_slopes=al)
    out, lse = fa.fa_fwd_varlen(q, k, v, cq, ck, c.max_seqlen_q, c.max_seqlen_k, **kw)
    grads = None
    if bwd:
        grads = fa.fa_bwd_varlen(q, k, v, out, c.dout.to(DEV), lse, cq, ck, c.max_seqlen_q,
                                 c.max_seqlen_k, **kw)
    torch.cuda.synchronize()
    return out, lse, grads


@pytest.mark.parametrize("causal,window,softcap,alibi,hkv", [
    (True, (-1, -1), 0.0, False, 2), (False, (-1, -1), 0.0, False, 4), (True, (50, 0), 20.0, True, 1)])
def test_small_varlen(causal, window, softcap, alibi, hkv):
    lens = [5, 0, 130, 1, 257, 64, 300]
    c = varlen_case(lens, Hq=4, Hkv=hkv, D=128, seed=41, causal=causal, window=window, softcap=softcap,
                    alibi=alibi)
    say("varlen small", lens, causal, window, softcap, alibi, hkv)
    out, lse, (dq, dk, dv) = _run(c)
    args = (c.q, c.k, c.v, c.cu_seqlens_q, c.cu_seqlens_k, c.scale, causal, window, softcap, c.alibi_slopes)
    ro, rl = varlen_fwd(*args[:3], *args[3:])
    assert_out(out, ro, torch.bfloat16)
    assert_lse(lse, rl)
    gq, gk, gv = varlen_bwd(c.q, c.k, c.v, c.dout, *args[3:])
    assert_grad(dq, gq, "dq")
    assert_grad(dk, gk, "dk")
    assert_grad(dv, gv, "dv")


def test_varlen_unequal_q_k_lengths():
    lq, lk = [3, 70, 129, 1], [10, 70, 300, 64]
    c = varlen_case(lq, lk, Hq=2, Hkv=2, D=64, dtype="fp16", seed=42, causal=True)
    say("varlen q/k lengths differ")
    out, lse, (dq, dk, dv) = _run(c)
    args = (c.cu_seqlens_q, c.cu_seqlens_k, c.scale, True)
    ro, rl = varlen_fwd(c.q, c.k, c.v, *args)
    assert_out(out, ro, torch.float16)
    assert_lse(lse, rl)
    gq, gk, gv = varlen_bwd(c.q, c.k, c.v, c.dout, *args)
    assert_grad(dq, gq, "dq")
    assert_grad(dk, gk, "dk")
    assert_grad(dv, gv, "dv")


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_queries_without_keys_and_keys_without_queries(causal):
    # sequence 0: queries, no keys (O = 0, LSE = +inf, dQ = 0); sequence 1:
    # keys, no queries (dK = dV = 0); the rest ordinary.  The dQ kernel writes
    # the row terms the dK/dV kernel reads, so both kinds of empty side meet.
    lq, lk = [4, 0, 100, 33], [0, 50, 100, 70]
    c = varlen_case(lq, lk, Hq=4, Hkv=2, D=128, seed=43, causal=causal)
    say("varlen empty sides", lq, lk, causal)
    out, lse, (dq, dk, dv) = _run(c)
    args = (c.cu_seqlens_q, c.cu_seqlens_k, c.scale, causal)
    ro, rl = varlen_fwd(c.q, c.k, c.v, *args)
    assert_out(out, ro, torch.bfloat16)
    assert_lse(lse, rl)
    assert torch.isinf(lse[:, :4]).all() and (out[:4] == 0).all()
    gq, gk, gv = varlen_bwd(c.q, c.k, c.v, c.dout, *args)
    assert_grad(dq, gq, "dq")
    assert_grad(dk, gk, "dk")
    assert_grad(dv, gv, "dv")
    assert (dq[:4] == 0).all() and (dk[:50] == 0).all() and (dv[:50] == 0).all()


@pytest.mark.parametrize("side", ["no_keys", "no_queries"])
def test_varlen_one_side_empty_everywhere(side):
    """total_k = 0: O = 0, LSE = +inf and dQ = 0 are written (over NaN-filled
    buffers); total_q = 0: dK = dV = 0 are written.  The empty side's tensors
    have no storage at all."""
    lq, lk = ([5, 130, 1], [0, 0, 0]) if side == "no_keys" else ([0, 0, 0], [7, 140, 2])
    c = varlen_case(lq, lk, Hq=4, Hkv=2, D=128, seed=44, causal=False)
    q, k, v, do = (t.to(DEV) for t in (c.q, c.k, c.v, c.dout))
    cq, ck = c.cu_seqlens_q.to(DEV), c.cu_seqlens_k.to(DEV)
    nan = float("nan")
    out = torch.full_like(q, nan)
    lse = torch.full((4, q.shape[0]), nan, device=DEV)
    dq, dk, dv = torch.full_like(q, nan), torch.full_like(k, nan), torch.full_like(v, nan)
    say("varlen one side empty", side)
    fa.fa_fwd_varlen(q, k, v, cq, ck, c.max_seqlen_q, c.max_seqlen_k, out=out, lse=lse, scale=c.scale)
    fa.fa_bwd_varlen(q, k, v, out, do, lse, cq, ck, c.max_seqlen_q, c.max_seqlen_k, dq=dq, dk=dk, dv=dv,
                     scale=c.scale)
    torch.cuda.synchronize()
    if side == "no_keys":
        assert (out == 0).all() and torch.isposinf(lse).all() and (dq == 0).all()
    else:
        assert (dk == 0).all() and (dv == 0).all()


def test_cfg4_full_size_sampled():
    """Every sequence, every head: O, LSE and dQ on one seeded row of every
    128-row query tile (plus first and last rows); dK/dV on one seeded key of
    every 256-key block for one head per sequence."""
    c = cfg4()
    say("varlen", c.name)
    out, lse, (dq, dk, dv) = _run(c)
    o_g, l_g, dq_g, dk_g, dv_g = (np64(x) for x in (out, lse, dq, dk, dv))
    cq = c.cu_seqlens_q.tolist()
    H = c.q.shape[1]
    for s in range(len(cq) - 1):
        a, b = cq[s], cq[s + 1]
        L = b - a
        qs, ks, vs, ds = (t[a:b][None] for t in (c.q, c.k, c.v, c.dout))
        for h in range(H):
            rows = tile_rows(L, 128, 4000 + 100 * s + h)
            ro, rl = attention_fwd(qs, ks, vs, c.scale, True, heads=[h], q_rows=rows)
            ar = np.asarray(rows) + a
            assert_out(o_g[ar, h], ro[0, rows, h], torch.bfloat16, what=f"out seq {s} head {h}")
            assert_lse(l_g[h, ar], rl[0, h, rows], what=f"lse seq {s} head {h}")
            gq, _, _ = attention_bwd(qs, ks, vs, ds, c.scale, True, heads=[h], q_rows=rows)
            assert_grad(dq_g[ar, h], gq[0, rows, h], f"dq seq {s} head {h}")
        h = s % H
        keys = tile_rows(L, 256, 4500 + s)
        _, gk, gv = attention_bwd(qs, ks, vs, ds, c.scale, True, heads=[h], k_rows=keys)
        ak = np.asarray(keys) + a
        assert_grad(dk_g[ak, h], gk[0, keys, h], f"dk seq {s} head {h}")
        assert_grad(dv_g[ak, h], gv[0, keys, h], f"dv seq {s} head {h}")


def test_sequence_isolation_bitwise():
    lens = [100, 260, 7, 190]
    c = varlen_case(lens, Hq=4, Hkv=2, D=128, seed=43, causal=True)
    say("varlen isolation")
    o1, l1, g1 = _run(c)
    cq = c.cu_seqlens_q.tolist()
    a, b = cq[1], cq[2]
    c.q[a:b] = -c.q[a:b]
    c.k[a:b] = c.k[a:b] * 2
    c.dout[a:b] = c.dout[a:b] * 3
    o2, l2, g2 = _run(c)
    keep = torch.cat([torch.arange(0, a), torch.arange(b, cq[-1])]).to(DEV)
    assert torch.equal(o1[keep], o2[keep])
    assert torch.equal(l1[:, keep], l2[:, keep])
    for x, y in zip(g1, g2):
        assert torch.equal(x[keep], y[keep])
    assert not torch.equal(o1[a:b], o2[a:b])


def _tile_list(lengths, tile, levels, ascending, heads):
    """The tile list the library builds, written out in Python.  Every
    (sequence, t) with t < min(ceil(L / tile), levels).  Up to 4096
    sequences: sequences sorted by that tile count, most first (ties: lower
    index first), in groups of 32 // heads (at least 1); each group level by
    level (t from its highest down, or from 0 up), sorted order within a
    level.  More sequences: level by level (levels - 1 down, or 0 up),
    index order within a level.  Then (-1, -1) up to the bound
    (total + nseq (tile - 1)) // tile."""
    n = [min(-(-L // tile), levels) for L in lengths]
    if len(n) <= 4096:
        grp = max(1, 32 // heads)
        order = sorted(range(len(n)), key=lambda s: (-n[s], s))
        out = []
        for g0 in range(0, len(n), grp):
            members = order[g0:g0 + grp]
            top = max(n[s] for s in members)
            for t in (range(top) if ascending else range(top - 1, -1, -1)):
                out += [(s, t) for s in members if n[s] > t]
    else:
        lv = range(levels) if ascending else range(levels - 1, -1, -1)
        out = [(s, t) for t in lv for s, ns in enumerate(n) if ns > t]
    bound = (sum(lengths) + len(lengths) * (tile - 1)) // tile
    return np.array(out + [(-1, -1)] * (bound - len(out)), dtype=np.int32).reshape(-1, 2)


@pytest.mark.parametrize("shape", ["many_short", "very_long", "mixed", "gqa", "very_many"])
def test_tile_lists_bit_exact(shape):
    """The (sequence, tile) lists of the forward (128-row query tiles) and the
    backward (query tiles for dQ, 256-key tiles for dK/dV, key tiles heaviest
    first = from tile 0 for causal) equal the Python construction, entry for
    entry, including lengths of 0, sequences longer than 1024 tiles, group
    sizes 32 (one head), 2 and 16 (16 query heads, 2 K/V heads), and more
    sequences than the sorted construction takes (the level-by-level one)."""
    rng = np.random.default_rng({"many_short": 1, "very_long": 2, "mixed": 3, "gqa": 4, "very_many": 5}[shape])
    Hq = Hkv = 1
    if shape == "many_short":
        lq = [int(x) for x in rng.integers(0, 300, size=2500)]
    elif shape == "very_long":
        lq = [140000, 0, 5, 300]
    elif shape == "gqa":
        lq = [int(x) for x in rng.integers(0, 1500, size=60)] + [0, 256, 255]
        Hq, Hkv = 16, 2
    elif shape == "very_many":
        lq = [int(x) for x in rng.integers(0, 40, size=5000)] + [700]
    else:
        lq = [int(x) for x in rng.integers(0, 5000, size=40)] + [0, 129, 128, 127, 1]
    lk = [L + int(rng.integers(0, 3)) if L else 0 for L in lq]
    c = varlen_case(lq, lk, Hq=Hq, Hkv=Hkv, D=32, seed=45, causal=True, window=(32, 0))
    q, k, v, do = (t.to(DEV) for t in (c.q, c.k, c.v, c.dout))
    cq, ck = c.cu_seqlens_q.to(DEV), c.cu_seqlens_k.to(DEV)
    L = fa.lib()
    nseq, tq, tk = len(lq), q.shape[0], k.shape[0]
    wsf = torch.full((L.fa_fwd_varlen_workspace_size(nseq, tq, Hq, 32),), 0x7F, dtype=torch.uint8, device=DEV)
    wsb = torch.full((L.fa_bwd_varlen_workspace_size(nseq, tq, tk, Hq, 32, 0),), 0x7F, dtype=torch.uint8,
                     device=DEV)
    say("varlen tile lists", shape, nseq, tq, tk)
    kw = dict(scale=c.scale, causal=True, window=(32, 0))
    out, lse = fa.fa_fwd_varlen(q, k, v, cq, ck, c.max_seqlen_q, c.max_seqlen_k, workspace=wsf, **kw)
    fa.fa_bwd_varlen(q, k, v, out, do, lse, cq, ck, c.max_seqlen_q, c.max_seqlen_k, workspace=wsb, **kw)
    torch.cuda.synchronize()
    want_q = _tile_list(lq, 128, -(-c.max_seqlen_q // 128), False, Hq)
    want_k = _tile_list(lk, 256, -(-c.max_seqlen_k // 256), True, Hkv)
    got_f = wsf.cpu().numpy().view(np.int32)[:want_q.size].reshape(-1, 2)
    np.testing.assert_array_equal(got_f, want_q)
    rows = -(-(Hq * tq * 4) // 256) * 256
    lists = wsb.cpu().numpy()[2 * rows:]
    q_bytes = -(-(want_q.size * 4) // 256) * 256
    np.testing.assert_array_equal(lists[:want_q.size * 4].view(np.int32).reshape(-1, 2), want_q)
    np.testing.assert_array_equal(lists[q_bytes:q_bytes + want_k.size * 4].view(np.int32).reshape(-1, 2), want_k)
    # the launch itself is still right (a window of 32 keys keeps the check cheap)
    pick = [i for i, n in enumerate(lq) if n][:3] + [len(lq) - 1]
    cqs = c.cu_seqlens_q.tolist()
    cks = c.cu_seqlens_k.tolist()
    for s in pick:
        a, b, ka, kb = cqs[s], cqs[s + 1], cks[s], cks[s + 1]
        if b == a:
            continue
        rows_s = sorted(set([0, (b - a) // 2, b - a - 1]))
        ro, rl = attention_fwd(c.q[a:b][None], c.k[ka:kb][None], c.v[ka:kb][None], c.scale, True, (32, 0),
                               q_rows=rows_s)
        assert_out(out[a:b][None][:, rows_s], ro[:, rows_s], torch.bfloat16)
        assert_lse(lse[:, a:b][None][:, :, rows_s], rl[:, :, rows_s])
