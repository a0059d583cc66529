"""GPU parity of the paged KV-cache decode (split + combine) against the oracle."""
import numpy as np
import pytest
import torch

import io_aware_exact_qk_amd as fa
from oracle import kvcache_fwd
from workloads import decode_case, cfg5, alibi_slopes
from _helpers import DEV, assert_out, assert_lse, say, np64

pytestmark = pytest.mark.gpu


def _run(c, num_splits, append=True, block_table="given", **opts):
    q = c.q.to(DEV)
    kc, vc = c.k_cache.to(DEV), c.v_cache.to(DEV)
    bt = c.block_table.to(DEV) if (c.block_table is not None and block_table == "given") else None
    rot = (c.rotary_cos.to(DEV), c.rotary_sin.to(DEV)) if c.rotary_cos is not None else (None, None)
    out, lse = fa.fa_fwd_kvcache(q, kc, vc, c.cache_seqlens.to(DEV),
                                 c.k_new.to(DEV) if append else None,
                                 c.v_new.to(DEV) if append else None,
                                 bt, rot[0], rot[1], c.rotary_dim if rot[0] is not None else None,
                                 num_splits=num_splits, scale=c.scale, **opts)
    torch.cuda.synchronize()
    return out, lse, kc, vc


def _oracle(c, append=True, **opts):
    return kvcache_fwd(c.q, c.k_new if append else None, c.v_new if append else None, c.k_cache,
                       c.v_cache, c.cache_seqlens, c.block_table, c.page_size, c.rotary_cos,
                       c.rotary_sin, c.rotary_dim, c.scale,
                       cache_dtype="bf16" if c.q.dtype == torch.bfloat16 else "fp16", **opts)


def _masked_lse_ok(lse, ref):
    """LSE check that treats empty rows (+inf on both sides) as equal."""
    assert_lse(lse, ref)


def _check_cache(c, ref, kc, vc, paged=True):
    """Appended slots hold the oracle's k_app (within 1 ulp when rotated) and
    v_new exactly; every other cache byte is unchanged."""
    k_after, v_after = kc.cpu(), vc.cpu()
    k_before, v_before = c.k_cache.clone(), c.v_cache.clone()
    for (b, t, phys) in ref["slots"]:
        ka = k_after[phys[0], phys[1]].double().numpy()
        ref_k = ref["k_app"][b, t]
        if c.rotary_cos is None or c.rotary_dim == 0:
            np.testing.assert_array_equal(ka, ref_k)
        else:
            ulp = np.abs(ref_k) * 2.0 ** -7 + 1e-30
            assert (np.abs(ka - ref_k) <= ulp).all(), "appended key differs by more than 1 ulp"
        np.testing.assert_array_equal(v_after[phys[0], phys[1]].double().numpy(), ref["v_app"][b, t])
        k_before[phys[0], phys[1]] = k_after[phys[0], phys[1]]
        v_before[phys[0], phys[1]] = v_after[phys[0], phys[1]]
    # compared as bit patterns, so NaN-filled slots compare equal to themselves
    assert torch.equal(k_before.view(torch.int16), k_after.view(torch.int16)), \
        "cache bytes outside the appended slots changed"
    assert torch.equal(v_before.view(torch.int16), v_after.view(torch.int16)), \
        "cache bytes outside the appended slots changed"


SMALL = [
    # B, Hq, Hkv, D, page, seqlens, dtype, rotary_dim, paged
    (3, 8, 2, 128, 64, [300, 77, 64], "bf16", 128, True),
    (2, 4, 4, 64, 32, [31, 200], "fp16", 32, True),
    (2, 32, 1, 128, 256, [1000, 1], "bf16", 0, True),
    (4, 16, 4, 128, 128, [0, 5, 127, 128], "bf16", 64, False),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"d{i}" for i in range(len(SMALL))])
@pytest.mark.parametrize("num_splits", [1, 3, 16])
def test_small_decode(case, num_splits):
    B, Hq, Hkv, D, page, lens, dt, rd, paged = case
    c = decode_case(B=B, Hq=Hq, Hkv=Hkv, D=D, page=page, seqlens=lens, seed=51, dtype=dt,
                    rotary_dim=rd, paged=paged)
    say("decode small", case, num_splits)
    out, lse, kc, vc = _run(c, num_splits)
    ref = _oracle(c)
    assert_out(out, ref["out"], c.q.dtype)
    assert_lse(lse, ref["lse"])
    _check_cache(c, ref, kc, vc, paged)


# Cache slots past the live keys hold non-finite values (never-written or
# recycled pages): they must not reach the output, at any split count, with
# and without the append, with one and several new tokens.
POISON = [
    # B, Hq, Hkv, D, page, seqlens, rotary_dim, sq_new, append
    (3, 8, 2, 128, 64, [300, 77, 64], 128, 1, True),
    (2, 4, 4, 64, 32, [31, 200], 32, 1, False),
    (2, 8, 2, 128, 64, [190, 33], 64, 3, True),
]


@pytest.mark.parametrize("poison", [float("nan"), float("inf")], ids=["nan", "inf"])
@pytest.mark.parametrize("num_splits", [1, 3, 16])
@pytest.mark.parametrize("case", POISON, ids=[f"p{i}" for i in range(len(POISON))])
def test_nonfinite_cache_tail(case, num_splits, poison):
    B, Hq, Hkv, D, page, lens, rd, T, append = case
    c = decode_case(B=B, Hq=Hq, Hkv=Hkv, D=D, page=page, seqlens=lens, seed=58, rotary_dim=rd,
                    poison=poison, sq_new=T)
    say("decode non-finite tail", case, num_splits, poison)
    out, lse, kc, vc = _run(c, num_splits, append=append)
    ref = _oracle(c, append=append)
    assert torch.isfinite(out).all()
    assert_out(out, ref["out"], c.q.dtype)
    assert_lse(lse, ref["lse"])
    if append:
        _check_cache(c, ref, kc, vc)


def test_decode_without_append():
    c = decode_case(B=2, Hq=8, Hkv=2, D=128, page=64, seqlens=[150, 64], seed=52)
    say("decode no append")
    out, lse, kc, vc = _run(c, 2, append=False)
    ref = _oracle(c, append=False)
    assert_out(out, ref["out"], torch.bfloat16)
    assert_lse(lse, ref["lse"])
    assert torch.equal(kc.cpu(), c.k_cache) and torch.equal(vc.cpu(), c.v_cache)


def test_block_table_permutation_bitwise():
    c = decode_case(B=2, Hq=8, Hkv=2, D=128, page=64, seqlens=[500, 260], seed=53)
    say("decode permuted pages")
    o1, l1, _, _ = _run(c, 4)
    n = c.k_cache.shape[0]
    perm = torch.from_numpy(np.random.default_rng(7).permutation(n))
    inv = torch.argsort(perm)
    c.k_cache = c.k_cache[perm].contiguous()
    c.v_cache = c.v_cache[perm].contiguous()
    live = c.block_table >= 0
    bt = c.block_table.clone()
    bt[live] = inv[c.block_table[live].long()].to(torch.int32)
    c.block_table = bt
    o2, l2, _, _ = _run(c, 4)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_cfg5_full():
    """The paged decode workload at num_splits 1, 4 and 16: each against the
    oracle (all sequences, all heads), the cache append checked byte by byte,
    and the three outputs within one bf16 ulp of each other at the scale of
    their row (largest |O| of the row): the split count moves each part's
    exponent reference and so the rounding of its 16-bit weights, which
    changes small elements of a row by more than their own ulp.  The spread
    in units of each element's own ulp is printed."""
    c = cfg5()
    ref = _oracle(c)
    outs = {}
    for num_splits in (1, 4, 16):
        say("decode", c.name, "splits", num_splits)
        out, lse, kc, vc = _run(c, num_splits)
        assert_out(out, ref["out"], torch.bfloat16, what=f"out splits={num_splits}")
        assert_lse(lse, ref["lse"], what=f"lse splits={num_splits}")
        _check_cache(c, ref, kc, vc)
        outs[num_splits] = (np64(out), np64(lse))
        del kc, vc
    def ulp(x):
        return np.exp2(np.floor(np.log2(np.maximum(x, 2.0 ** -126))) - 7)

    for a, b in ((1, 4), (1, 16), (4, 16)):
        oa, ob = outs[a][0], outs[b][0]
        d = np.abs(oa - ob)
        own = d / ulp(np.maximum(np.abs(oa), np.abs(ob)))
        row = d / ulp(np.maximum(np.abs(oa), np.abs(ob)).max(axis=-1, keepdims=True))
        say(f"splits {a} vs {b}: {int((d > 0).sum())} elements differ; max {own.max():.2f} ulp of the "
            f"element ({int((own > 1).sum())} beyond 1), max {row.max():.3f} ulp of the row's largest |O|")
        assert (row <= 1.0).all(), f"splits {a} and {b} differ by more than one bf16 ulp of the row scale"
        assert np.abs(outs[a][1] - outs[b][1]).max() <= 1e-5, f"lse of splits {a} and {b}"


# Rotary half-widths of 8 and 24 elements (rotary_dim 16 and 48): the partner
# of a chunk then sits in the other half of the wave's chunk split.
@pytest.mark.parametrize("rotary_dim", [16, 48])
def test_partial_rotary_odd_chunk_offset(rotary_dim):
    c = decode_case(B=3, Hq=8, Hkv=2, D=128, page=64, seqlens=[190, 64, 1], seed=54, rotary_dim=rotary_dim)
    say("decode rotary_dim", rotary_dim)
    out, lse, kc, vc = _run(c, 3)
    ref = _oracle(c)
    assert_out(out, ref["out"], c.q.dtype)
    assert_lse(lse, ref["lse"])
    _check_cache(c, ref, kc, vc)


def test_large_batch_unsorted_order():
    """More sequences than the longest-first scheduler ranks (identity order)."""
    lens = [int(x) for x in np.random.default_rng(55).integers(0, 300, size=70)]
    c = decode_case(B=70, Hq=4, Hkv=2, D=64, page=32, seqlens=lens, seed=55)
    say("decode B=70")
    out, lse, kc, vc = _run(c, 2)
    ref = _oracle(c)
    assert_out(out, ref["out"], c.q.dtype)
    assert_lse(lse, ref["lse"])
    _check_cache(c, ref, kc, vc)


def test_many_splits_combine():
    """More splits than one wave's lanes (the combine walks them 64 at a time),
    most of them empty."""
    c = decode_case(B=2, Hq=8, Hkv=2, D=128, page=32, seqlens=[4000, 33], seed=56)
    say("decode 100 splits")
    out, lse, kc, vc = _run(c, 100)
    ref = _oracle(c)
    assert_out(out, ref["out"], c.q.dtype)
    assert_lse(lse, ref["lse"])
    _check_cache(c, ref, kc, vc)


# Logit options: softcap, ALiBi and a left window.  The window edge falls
# inside a page, on a page boundary, past the start of the cache, and at 0
# (the new query sees only itself).
OPTS = [
    # window_left, softcap, alibi
    (100, 0.0, False),
    (64, 0.0, False),
    (0, 0.0, False),
    (5000, 0.0, False),
    (-1, 30.0, False),
    (-1, 0.0, True),
    (150, 20.0, True),
]


@pytest.mark.parametrize("opt", OPTS, ids=[f"o{i}" for i in range(len(OPTS))])
@pytest.mark.parametrize("num_splits", [1, 4])
def test_decode_logit_options(opt, num_splits):
    wl, sc, al = opt
    c = decode_case(B=3, Hq=8, Hkv=2, D=128, page=64, seqlens=[700, 63, 200], seed=57, rotary_dim=64)
    slopes = alibi_slopes(8) if al else None
    say("decode options", opt, num_splits)
    out, lse, kc, vc = _run(c, num_splits, window=(wl, -1), softcap=sc,
                            alibi_slopes=None if slopes is None else slopes.to(DEV))
    ref = _oracle(c, window=(wl, -1), softcap=sc, alibi_slopes=slopes)
    assert_out(out, ref["out"], c.q.dtype)
    assert_lse(lse, ref["lse"])
    _check_cache(c, ref, kc, vc)


@pytest.mark.parametrize("B,Hkv,lens", [(1, 8, [5000]), (8, 8, None), (40, 2, None)])
def test_auto_splits(B, Hkv, lens):
    """num_splits = 0: the library picks the count; the result is the oracle's."""
    if lens is None:
        lens = [int(x) for x in np.random.default_rng(58).integers(1, 3000, size=B)]
    c = decode_case(B=B, Hq=4 * Hkv, Hkv=Hkv, D=128, page=256, seqlens=lens, seed=58)
    say("decode auto splits", B, Hkv)
    out, lse, kc, vc = _run(c, 0)
    ref = _oracle(c)
    assert_out(out, ref["out"], c.q.dtype)
    assert_lse(lse, ref["lse"])
    _check_cache(c, ref, kc, vc)


# Several new tokens per sequence (chunked append): G * T <= 32 columns.
MULTI = [
    # B, Hq, Hkv, D, page, seqlens, T, causal, append, paged, rotary, opts, splits
    (3, 8, 2, 128, 64, [300, 62, 1], 4, True, True, True, 64, {}, 1),
    (3, 8, 2, 128, 64, [300, 62, 1], 4, True, True, True, 64, {}, 3),
    (2, 4, 4, 64, 32, [31, 200], 8, True, True, False, 32, {}, 2),
    (2, 8, 1, 128, 128, [500, 129], 4, False, True, True, 0, {}, 4),
    (2, 4, 2, 128, 64, [190, 70], 16, True, False, True, 0, {}, 2),
    (2, 8, 2, 128, 64, [400, 90], 3, True, True, True, 64,
     dict(window=(50, -1), softcap=20.0, alibi=True), 3),
    (1, 2, 1, 128, 32, [5], 16, True, True, True, 0, {}, 1),
    (2, 4, 2, 64, 64, [150, 300], 6, False, True, True, 0, dict(window=(40, 3)), 2),
]


@pytest.mark.parametrize("case", MULTI, ids=[f"m{i}" for i in range(len(MULTI))])
def test_multi_token_decode(case):
    B, Hq, Hkv, D, page, lens, T, causal, append, paged, rd, opts, splits = case
    c = decode_case(B=B, Hq=Hq, Hkv=Hkv, D=D, page=page, seqlens=lens, seed=59 + T, rotary_dim=rd,
                    paged=paged, sq_new=T)
    slopes = alibi_slopes(Hq) if opts.get("alibi") else None
    kw = dict(window=opts.get("window", (-1, -1)), softcap=opts.get("softcap", 0.0))
    say("decode multi-token", case)
    out, lse, kc, vc = _run(c, splits, append=append, causal=causal,
                            alibi_slopes=None if slopes is None else slopes.to(DEV), **kw)
    ref = _oracle(c, append=append, causal=causal, alibi_slopes=slopes, **kw)
    assert_out(out, ref["out"], c.q.dtype)
    _masked_lse_ok(lse, ref["lse"])
    if append:
        _check_cache(c, ref, kc, vc)
    else:
        assert torch.equal(kc.cpu(), c.k_cache) and torch.equal(vc.cpu(), c.v_cache)


# Head dims 32 and 96 (96 runs padded on the 128-wide kernel).
@pytest.mark.parametrize("D,rd", [(32, 32), (96, 96), (96, 32)])
@pytest.mark.parametrize("num_splits,T", [(1, 1), (3, 1), (2, 3)])
def test_decode_head_dims(D, rd, num_splits, T):
    c = decode_case(B=3, Hq=8, Hkv=2, D=D, page=64, seqlens=[300, 63, 1], seed=60 + D, rotary_dim=rd, sq_new=T)
    say("decode head dim", D, rd, num_splits, T)
    out, lse, kc, vc = _run(c, num_splits, causal=True)
    ref = _oracle(c, causal=True)
    assert_out(out, ref["out"], c.q.dtype)
    assert_lse(lse, ref["lse"])
    _check_cache(c, ref, kc, vc)
