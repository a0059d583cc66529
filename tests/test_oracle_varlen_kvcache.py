"""Pins for the varlen and KV-cache oracles and for the input recipes (CPU)."""
import math

import numpy as np
import pytest
import torch

from oracle import (attention_fwd, attention_bwd, varlen_fwd, varlen_bwd, rotary_apply,
                    round_bf16, kvcache_fwd, gather_logical_cache)
from oracle.kvcache import round_fp16
from workloads import (varlen_case, varlen_lengths, decode_case, rotary_tables, dense_case,
                       cfg4, cfg5)

F64 = torch.float64


# ------------------------------------------------------------- varlen ----
def test_varlen_equal_lengths_equals_dense_batch():
    B, S, H, D = 3, 17, 4, 8
    c = dense_case(B, S, S, H, 2, D, "bf16", seed=21, causal=True, alibi=True)
    cu = torch.arange(0, (B + 1) * S, S, dtype=torch.int32)
    q, k, v, do = (t.reshape(B * S, *t.shape[2:]) for t in (c.q, c.k, c.v, c.dout))
    o, l = varlen_fwd(q, k, v, cu, cu, c.scale, True, (-1, -1), 0.0, c.alibi_slopes)
    ro, rl = attention_fwd(c.q, c.k, c.v, c.scale, True, (-1, -1), 0.0, c.alibi_slopes)
    np.testing.assert_allclose(o, ro.reshape(B * S, H, D), atol=0)
    np.testing.assert_allclose(l, rl.transpose(1, 0, 2).reshape(H, B * S), atol=0)
    g = varlen_bwd(q, k, v, do, cu, cu, c.scale, True, (-1, -1), 0.0, c.alibi_slopes)
    rg = attention_bwd(c.q, c.k, c.v, c.dout, c.scale, True, (-1, -1), 0.0, c.alibi_slopes)
    for a, b in zip(g, rg):
        np.testing.assert_allclose(a, b.reshape(a.shape), atol=1e-14)


def test_varlen_isolation_and_empty_sequences():
    lens = [5, 0, 12, 1, 9]
    c = varlen_case(lens, Hq=4, Hkv=2, D=8, seed=22, causal=True)
    o1, l1 = varlen_fwd(c.q, c.k, c.v, c.cu_seqlens_q, c.cu_seqlens_k, c.scale, True)
    # perturb sequence 2 only
    a, b = int(c.cu_seqlens_q[2]), int(c.cu_seqlens_q[3])
    q2, k2 = c.q.clone(), c.k.clone()
    q2[a:b] = -q2[a:b]
    k2[a:b] = k2[a:b] * 2
    o2, l2 = varlen_fwd(q2, k2, c.v, c.cu_seqlens_q, c.cu_seqlens_k, c.scale, True)
    keep = np.r_[0:a, b:o1.shape[0]]
    np.testing.assert_array_equal(o1[keep], o2[keep])
    np.testing.assert_array_equal(l1[:, keep], l2[:, keep])
    assert not np.allclose(o1[a:b], o2[a:b])
    # a length-1 causal sequence returns its own value row
    s3 = int(c.cu_seqlens_q[3])
    np.testing.assert_allclose(o1[s3], c.v.to(F64).numpy()[s3].repeat(2, axis=0), atol=0)


def test_varlen_length_recipe():
    lens = varlen_lengths(32768, 128, 4096, seed=4)
    assert sum(lens) == 32768
    assert all(128 <= L <= 4096 for L in lens[:-1]) and 0 < lens[-1] <= 4096
    # numpy default_rng(4) draw (the check value recorded with the recipe)
    assert lens == [3011, 3870, 3626, 2157, 3860, 4002, 3979, 448, 1928, 2538, 1251, 1622, 476]
    c = cfg4()
    assert c.cu_seqlens_q.dtype == torch.int32 and int(c.cu_seqlens_q[-1]) == 32768
    assert c.max_seqlen_q == 4002


# ------------------------------------------------------------- rotary ----
def test_rotary_tables_and_rotation():
    cos, sin = rotary_tables(64, 16)
    assert cos.dtype == torch.float32 and cos.shape == (64, 8)
    np.testing.assert_array_equal(cos[0].numpy(), 1.0)
    np.testing.assert_array_equal(sin[0].numpy(), 0.0)
    # angle(pos, i) = pos * 10000^(-2i/16)
    assert float(cos[3, 2]) == pytest.approx(math.cos(3 * 10000 ** (-4 / 16)), abs=1e-7)
    x = np.random.default_rng(1).standard_normal((5, 16))
    # position 0 is the identity
    np.testing.assert_array_equal(rotary_apply(x, cos[0].numpy(), sin[0].numpy(), 16), x)
    # a quarter turn maps the pair (a, b) to (-b, a); dims past rotary_dim untouched
    y = rotary_apply(x, np.zeros(4), np.ones(4), 8)
    np.testing.assert_array_equal(y[:, :4], -x[:, 4:8])
    np.testing.assert_array_equal(y[:, 4:8], x[:, :4])
    np.testing.assert_array_equal(y[:, 8:], x[:, 8:])


def test_rotary_preserves_pair_norms_and_is_relative():
    D, r = 16, 16
    half = r // 2
    inv = 10000.0 ** (-np.arange(half) * 2.0 / r)
    ang = lambda p: p * inv  # noqa: E731
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    for p in (0, 3, 100):
        qr = rotary_apply(q, np.cos(ang(p)), np.sin(ang(p)), r)
        np.testing.assert_allclose(qr[:half] ** 2 + qr[half:] ** 2, q[:half] ** 2 + q[half:] ** 2, atol=1e-12)
    dots = []
    for m, n in ((7, 3), (27, 23), (1007, 1003)):
        qm = rotary_apply(q, np.cos(ang(m)), np.sin(ang(m)), r)
        kn = rotary_apply(k, np.cos(ang(n)), np.sin(ang(n)), r)
        dots.append(qm @ kn)
    np.testing.assert_allclose(dots, dots[0], atol=1e-10)


def test_round_bf16_matches_torch():
    rng = np.random.default_rng(3)
    x32 = (rng.standard_normal(20000) * np.exp(rng.uniform(-10, 10, 20000))).astype(np.float32)
    # exact ties in float32: 1 + 2^-8 -> 1 (even), 1 + 3*2^-8 -> 1 + 2^-6
    x32 = np.concatenate([x32, np.float32([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8)])])
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(F64).numpy()
    np.testing.assert_array_equal(round_bf16(x32.astype(np.float64)), ref)
    assert round_bf16(1 + 2 ** -8) == 1.0 and round_bf16(1 + 3 * 2 ** -8) == 1 + 2 ** -6


def _all_finite(kind):
    """Every finite value of a 16-bit format, ascending, as float64 (the
    65536 bit patterns decoded by numpy / torch, NaNs and infinities dropped)."""
    bits = np.arange(1 << 16, dtype=np.uint16)
    if kind == "fp16":
        vals = bits.view(np.float16).astype(np.float64)
    else:
        vals = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(F64).numpy()
    vals = np.unique(vals[np.isfinite(vals)])  # +0 and -0 merge
    return vals


@pytest.mark.parametrize("kind", ["fp16", "bf16"])
def test_round16_exhaustive_ties_and_neighbours(kind):
    """Round-to-nearest-even against the format itself: every finite value is
    kept; every midpoint of two neighbours goes to the one with an even last
    significand bit; a float64 step either side of the midpoint goes to the
    nearer neighbour (a rounder that passed through float32 first would send
    those to the even one); past the largest value by half an ulp is inf."""
    rnd = round_fp16 if kind == "fp16" else round_bf16
    vals = _all_finite(kind)
    np.testing.assert_array_equal(rnd(vals), vals)
    a, b = vals[:-1], vals[1:]
    mid = (a + b) / 2.0  # exact: one more bit than the format
    # the neighbour whose last significand bit is 0
    bits_a = (np.asarray(a, np.float16).view(np.uint16) if kind == "fp16"
              else torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16))
    even = np.where((bits_a & 1) == 0, a, b)
    np.testing.assert_array_equal(rnd(mid), even)
    np.testing.assert_array_equal(rnd(np.nextafter(mid, -np.inf)), a)
    np.testing.assert_array_equal(rnd(np.nextafter(mid, np.inf)), b)
    top = vals[-1]
    half_ulp = (top - vals[-2]) / 2.0
    assert rnd(top + half_ulp) == np.inf and rnd(np.nextafter(top + half_ulp, 0.0)) == top
    assert rnd(-(top + half_ulp)) == -np.inf
    assert np.isnan(rnd(np.nan)) and rnd(np.inf) == np.inf


def test_round_fp16_matches_torch():
    """float32 inputs (one rounding in torch's float32 -> float16 cast), over
    the normal and subnormal range of binary16, with exact float32 ties."""
    rng = np.random.default_rng(5)
    x32 = (rng.standard_normal(40000) * np.exp2(rng.uniform(-27, 17, 40000))).astype(np.float32)
    ties = np.float32([1 + 2 ** -11, 1 + 3 * 2 ** -11, 2 ** -25, 3 * 2 ** -25, -(1 + 2 ** -11), 65520.0, 65519.0])
    x32 = np.concatenate([x32, ties])
    ref = torch.from_numpy(x32).to(torch.float16).to(F64).numpy()
    np.testing.assert_array_equal(round_fp16(x32.astype(np.float64)), ref)
    assert round_fp16(1 + 2 ** -11) == 1.0 and round_fp16(1 + 3 * 2 ** -11) == 1 + 2 ** -9
    assert round_fp16(2 ** -25) == 0.0 and round_fp16(3 * 2 ** -25) == 2 ** -23


# ------------------------------------------------------------ kvcache ----
def _sdpa_rows(q, K, V, scale):
    """torch float64 SDPA of (Sq, H, D) queries over full (L, H, D) keys."""
    qt = torch.as_tensor(q).permute(1, 0, 2)[None]
    kt = torch.as_tensor(K).permute(1, 0, 2)[None]
    vt = torch.as_tensor(V).permute(1, 0, 2)[None]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)[0].permute(1, 0, 2).numpy()


def test_kvcache_no_rotary_equals_sdpa_and_last_prefill_row():
    c = decode_case(B=3, Hq=4, Hkv=2, D=16, page=8, seqlens=[5, 17, 8], seed=31, rotary_dim=0)
    r = kvcache_fwd(c.q, c.k_new, c.v_new, c.k_cache, c.v_cache, c.cache_seqlens, c.block_table,
                    c.page_size, None, None, 0, c.scale)
    for b, L in enumerate([5, 17, 8]):
        K = np.concatenate([gather_logical_cache(c.k_cache, b, L, c.block_table, 8),
                            c.k_new[b].to(F64).numpy()])
        V = np.concatenate([gather_logical_cache(c.v_cache, b, L, c.block_table, 8),
                            c.v_new[b].to(F64).numpy()])
        ref = _sdpa_rows(c.q[b].to(F64).numpy(), K.repeat(2, axis=1), V.repeat(2, axis=1), c.scale)
        np.testing.assert_allclose(r["out"][b], ref, atol=1e-13)
        # the same query as the last row of a causal prefill over L + 1 tokens
        qfull = np.concatenate([np.zeros((L, 4, 16)), c.q[b].to(F64).numpy()])
        o, _ = attention_fwd(qfull[None], K[None], V[None], c.scale, causal=True)
        np.testing.assert_allclose(r["out"][b], o[0, -1:], atol=1e-13)
        # without rotary the appended key is k_new itself
        np.testing.assert_array_equal(r["k_app"][b], c.k_new[b].to(F64).numpy())


def test_kvcache_block_table_permutation_and_contiguous():
    kw = dict(B=2, Hq=4, Hkv=1, D=8, page=4, seqlens=[6, 11], rotary_dim=8)
    c = decode_case(seed=32, **kw)
    r1 = kvcache_fwd(c.q, c.k_new, c.v_new, c.k_cache, c.v_cache, c.cache_seqlens, c.block_table,
                     c.page_size, c.rotary_cos, c.rotary_sin, 8, c.scale)
    # move every page to a new physical index; the logical cache is unchanged
    n = c.k_cache.shape[0]
    perm = np.random.default_rng(5).permutation(n)
    inv = np.argsort(perm)
    k2, v2 = c.k_cache[torch.from_numpy(perm)], c.v_cache[torch.from_numpy(perm)]
    bt2 = c.block_table.clone()
    live = bt2 >= 0
    bt2[live] = torch.from_numpy(inv[bt2[live].numpy()]).to(torch.int32)
    r2 = kvcache_fwd(c.q, c.k_new, c.v_new, k2, v2, c.cache_seqlens, bt2, c.page_size,
                     c.rotary_cos, c.rotary_sin, 8, c.scale)
    np.testing.assert_array_equal(r1["out"], r2["out"])
    # contiguous layout with the same logical contents
    cap = 12
    kc = torch.zeros(2, cap, 1, 8, dtype=c.k_cache.dtype)
    vc = torch.zeros_like(kc)
    for b, L in enumerate([6, 11]):
        kc[b, :L] = torch.from_numpy(gather_logical_cache(c.k_cache, b, L, c.block_table, 4)).to(kc.dtype)
        vc[b, :L] = torch.from_numpy(gather_logical_cache(c.v_cache, b, L, c.block_table, 4)).to(kc.dtype)
    r3 = kvcache_fwd(c.q, c.k_new, c.v_new, kc, vc, c.cache_seqlens, None, None,
                     c.rotary_cos, c.rotary_sin, 8, c.scale)
    np.testing.assert_array_equal(r1["out"], r3["out"])
    assert [s[2] for s in r3["slots"]] == [(0, 6), (1, 11)]


def test_kvcache_rotary_is_applied_at_position():
    # with q and k rotated at the same position and a single cached key at
    # position 0 that is rotated by the caller, the logits follow R(m)q.R(n)k
    c = decode_case(B=1, Hq=1, Hkv=1, D=8, page=4, seqlens=[3], seed=33, rotary_dim=8)
    r = kvcache_fwd(c.q, c.k_new, c.v_new, c.k_cache, c.v_cache, c.cache_seqlens, c.block_table,
                    4, c.rotary_cos, c.rotary_sin, 8, c.scale)
    cos, sin = c.rotary_cos.double().numpy(), c.rotary_sin.double().numpy()
    q = c.q[0, 0, 0].double().numpy()
    kn = c.k_new[0, 0, 0].double().numpy()
    qr = rotary_apply(q, cos[3], sin[3], 8)
    kr = rotary_apply(kn, cos[3], sin[3], 8)
    np.testing.assert_allclose(r["k_app"][0, 0, 0], round_bf16(kr), atol=0)
    K = np.concatenate([gather_logical_cache(c.k_cache, 0, 3, c.block_table, 4)[:, 0], r["k_app"][0, :, 0]])
    s = c.scale * K @ qr
    lse = s.max() + math.log(np.exp(s - s.max()).sum())
    assert r["lse"][0, 0, 0] == pytest.approx(lse, abs=1e-13)
    # the query rotation at its own position cancels against the new key's
    # (up to the float32 rounding of the caller's cos/sin tables)
    assert c.scale * (qr @ kr) == pytest.approx(c.scale * (q @ kn), abs=1e-6)


def test_split_partition_and_merge_equals_unsplit():
    # partial (O_s, LSE_s) over contiguous key ranges merged with
    # M = max LSE_s, LSE = M + ln sum e^(LSE_s - M), O = sum e^(LSE_s - LSE) O_s
    c = dense_case(1, 1, 300, 4, 4, 16, "bf16", seed=34)
    o, l = attention_fwd(c.q, c.k, c.v, c.scale)
    for n_split in (1, 4, 16, 37):
        per = -(-300 // n_split)
        Os, Ls = [], []
        for s in range(n_split):
            a, b = s * per, min(300, (s + 1) * per)
            if a >= b:
                Os.append(np.zeros((1, 1, 4, 16)))
                Ls.append(np.full((1, 4, 1), -np.inf))
                continue
            oo, ll = attention_fwd(c.q, c.k[:, a:b], c.v[:, a:b], c.scale)
            Os.append(oo)
            Ls.append(ll)
        Ls = np.stack(Ls)
        M = Ls.max(axis=0)
        lse = M + np.log(np.exp(Ls - M).sum(axis=0))
        out = sum(np.exp(Ls[s] - lse).transpose(0, 2, 1)[..., None] * Os[s] for s in range(n_split))
        np.testing.assert_allclose(lse, l, atol=1e-13)
        np.testing.assert_allclose(out, o, atol=1e-13)


def test_decode_recipe():
    c = cfg5()
    L = c.cache_seqlens.numpy().tolist()
    assert L == [44298, 52957, 2485, 53146, 31271, 34269, 41682, 19461]
    assert c.k_cache.shape == (1096, 256, 8, 128) and c.block_table.shape == (8, 257)
    bt = c.block_table.numpy()
    live = np.concatenate([bt[b, :(L[b] + 256) // 256] for b in range(8)])
    assert sorted(live.tolist()) == list(range(1096))
    # poison sits past every live length
    b = 2
    p, s = bt[b, L[b] // 256], L[b] % 256
    assert abs(float(c.k_cache[p, s, 0, 0])) == pytest.approx(1e4, rel=1e-2)
    assert abs(float(c.k_cache[bt[b, 0], 0, 0, 0])) < 10
