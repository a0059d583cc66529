"""Data that lies more than 4 GiB past the base pointer of its tensor.

The tile copies address memory through a buffer resource built per tile from
a 64-bit base with 32-bit offsets inside the tile, so the last batch entry of
a dense batch larger than 4 GiB, and cache pages beyond 4 GiB in a paged pool,
must still match the oracle.  Inputs are drawn on the device from a seeded
generator; the oracle sees copies of exactly the slices it checks.
"""
import numpy as np
import pytest
import torch

import io_aware_exact_qk_amd as fa
from oracle import attention_fwd, attention_bwd, kvcache_fwd
from workloads import decode_case
from _helpers import DEV, assert_out, assert_lse, assert_grad, say

pytestmark = pytest.mark.gpu


def test_dense_last_batch_beyond_4gib():
    B, S, H, D = 520, 2048, 16, 128  # 8 MiB per batch entry: entry 519 starts 4.06 GiB in
    assert (B - 1) * S * H * D * 2 > 1 << 32
    g = torch.Generator(device=DEV).manual_seed(21)
    q, k, v, do = (torch.randn((B, S, H, D), generator=g, device=DEV, dtype=torch.bfloat16) for _ in range(4))
    scale = D ** -0.5
    say("large offsets: dense fwd+bwd causal, B=520 S=2048 H=16 D=128")
    out, lse = fa.fa_fwd(q, k, v, scale=scale, causal=True)
    dq, dk, dv = fa.fa_bwd(q, k, v, out, do, lse, scale=scale, causal=True)
    torch.cuda.synchronize()

    def last(t):
        return t[B - 1:].cpu()

    ql, kl, vl, dol = last(q), last(k), last(v), last(do)
    heads, rows = [0, H - 1], [0, 1, S // 2, S - 1]
    ro, rl = attention_fwd(ql, kl, vl, scale, True, heads=heads, q_rows=rows)
    m_o = np.zeros(ro.shape, bool)
    m_l = np.zeros(rl.shape, bool)
    for h in heads:
        m_o[:, rows, h, :] = True
        m_l[:, h, rows] = True
    assert_out(last(out), ro, torch.bfloat16, mask=m_o)
    assert_lse(lse[B - 1:].cpu(), rl, mask=m_l)

    args = (ql, kl, vl, dol, scale, True)
    gq, _, _ = attention_bwd(*args, heads=heads, q_rows=rows)
    _, gk, gv = attention_bwd(*args, heads=heads, k_rows=rows)
    assert_grad(last(dq), gq, "dq", mask=m_o)
    assert_grad(last(dk), gk, "dk", mask=m_o)
    assert_grad(last(dv), gv, "dv", mask=m_o)
    # the first entry (small offsets) is untouched by the large ones
    assert torch.isfinite(out[0]).all() and torch.isfinite(dq[0]).all()


def test_decode_pages_beyond_4gib():
    c = decode_case(B=2, Hq=8, Hkv=2, D=128, page=256, seqlens=[700, 300], seed=57)
    n_small = c.k_cache.shape[0]
    page_bytes = c.k_cache[0].numel() * 2  # 128 KiB
    n_big = 33000
    base = n_big - n_small  # the case's pages sit at the top of the big pool
    assert base * page_bytes > 1 << 32
    say("large offsets: paged decode, pool of", n_big, "pages, pages from", base)
    kc = torch.empty((n_big,) + tuple(c.k_cache.shape[1:]), dtype=c.k_cache.dtype, device=DEV)
    vc = torch.empty_like(kc)
    kc[base:] = c.k_cache.to(DEV)
    vc[base:] = c.v_cache.to(DEV)
    bt = c.block_table.clone()
    bt[bt >= 0] += base
    ref = kvcache_fwd(c.q, c.k_new, c.v_new, c.k_cache, c.v_cache, c.cache_seqlens, c.block_table,
                      c.page_size, c.rotary_cos, c.rotary_sin, c.rotary_dim, c.scale)
    for ns in (1, 3):
        kc[base:] = c.k_cache.to(DEV)
        vc[base:] = c.v_cache.to(DEV)
        out, lse = fa.fa_fwd_kvcache(c.q.to(DEV), kc, vc, c.cache_seqlens.to(DEV), c.k_new.to(DEV),
                                     c.v_new.to(DEV), bt.to(DEV), c.rotary_cos.to(DEV), c.rotary_sin.to(DEV),
                                     c.rotary_dim, num_splits=ns, scale=c.scale)
        torch.cuda.synchronize()
        assert_out(out, ref["out"], torch.bfloat16, what=f"out (splits {ns})")
        assert_lse(lse, ref["lse"], what=f"lse (splits {ns})")
        # the appended rows landed in the high pages
        for (b, t, (pg, slot)) in ref["slots"]:
            np.testing.assert_array_equal(vc[base + pg, slot].double().cpu().numpy(), ref["v_app"][b, t])
            ka = kc[base + pg, slot].double().cpu().numpy()
            ref_k = ref["k_app"][b, t]
            assert (np.abs(ka - ref_k) <= np.abs(ref_k) * 2.0 ** -7 + 1e-30).all()
