"""GPU check of fa_fwd_kvcache_noalloc (the decode entry point without a
workspace argument, for callers that cannot allocate device memory): two
calls in a row, the second smaller, each equal bit for bit to fa_fwd_kvcache
on the same inputs (same kernels; the static scratch replaces the caller's
workspace) and within tolerance of the oracle."""
import numpy as np
import pytest
import torch

import io_aware_exact_qk_amd as fa
from oracle import kvcache_fwd
from workloads import decode_case
from _helpers import DEV, assert_out, assert_lse, say

pytestmark = pytest.mark.gpu


def _inputs(c):
    rot = (c.rotary_cos.to(DEV), c.rotary_sin.to(DEV))
    return dict(q=c.q.to(DEV), kc=c.k_cache.to(DEV), vc=c.v_cache.to(DEV), sl=c.cache_seqlens.to(DEV),
                kn=c.k_new.to(DEV), vn=c.v_new.to(DEV), bt=c.block_table.to(DEV), cos=rot[0], sin=rot[1])


def _call(fn, t, num_splits, scale, rd):
    out = torch.empty_like(t["q"])
    lse = torch.empty(t["q"].shape[0], t["q"].shape[2], t["q"].shape[1], device=DEV)
    fn(t["q"], t["kc"], t["vc"], t["sl"], t["kn"], t["vn"], t["bt"], t["cos"], t["sin"], rd,
       num_splits=num_splits, out=out, lse=lse, scale=scale)
    return out, lse


# (B, Hq, Hkv, D, page, seqlens, num_splits); the second case is smaller
CASES = [
    (4, 32, 8, 128, 256, [9000, 2500, 17000, 4100], 16),
    (2, 8, 2, 64, 64, [500, 70], 3),
]


def test_noalloc_matches_workspace_entry_point_two_calls():
    for i, (B, Hq, Hkv, D, page, lens, splits) in enumerate(CASES):
        c = decode_case(B=B, Hq=Hq, Hkv=Hkv, D=D, page=page, seqlens=lens, seed=90 + i)
        say("noalloc call", i, (B, Hq, Hkv, D, page, lens, splits))
        a, b = _inputs(c), _inputs(c)
        o1, l1 = _call(fa.fa_fwd_kvcache_noalloc, a, splits, c.scale, c.rotary_dim)
        o2, l2 = _call(fa.fa_fwd_kvcache, b, splits, c.scale, c.rotary_dim)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), "noalloc output differs from fa_fwd_kvcache"
        assert torch.equal(a["kc"], b["kc"]) and torch.equal(a["vc"], b["vc"]), "cache append differs"
        ref = kvcache_fwd(c.q, c.k_new, c.v_new, c.k_cache, c.v_cache, c.cache_seqlens, c.block_table,
                          c.page_size, c.rotary_cos, c.rotary_sin, c.rotary_dim, c.scale)
        assert_out(o1, ref["out"], c.q.dtype)
        assert_lse(l1, ref["lse"])


def test_noalloc_automatic_splits_and_limit():
    c = decode_case(B=3, Hq=16, Hkv=4, D=128, page=128, seqlens=[3000, 40, 1200], seed=95)
    say("noalloc automatic splits")
    a, b = _inputs(c), _inputs(c)
    o1, l1 = _call(fa.fa_fwd_kvcache_noalloc, a, 0, c.scale, c.rotary_dim)
    o2, l2 = _call(fa.fa_fwd_kvcache, b, 0, c.scale, c.rotary_dim)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # beyond the static scratch: refused before any launch, nothing written
    q = torch.zeros(64, 1, 64, 128, dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros(64, 256, 8, 128, dtype=torch.bfloat16, device=DEV)
    sl = torch.ones(64, dtype=torch.int32, device=DEV)
    bt = torch.arange(64, dtype=torch.int32, device=DEV).reshape(64, 1)
    out = torch.full_like(q, 3.0)
    with pytest.raises(fa.FAError) as e:
        fa.fa_fwd_kvcache_noalloc(q, kc, kc, sl, block_table=bt, num_splits=32, out=out)
    assert e.value.status == 5
    torch.cuda.synchronize()
    assert (out == 3.0).all()
