"""Outputs placed inside larger buffers: nothing outside each output view is
written (backward, padded head dim 96, packed layouts, FP8 workspace, decode
partials).  Each view sits 2048 elements into a buffer filled with 7."""
import pytest
import torch

import io_aware_exact_qk_amd as fa
from workloads import dense_case, decode_case
from _helpers import DEV, say

pytestmark = pytest.mark.gpu
PAD = 2048


def _guarded(shape, dtype):
    n = 1
    for s in shape:
        n *= s
    big = torch.full((n + 2 * PAD,), 7.0, device=DEV, dtype=dtype)
    return big, big[PAD:PAD + n].view(shape)


def _untouched(big, n):
    return bool((big[:PAD] == 7).all()) and bool((big[PAD + n:] == 7).all())


@pytest.mark.parametrize("D", [96, 128])
def test_bwd_guard_bands(D):
    c = dense_case(1, 150, 150, 4, 2, D, "bf16", seed=7, causal=True)
    q, k, v, do = (t.to(DEV) for t in (c.q, c.k, c.v, c.dout))
    say("bwd guard bands", D)
    ob, out = _guarded(q.shape, q.dtype)
    lb, lse = _guarded((1, 4, 150), torch.float32)
    fa.fa_fwd(q, k, v, out=out, lse=lse, scale=c.scale, causal=True)
    bufs = [_guarded(t.shape, t.dtype) for t in (q, k, v)]
    fa.fa_bwd(q, k, v, out, do, lse, dq=bufs[0][1], dk=bufs[1][1], dv=bufs[2][1], scale=c.scale, causal=True)
    torch.cuda.synchronize()
    assert _untouched(ob, out.numel()) and _untouched(lb, lse.numel())
    for big, view in bufs:
        assert _untouched(big, view.numel())


def test_packed_guard_bands():
    c = dense_case(1, 130, 130, 2, 2, 96, "bf16", seed=8, causal=False)
    q, k, v, do = (t.to(DEV) for t in (c.q, c.k, c.v, c.dout))
    qkv = torch.stack([q, k, v], dim=2).contiguous()
    say("qkvpacked guard bands")
    ob, out = _guarded(q.shape, q.dtype)
    lb, lse = _guarded((1, 2, 130), torch.float32)
    fa.fa_fwd_qkvpacked(qkv, out=out, lse=lse, scale=c.scale)
    gb, dqkv = _guarded(qkv.shape, qkv.dtype)
    fa.fa_bwd_qkvpacked(qkv, out, do, lse, dqkv=dqkv, scale=c.scale)
    torch.cuda.synchronize()
    assert _untouched(ob, out.numel()) and _untouched(lb, lse.numel()) and _untouched(gb, dqkv.numel())


def test_fp8_workspace_guard_bands():
    c = dense_case(1, 100, 100, 2, 2, 128, "bf16", seed=9, with_dout=False)
    f8 = [t.float().to(torch.float8_e4m3fn).to(DEV) for t in (c.q, c.k, c.v)]
    n = fa.lib().fa_fwd_fp8_workspace_size(1, 100, 2, 128)
    wb = torch.full((n + 2 * PAD,), 7, device=DEV, dtype=torch.uint8)
    ws = wb[PAD:PAD + n]
    say("fp8 workspace guard bands")
    fa.fa_fwd_fp8(*f8, scale=c.scale, workspace=ws)
    torch.cuda.synchronize()
    assert (wb[:PAD] == 7).all() and (wb[PAD + n:] == 7).all()


@pytest.mark.parametrize("D,T", [(96, 1), (128, 3)])
def test_decode_guard_bands(D, T):
    c = decode_case(B=2, Hq=8, Hkv=2, D=D, page=64, seqlens=[200, 70], seed=61, rotary_dim=32, sq_new=T)
    say("decode guard bands", D, T)
    ob, out = _guarded(c.q.shape, c.q.dtype)
    lb, lse = _guarded((2, 8, T), torch.float32)
    n = fa.lib().fa_kvcache_workspace_size(2, T, 8, D, 3)
    wb = torch.full((n + 2 * PAD,), 7, device=DEV, dtype=torch.uint8)
    fa.fa_fwd_kvcache(c.q.to(DEV), c.k_cache.to(DEV), c.v_cache.to(DEV), c.cache_seqlens.to(DEV),
                      c.k_new.to(DEV), c.v_new.to(DEV), c.block_table.to(DEV), c.rotary_cos.to(DEV),
                      c.rotary_sin.to(DEV), 32, num_splits=3, out=out, lse=lse, scale=c.scale,
                      workspace=wb[PAD:PAD + n])
    torch.cuda.synchronize()
    assert _untouched(ob, out.numel()) and _untouched(lb, lse.numel())
    assert (wb[:PAD] == 7).all() and (wb[PAD + n:] == 7).all()
