"""Packed layouts (qkv (B,S,3,H,D), kv (B,Sk,2,Hkv,D)): the packed entry
points run the same kernels with packed row strides, so their results must
equal the unpacked calls bit for bit, and the oracle within tolerance."""
import pytest
import torch

import io_aware_exact_qk_amd as fa
from oracle import attention_fwd, attention_bwd
from workloads import dense_case
from _helpers import DEV, assert_out, assert_lse, assert_grad, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("S,H,D,dt,causal,window,softcap,alibi", [
    (200, 4, 128, "bf16", True, (-1, -1), 0.0, False),
    (333, 2, 64, "fp16", False, (40, 7), 10.0, True),
])
def test_qkvpacked(S, H, D, dt, causal, window, softcap, alibi):
    c = dense_case(2, S, S, H, H, D, dt, seed=800 + S, causal=causal, window=window, softcap=softcap,
                   alibi=alibi)
    say("qkvpacked", S, H, D, dt)
    q, k, v, do = (t.to(DEV) for t in (c.q, c.k, c.v, c.dout))
    qkv = torch.stack([q, k, v], dim=2).contiguous()
    al = None if c.alibi_slopes is None else c.alibi_slopes.to(DEV)
    kw = dict(scale=c.scale, causal=causal, window=window, softcap=softcap, alibi_slopes=al)
    out_p, lse_p = fa.fa_fwd_qkvpacked(qkv, **kw)
    dqkv = fa.fa_bwd_qkvpacked(qkv, out_p, do, lse_p, **kw)
    out, lse = fa.fa_fwd(q, k, v, **kw)
    dq, dk, dv = fa.fa_bwd(q, k, v, out, do, lse, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out_p, out) and torch.equal(lse_p, lse)
    assert torch.equal(dqkv[:, :, 0], dq) and torch.equal(dqkv[:, :, 1], dk) and torch.equal(dqkv[:, :, 2], dv)
    ro, rl = attention_fwd(c.q, c.k, c.v, c.scale, causal, window, softcap, c.alibi_slopes)
    assert_out(out_p, ro, c.q.dtype)
    assert_lse(lse_p, rl)
    gq, gk, gv = attention_bwd(c.q, c.k, c.v, c.dout, c.scale, causal, window, softcap, c.alibi_slopes)
    assert_grad(dqkv[:, :, 0], gq, "dq")
    assert_grad(dqkv[:, :, 1], gk, "dk")
    assert_grad(dqkv[:, :, 2], gv, "dv")


@pytest.mark.parametrize("Sq,Sk,Hq,Hkv,D,causal", [(150, 300, 8, 2, 128, True), (97, 97, 4, 4, 64, False)])
def test_kvpacked(Sq, Sk, Hq, Hkv, D, causal):
    c = dense_case(1, Sq, Sk, Hq, Hkv, D, "bf16", seed=900 + Sq, causal=causal)
    say("kvpacked", Sq, Sk, Hq, Hkv, D)
    q, k, v, do = (t.to(DEV) for t in (c.q, c.k, c.v, c.dout))
    kv = torch.stack([k, v], dim=2).contiguous()
    kw = dict(scale=c.scale, causal=causal)
    out_p, lse_p = fa.fa_fwd_kvpacked(q, kv, **kw)
    dq_p, dkv = fa.fa_bwd_kvpacked(q, kv, out_p, do, lse_p, **kw)
    out, lse = fa.fa_fwd(q, k, v, **kw)
    dq, dk, dv = fa.fa_bwd(q, k, v, out, do, lse, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out_p, out) and torch.equal(lse_p, lse)
    assert torch.equal(dq_p, dq) and torch.equal(dkv[:, :, 0], dk) and torch.equal(dkv[:, :, 1], dv)
    gq, gk, gv = attention_bwd(c.q, c.k, c.v, c.dout, c.scale, causal)
    assert_grad(dq_p, gq, "dq")
    assert_grad(dkv[:, :, 0], gk, "dk")
    assert_grad(dkv[:, :, 1], gv, "dv")
