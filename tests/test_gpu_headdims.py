"""Head dims 32, 96 and 256 (besides 64 and 128): forward and backward parity
with the oracle over the option mixes, varlen, dropout and the packed entry
points, at sizes that span several tiles with ragged tails.  Outputs use the
plain bound except on rows with at most three visible keys and on
|O| >= 2 (_helpers.assert_out_rounded)."""
import numpy as np
import pytest
import torch

import io_aware_exact_qk_amd as fa
from oracle import attention_fwd, attention_bwd, varlen_fwd, varlen_bwd
from workloads import dense_case, varlen_case
from _helpers import DEV, assert_out_rounded, assert_lse, assert_grad, say, visible_dense, visible_varlen

pytestmark = pytest.mark.gpu

CASES = [
    # B, Sq, Sk, Hq, Hkv, D, dtype, causal, window, softcap, alibi
    (2, 200, 200, 4, 4, 256, "bf16", False, (-1, -1), 0.0, False),
    (1, 333, 333, 4, 2, 256, "bf16", True, (-1, -1), 0.0, False),
    (1, 257, 190, 4, 1, 256, "fp16", True, (64, 0), 30.0, True),
    (2, 130, 257, 8, 2, 32, "bf16", True, (-1, -1), 0.0, False),
    (1, 300, 300, 2, 2, 32, "fp16", False, (17, 33), 5.0, True),
    (1, 1, 1, 1, 1, 256, "bf16", False, (-1, -1), 0.0, False),
    (2, 200, 200, 4, 2, 96, "bf16", True, (-1, -1), 0.0, False),
    (1, 257, 190, 4, 4, 96, "fp16", False, (64, 7), 20.0, True),
]


def _kw(c):
    al = None if c.alibi_slopes is None else c.alibi_slopes.to(DEV)
    return dict(scale=c.scale, causal=c.causal, window=c.window, softcap=c.softcap, alibi_slopes=al)


@pytest.mark.parametrize("case", CASES, ids=[f"h{i}" for i in range(len(CASES))])
def test_fwd_bwd(case):
    B, Sq, Sk, Hq, Hkv, D, dt, causal, window, softcap, alibi = case
    c = dense_case(B, Sq, Sk, Hq, Hkv, D, dt, seed=1000 + Sq + D, causal=causal, window=window,
                   softcap=softcap, alibi=alibi)
    say("headdim", case)
    q, k, v, do = (t.to(DEV) for t in (c.q, c.k, c.v, c.dout))
    out, lse = fa.fa_fwd(q, k, v, **_kw(c))
    dq, dk, dv = fa.fa_bwd(q, k, v, out, do, lse, **_kw(c))
    torch.cuda.synchronize()
    ro, rl = attention_fwd(c.q, c.k, c.v, c.scale, causal, window, softcap, c.alibi_slopes)
    assert_out_rounded(out, ro, c.q.dtype, visible_dense(Sq, Sk, causal, window))
    assert_lse(lse, rl)
    gq, gk, gv = attention_bwd(c.q, c.k, c.v, c.dout, c.scale, causal, window, softcap, c.alibi_slopes)
    if Sk == 1:
        # one key: P = 1 and dS = P (dP - delta) cancels exactly, so dq = dk = 0
        # and the relative bound degenerates; float32 leaves only the rounding
        # residue of dP - delta (dP from the MFMA, delta = dO . O summed apart)
        assert np.abs(dq.float().cpu().numpy()).max() <= 1e-5
        assert np.abs(dk.float().cpu().numpy()).max() <= 1e-5
    else:
        assert_grad(dq, gq, "dq")
        assert_grad(dk, gk, "dk")
    assert_grad(dv, gv, "dv")


@pytest.mark.parametrize("D", [32, 96, 256])
def test_varlen(D):
    c = varlen_case([300, 77, 1, 190], Hq=4, Hkv=2, D=D, seed=1100 + D, causal=True)
    q, k, v, do = (t.to(DEV) for t in (c.q, c.k, c.v, c.dout))
    cq, ck = c.cu_seqlens_q.to(DEV), c.cu_seqlens_k.to(DEV)
    say("headdim varlen", D)
    out, lse = fa.fa_fwd_varlen(q, k, v, cq, ck, c.max_seqlen_q, c.max_seqlen_k, scale=c.scale, causal=True)
    dq, dk, dv = fa.fa_bwd_varlen(q, k, v, out, do, lse, cq, ck, c.max_seqlen_q, c.max_seqlen_k,
                                  scale=c.scale, causal=True)
    torch.cuda.synchronize()
    ro, rl = varlen_fwd(c.q, c.k, c.v, c.cu_seqlens_q, c.cu_seqlens_k, c.scale, True)
    assert_out_rounded(out, ro, c.q.dtype, visible_varlen(c.cu_seqlens_q, c.cu_seqlens_k, True))
    assert_lse(lse, rl)
    gq, gk, gv = varlen_bwd(c.q, c.k, c.v, c.dout, c.cu_seqlens_q, c.cu_seqlens_k, c.scale, True)
    assert_grad(dq, gq, "dq")
    assert_grad(dk, gk, "dk")
    assert_grad(dv, gv, "dv")


@pytest.mark.parametrize("D", [32, 96, 256])
def test_dropout_and_packed(D):
    c = dense_case(1, 160, 160, 2, 2, D, "bf16", seed=1200 + D, causal=True)
    q, k, v, do = (t.to(DEV) for t in (c.q, c.k, c.v, c.dout))
    say("headdim dropout/packed", D)
    drop = (0.2, 77, 1)
    out, lse = fa.fa_fwd_dropout(q, k, v, *drop, scale=c.scale, causal=True)
    dq, dk, dv = fa.fa_bwd_dropout(q, k, v, out, do, lse, *drop, scale=c.scale, causal=True)
    qkv = torch.stack([q, k, v], dim=2).contiguous()
    out_p, lse_p = fa.fa_fwd_qkvpacked(qkv, scale=c.scale, causal=True)
    out_u, lse_u = fa.fa_fwd(q, k, v, scale=c.scale, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(out_p, out_u) and torch.equal(lse_p, lse_u)
    ro, rl = attention_fwd(c.q, c.k, c.v, c.scale, True, dropout=drop)
    assert_out_rounded(out, ro, c.q.dtype, visible_dense(160, 160, True))
    assert_lse(lse, rl)
    gq, gk, gv = attention_bwd(c.q, c.k, c.v, c.dout, c.scale, True, dropout=drop)
    assert_grad(dq, gq, "dq")
    assert_grad(dk, gk, "dk")
    assert_grad(dv, gv, "dv")


def test_decode_rejects_unbuilt_head_dims():
    for D in (256,):
        q = torch.zeros(1, 1, 4, D, dtype=torch.bfloat16, device=DEV)
        kc = torch.zeros(1, 64, 4, D, dtype=torch.bfloat16, device=DEV)
        sl = torch.ones(1, dtype=torch.int32, device=DEV)
        with pytest.raises(fa.FAError):
            fa.fa_fwd_kvcache(q, kc, kc.clone(), sl)
