"""GPU parity of the dropout entry points against the float64 oracle.

Besides the output / gradient tolerances, the keep mask itself is read back
exactly: with q = 0 every weight is 1/Sk, so V = identity makes each output
element keep * scale / Sk (the forward's query-major mask), and dO =
identity does the same for dV (the dK/dV kernel's key-major mask).  Those
must equal the oracle's mask bit for bit.
"""
import numpy as np
import pytest
import torch

import io_aware_exact_qk_amd as fa
from oracle import attention_fwd, attention_bwd, varlen_fwd, varlen_bwd
from oracle.dropout import keep_mask, keep_scale
from workloads import dense_case, varlen_case
from _helpers import DEV, assert_lse, assert_grad, assert_out_rounded, say, visible_dense, visible_varlen

pytestmark = pytest.mark.gpu


DROP = [
    # B, Sq, Sk, Hq, Hkv, D, dtype, causal, window, softcap, alibi, p
    (2, 200, 200, 4, 4, 128, "bf16", False, (-1, -1), 0.0, False, 0.1),
    (1, 333, 333, 4, 2, 128, "bf16", True, (-1, -1), 0.0, False, 0.2),
    (2, 130, 257, 8, 2, 64, "bf16", True, (-1, -1), 0.0, False, 0.5),
    (1, 257, 257, 4, 1, 128, "bf16", True, (64, 0), 30.0, True, 0.1),
    (2, 129, 129, 3, 3, 64, "fp16", False, (-1, -1), 5.0, False, 0.3),
    (1, 190, 180, 2, 2, 128, "fp16", False, (17, 33), 0.0, True, 0.15),
]


def _kw(c):
    al = None if c.alibi_slopes is None else c.alibi_slopes.to(DEV)
    return dict(scale=c.scale, causal=c.causal, window=c.window, softcap=c.softcap, alibi_slopes=al)


@pytest.mark.parametrize("case", DROP, ids=[f"d{i}" for i in range(len(DROP))])
def test_dropout_fwd_bwd(case):
    B, Sq, Sk, Hq, Hkv, D, dt, causal, window, softcap, alibi, p = case
    c = dense_case(B, Sq, Sk, Hq, Hkv, D, dt, seed=600 + Sq, causal=causal, window=window,
                   softcap=softcap, alibi=alibi)
    seed, off = 0x5EED0000ABCD + Sq, 17
    say("dropout", case)
    q, k, v, do = (t.to(DEV) for t in (c.q, c.k, c.v, c.dout))
    out, lse = fa.fa_fwd_dropout(q, k, v, p, seed, off, **_kw(c))
    dq, dk, dv = fa.fa_bwd_dropout(q, k, v, out, do, lse, p, seed, off, **_kw(c))
    torch.cuda.synchronize()
    drop = (p, seed, off)
    ro, rl = attention_fwd(c.q, c.k, c.v, c.scale, causal, window, softcap, c.alibi_slopes, dropout=drop)
    assert_out_rounded(out, ro, c.q.dtype, visible_dense(Sq, Sk, causal, window))
    assert_lse(lse, rl)
    gq, gk, gv = attention_bwd(c.q, c.k, c.v, c.dout, c.scale, causal, window, softcap, c.alibi_slopes,
                               dropout=drop)
    assert_grad(dq, gq, "dq")
    assert_grad(dk, gk, "dk")
    assert_grad(dv, gv, "dv")


@pytest.mark.parametrize("D,Sq,dt", [(128, 256, "bf16"), (64, 200, "fp16")])
def test_keep_mask_readout_bit_exact(D, Sq, dt):
    """Forward mask (query-major) and dK/dV mask (key-major) equal the oracle's."""
    Sk = D
    B, Hq = 2, 3
    p, seed, off = 0.25, 0x0123456789ABCDEF, 5
    dtype = torch.bfloat16 if dt == "bf16" else torch.float16
    q = torch.zeros(B, Sq, Hq, D, dtype=dtype, device=DEV)
    k = torch.randn(B, Sk, Hq, D, generator=torch.Generator().manual_seed(7)).to(dtype).to(DEV)
    eye = torch.eye(D, dtype=dtype, device=DEV)
    v = eye[None, :, None, :].expand(B, Sk, Hq, D).contiguous()
    say("dropout mask readout", D, Sq, dt)
    out, lse = fa.fa_fwd_dropout(q, k, v, p, seed, off, scale=0.1)
    # dO_i = e_(i mod D): dV[j, d] sums keep_ij * scale / Sk over rows i = d (mod D)
    rows = torch.arange(Sq, device=DEV) % D
    do = eye[rows][None, :, None, :].expand(B, Sq, Hq, D).contiguous()
    _, _, dv = fa.fa_bwd_dropout(q, k, v, out, do, lse, p, seed, off, scale=0.1)
    torch.cuda.synchronize()
    unit = keep_scale(p) / Sk
    o = out.float().cpu().numpy()
    dvn = dv.float().cpu().numpy()
    for b in range(B):
        for h in range(Hq):
            want = keep_mask(p, seed, off, b * Hq + h, np.arange(Sq), np.arange(Sk))
            got = o[b, :, h, :] > 0.5 * unit
            assert (got == want).all(), f"forward mask differs at b={b} h={h}: {(got != want).sum()} pairs"
            # dV[j, d] = unit * #{i = d mod D : keep_ij}; recover it per row block of D
            cnt = np.rint(dvn[b, :, h, :] / unit).astype(np.int64)
            ref = np.zeros((Sk, D), np.int64)
            for i in range(Sq):
                ref[:, i % D] += want[i, :]
            assert (cnt == ref).all(), f"dK/dV mask differs at b={b} h={h}"


def test_dropout_deterministic_and_seeded():
    c = dense_case(1, 300, 300, 4, 2, 128, "bf16", seed=71, causal=True)
    q, k, v, do = (t.to(DEV) for t in (c.q, c.k, c.v, c.dout))
    say("dropout repeatability")
    runs = []
    for off in (3, 3, 4):
        out, lse = fa.fa_fwd_dropout(q, k, v, 0.2, 99, off, scale=c.scale, causal=True)
        g = fa.fa_bwd_dropout(q, k, v, out, do, lse, 0.2, 99, off, scale=c.scale, causal=True)
        torch.cuda.synchronize()
        runs.append([out.clone()] + [x.clone() for x in g])
    for a, b in zip(runs[0], runs[1]):
        assert torch.equal(a, b)
    assert not torch.equal(runs[0][0], runs[2][0])


def test_dropout_zero_matches_plain_bitwise():
    c = dense_case(2, 150, 150, 4, 4, 64, "bf16", seed=72, causal=True)
    q, k, v, do = (t.to(DEV) for t in (c.q, c.k, c.v, c.dout))
    say("dropout p=0")
    o1, l1 = fa.fa_fwd(q, k, v, scale=c.scale, causal=True)
    o2, l2 = fa.fa_fwd_dropout(q, k, v, 0.0, 5, 0, scale=c.scale, causal=True)
    g1 = fa.fa_bwd(q, k, v, o1, do, l1, scale=c.scale, causal=True)
    g2 = fa.fa_bwd_dropout(q, k, v, o2, do, l2, 0.0, 5, 0, scale=c.scale, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_dropout_varlen():
    c = varlen_case([300, 77, 1, 190], Hq=4, Hkv=2, D=128, seed=73, causal=True)
    seed, off, p = 1234567, 2, 0.2
    q, k, v, do = (t.to(DEV) for t in (c.q, c.k, c.v, c.dout))
    cq, ck = c.cu_seqlens_q.to(DEV), c.cu_seqlens_k.to(DEV)
    say("dropout varlen")
    out, lse = fa.fa_fwd_varlen_dropout(q, k, v, cq, ck, c.max_seqlen_q, c.max_seqlen_k, p, seed, off,
                                        scale=c.scale, causal=True)
    dq, dk, dv = fa.fa_bwd_varlen_dropout(q, k, v, out, do, lse, cq, ck, c.max_seqlen_q, c.max_seqlen_k, p, seed, off,
                                          scale=c.scale, causal=True)
    torch.cuda.synchronize()
    drop = (p, seed, off)
    ro, rl = varlen_fwd(c.q, c.k, c.v, c.cu_seqlens_q, c.cu_seqlens_k, c.scale, True, dropout=drop)
    assert_out_rounded(out, ro, c.q.dtype, visible_varlen(c.cu_seqlens_q, c.cu_seqlens_k, True))
    assert_lse(lse, rl)
    gq, gk, gv = varlen_bwd(c.q, c.k, c.v, c.dout, c.cu_seqlens_q, c.cu_seqlens_k, c.scale, True, dropout=drop)
    assert_grad(dq, gq, "dq")
    assert_grad(dk, gk, "dk")
    assert_grad(dv, gv, "dv")
