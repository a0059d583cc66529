"""GPU parity of fa_bwd against the float64 oracle (runs on an MI355X)."""
import numpy as np
import pytest
import torch

import io_aware_exact_qk_amd as fa
from oracle import attention_fwd, attention_bwd
from workloads import dense_case, cfg2, cfg3
from _helpers import DEV, assert_grad, say

pytestmark = pytest.mark.gpu


def _run(c, deterministic=False):
    q, k, v, do = (t.to(DEV) for t in (c.q, c.k, c.v, c.dout))
    al = None if c.alibi_slopes is None else c.alibi_slopes.to(DEV)
    kw = dict(scale=c.scale, causal=c.causal, window=c.window, softcap=c.softcap, alibi_slopes=al)
    out, lse = fa.fa_fwd(q, k, v, **kw)
    dq, dk, dv = fa.fa_bwd(q, k, v, out, do, lse, deterministic=deterministic, **kw)
    torch.cuda.synchronize()
    return dq, dk, dv


SMALL = [
    # B, Sq, Sk, Hq, Hkv, D, dtype, causal, window, softcap, alibi
    (2, 200, 200, 4, 4, 128, "bf16", False, (-1, -1), 0.0, False),
    (1, 333, 333, 4, 2, 128, "bf16", True, (-1, -1), 0.0, False),
    (2, 130, 257, 8, 2, 64, "bf16", True, (-1, -1), 0.0, False),
    (1, 300, 100, 2, 1, 128, "bf16", True, (-1, -1), 0.0, False),
    (1, 257, 257, 4, 1, 128, "bf16", True, (64, 0), 30.0, True),
    (1, 190, 190, 2, 2, 64, "bf16", False, (17, 33), 0.0, False),
    (1, 1, 1, 1, 1, 128, "bf16", False, (-1, -1), 0.0, False),
    (2, 129, 129, 3, 3, 64, "fp16", False, (-1, -1), 5.0, False),
    (1, 400, 380, 8, 8, 128, "fp16", False, (100, 7), 0.0, True),
    (1, 64, 1000, 2, 2, 128, "bf16", True, (200, 0), 0.0, False),
    (1, 256, 256, 32, 8, 128, "bf16", True, (96, 0), 30.0, True),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"s{i}" for i in range(len(SMALL))])
def test_small_cases(case):
    B, Sq, Sk, Hq, Hkv, D, dt, causal, window, softcap, alibi = case
    c = dense_case(B, Sq, Sk, Hq, Hkv, D, dt, seed=200 + Sq, causal=causal, window=window,
                   softcap=softcap, alibi=alibi)
    say("bwd small", case)
    dq, dk, dv = _run(c)
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


def _check_sampled(c, heads, q_rows, k_rows, dq, dk, dv):
    args = (c.q, c.k, c.v, c.dout, c.scale, c.causal, c.window, c.softcap, c.alibi_slopes)
    gq, _, _ = attention_bwd(*args, heads=heads, q_rows=q_rows)
    mq = np.zeros(gq.shape, bool)
    for h in heads:
        mq[:, q_rows, h, :] = True
    assert_grad(dq, gq, "dq", mask=mq)
    # dk/dv of the K/V heads of `heads` collect every query head of the group
    Hq, Hkv = c.q.shape[2], c.k.shape[2]
    g = Hq // Hkv
    kv_heads = sorted(set(h // g for h in heads))
    all_q = [hk * g + i for hk in kv_heads for i in range(g)]
    _, gk, gv = attention_bwd(*args, heads=all_q, k_rows=k_rows)
    mk = np.zeros(gk.shape, bool)
    for hk in kv_heads:
        mk[:, k_rows, hk, :] = True
    assert_grad(dk, gk, "dk", mask=mk)
    assert_grad(dv, gv, "dv", mask=mk)


@pytest.mark.parametrize("S", [512, 4096, 16384])
@pytest.mark.parametrize("causal", [False, True])
def test_cfg2_hd128_sampled(S, causal):
    c = cfg2(S, 16, 128, causal)
    say("bwd", c.name)
    dq, dk, dv = _run(c)
    rows = [0, 1, S // 2, S - 1]
    _check_sampled(c, [0, 15], rows, rows, dq, dk, dv)


@pytest.mark.parametrize("S", [1024, 8192])
def test_cfg2_hd64_sampled(S):
    c = cfg2(S, 32, 64, True)
    say("bwd", c.name)
    dq, dk, dv = _run(c)
    rows = [0, 3, S // 2, S - 1]
    _check_sampled(c, [0, 31], rows, rows, dq, dk, dv)


def test_cfg3_sampled():
    c = cfg3()
    say("bwd", c.name)
    dq, dk, dv = _run(c)
    rows = [0, 4095, 4096, 8191]
    _check_sampled(c, [0, 31], rows, [0, 4000, 4096, 8191], dq, dk, dv)


def test_deterministic_bitwise():
    c = dense_case(1, 300, 300, 8, 2, 128, "bf16", seed=9, causal=True, softcap=10.0)
    say("bwd deterministic repeat")
    a = _run(c, deterministic=True)
    b = _run(c, deterministic=True)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
