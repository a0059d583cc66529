"""GPU parity of the FP8 forward against the float64 oracle on the
dequantised inputs.  q/k/v are quantised per (batch entry, K/V head) to OCP
e4m3 with factors that map each slice's max |x| to 240; the oracle sees
exactly the fp8 values times their factors (formed in float64)."""
import numpy as np
import pytest
import torch

import io_aware_exact_qk_amd as fa
from oracle import attention_fwd
from workloads import dense_case
from _helpers import DEV, assert_out_rounded, assert_lse, say, visible_dense

pytestmark = pytest.mark.gpu
F8 = torch.float8_e4m3fn


def _quant(x, Hkv):
    """x (B, S, H, D) float -> (fp8 tensor, descale (B, Hkv), dequantised float64)."""
    B, S, H, D = x.shape
    g = H // Hkv
    xf = x.float()
    amax = xf.abs().reshape(B, S, Hkv, g, D).amax(dim=(1, 3, 4)).clamp_min(1e-6)  # (B, Hkv)
    ds = (amax / 240.0).float()
    per_head = ds.repeat_interleave(g, dim=1)[:, None, :, None]
    x8 = (xf / per_head).to(F8)
    deq = x8.double() * per_head.double()
    return x8, ds, deq


CASES = [
    # B, Sq, Sk, Hq, Hkv, D, causal, window, softcap, alibi, with_descale
    (2, 200, 200, 4, 4, 128, False, (-1, -1), 0.0, False, True),
    (1, 333, 333, 8, 2, 128, True, (-1, -1), 0.0, False, True),
    (2, 130, 257, 4, 2, 64, True, (-1, -1), 0.0, False, False),
    (1, 257, 257, 4, 1, 128, True, (64, 0), 30.0, True, True),
    (1, 190, 180, 2, 2, 64, False, (17, 33), 5.0, True, True),
]


@pytest.mark.parametrize("case", CASES, ids=[f"f{i}" for i in range(len(CASES))])
def test_fp8_forward(case):
    B, Sq, Sk, Hq, Hkv, D, causal, window, softcap, alibi, with_ds = case
    c = dense_case(B, Sq, Sk, Hq, Hkv, D, "bf16", seed=1300 + Sq, causal=causal, window=window,
                   softcap=softcap, alibi=alibi, with_dout=False)
    q8, dq, qd = _quant(c.q, Hkv)
    k8, dk, kd = _quant(c.k, Hkv)
    v8, dv, vd = _quant(c.v, Hkv)
    if not with_ds:  # raw fp8 values (factors 1): the inputs are the fp8 values themselves
        q8, k8, v8 = c.q.float().to(F8), c.k.float().to(F8), c.v.float().to(F8)
        qd, kd, vd = q8.double(), k8.double(), v8.double()
        dq = dk = dv = None
    say("fp8 forward", case)
    al = None if c.alibi_slopes is None else c.alibi_slopes.to(DEV)
    ds = [None if x is None else x.to(DEV) for x in (dq, dk, dv)]
    out, lse = fa.fa_fwd_fp8(q8.to(DEV), k8.to(DEV), v8.to(DEV), *ds, scale=c.scale, causal=causal,
                             window=window, softcap=softcap, alibi_slopes=al)
    torch.cuda.synchronize()
    ro, rl = attention_fwd(qd.numpy(), kd.numpy(), vd.numpy(), c.scale, causal, window, softcap,
                           c.alibi_slopes)
    assert_out_rounded(out, ro, torch.bfloat16, visible_dense(Sq, Sk, causal, window))
    assert_lse(lse, rl)


def test_fp8_v_conversion_exact():
    """Every e4m3 byte pattern survives the fp8 -> bfloat16 copy: with q = 0
    and one key per query (causal, Sq = Sk = 1 per batch entry) out = v."""
    vals = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    finite = ~torch.isnan(vals.view(F8).float())
    v8 = vals[finite].view(F8)
    n = v8.numel()
    pad = (-n) % 128
    v8 = torch.cat([v8, torch.zeros(pad, dtype=torch.uint8).view(F8)]).reshape(-1, 1, 1, 128)
    B = v8.shape[0]
    q8 = torch.zeros(B, 1, 1, 128, dtype=torch.uint8).view(F8)
    say("fp8 v conversion")
    out, _ = fa.fa_fwd_fp8(q8.to(DEV), q8.to(DEV), v8.to(DEV), scale=0.1)
    torch.cuda.synchronize()
    assert torch.equal(out.float().cpu(), v8.float())
