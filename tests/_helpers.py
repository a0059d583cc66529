"""Shared helpers for the GPU parity tests (comparison against the oracle)."""
import sys

import numpy as np
import torch

# Tolerances for N(0,1) inputs with scale 1/sqrt(D): output max-abs error
# 2e-3 (fp16) / 1e-2 (bf16); LSE max-abs 1e-4; each gradient max-abs error
# within 2e-2 of that gradient's max-abs.
TOL_OUT = {torch.float16: 2e-3, torch.bfloat16: 1e-2}
TOL_LSE = 1e-4
TOL_GRAD = 2e-2

DEV = "cuda:0"


def say(*a):
    """Name the case before a GPU step, flushed, so a crash still names it."""
    print(*a, flush=True)
    sys.stdout.flush()


def np64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def max_err(got, ref, mask=None):
    g = np64(got) if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    if mask is not None:
        g, r = g[mask], r[mask]
    both_inf = np.isinf(g) & np.isinf(r) & (np.sign(g) == np.sign(r))
    d = np.where(both_inf, 0.0, np.abs(g - r))
    d = np.where(np.isnan(d), np.inf, d)
    return float(d.max()) if d.size else 0.0


def assert_out(got, ref, dtype, what="out", mask=None):
    e = max_err(got, ref, mask)
    assert e <= TOL_OUT[dtype], f"{what}: max abs err {e:.3e} > {TOL_OUT[dtype]:.1e}"
    return e


def assert_lse(got, ref, what="lse", mask=None):
    e = max_err(got, ref, mask)
    assert e <= TOL_LSE, f"{what}: max abs err {e:.3e} > {TOL_LSE:.1e}"
    return e


def assert_grad(got, ref, what, mask=None):
    r = np.asarray(ref, np.float64)
    rr = r[mask] if mask is not None else r
    scale = float(np.abs(rr[np.isfinite(rr)]).max()) if rr.size else 0.0
    e = max_err(got, ref, mask)
    assert e <= TOL_GRAD * max(scale, 1e-30), f"{what}: max abs err {e:.3e} > {TOL_GRAD} * {scale:.3e}"
    return e


def assert_out_rounded(got, ref, dtype, what="out"):
    """Output tolerance plus half an ulp of the reference value in the output
    dtype, per element.

    Used where rows with one to a few visible keys (O close to a single v)
    or dropout's 1/(1-p) scaling put |O| where rounding the result once to
    16 bits, together with the 16-bit P operand of the PV product, already
    reaches the plain tolerance: e.g. row 1 of a causal D = 256 bf16 case
    gives 1.089e-2 both from the kernel and from the standard arithmetic
    emulated on the CPU (float32 P rounded to bf16, output rounded once)."""
    g, r = np64(got), np.asarray(ref, np.float64)
    mant = 7 if dtype == torch.bfloat16 else 10
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(r), 1e-30))) - mant)
    err = np.where(np.isinf(g) & np.isinf(r), 0.0, np.abs(g - r))
    bad = ~(err <= TOL_OUT[dtype] + 0.5 * ulp)
    assert not bad.any(), f"{what}: {int(bad.sum())} elements beyond tolerance, max err {float(np.nanmax(err)):.3e}"
