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


def visible_dense(Sq, Sk, causal=False, window=(-1, -1)):
    """Visible keys per query row of a dense call, shaped (1, Sq, 1) to
    broadcast against an output's (B, Sq, Hq) rows."""
    from oracle import allowed_mask
    return allowed_mask(np.arange(Sq), Sq, Sk, causal, window).sum(axis=1)[None, :, None]


def visible_varlen(cu_q, cu_k, causal=False, window=(-1, -1)):
    """Visible keys per packed query row of a varlen call, shaped (total_q, 1)."""
    from oracle import allowed_mask
    cq = [int(x) for x in (cu_q.tolist() if hasattr(cu_q, "tolist") else cu_q)]
    ck = [int(x) for x in (cu_k.tolist() if hasattr(cu_k, "tolist") else cu_k)]
    out = np.zeros((cq[-1], 1), np.int64)
    for s in range(len(cq) - 1):
        a, b, n = cq[s], cq[s + 1], ck[s + 1] - ck[s]
        if b > a:
            out[a:b, 0] = allowed_mask(np.arange(b - a), b - a, n, causal, window).sum(axis=1)
    return out


FEW_KEYS = 3  # rows with at most this many visible keys get the rounding margin


def assert_out_rounded(got, ref, dtype, visible, what="out"):
    """Output tolerance for shapes with very short rows.

    Every element is held to the plain bound TOL_OUT except two kinds, which
    get TOL_OUT plus half an ulp of the reference value in the output dtype:
    rows with at most FEW_KEYS visible keys (O close to a single v, so the
    16-bit P operand of the PV product and the one rounding of the output
    already reach the plain bound: e.g. row 1 of a causal D = 256 bf16 case
    gives 1.089e-2 from the kernel and from that arithmetic emulated on the
    CPU), and elements with |O_ref| >= 2 (half an ulp there is >= 3.9e-3 in
    bf16).  ``visible`` holds the visible-key count of each output row and
    broadcasts against ref.shape[:-1].  Prints how many rows needed the
    margin."""
    g, r = np64(got), np.asarray(ref, np.float64)
    mant = 7 if dtype == torch.bfloat16 else 10
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(r), 1e-30))) - mant)
    err = np.where(np.isinf(g) & np.isinf(r) & (np.sign(g) == np.sign(r)), 0.0, np.abs(g - r))
    err = np.where(np.isnan(err), np.inf, err)
    few = np.broadcast_to(np.asarray(visible) <= FEW_KEYS, r.shape[:-1])[..., None]
    exempt = few | (np.abs(r) >= 2.0)
    tol = TOL_OUT[dtype]
    bound = np.where(exempt, tol + 0.5 * ulp, tol)
    bad = ~(err <= bound)
    plain = float(err[~exempt].max()) if (~exempt).any() else 0.0
    used_rows = int((exempt & (err > tol)).any(axis=-1).sum())
    say(f"{what}: max err {plain:.3e} on plain-bound elements; {used_rows} rows used the rounding margin")
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements beyond tolerance, max err "
                           f"{float(err.max()):.3e} (plain-bound max {plain:.3e})")


def tile_rows(S, tile, seed):
    """One seeded row in every `tile`-row block of [0, S), plus rows 0 and
    S - 1 (sorted, unique): a sample that meets every tile of a launch."""
    rng = np.random.default_rng(seed)
    rows = {0, S - 1}
    for t0 in range(0, S, tile):
        rows.add(int(t0 + rng.integers(0, min(tile, S - t0))))
    return sorted(rows)
