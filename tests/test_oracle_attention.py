"""Pins for the dense attention oracle (CPU only).

Each test checks the oracle against something other than itself: a library
routine (torch SDPA / torch autograd in float64), a closed form, an invariant,
hand-derived masks, a scalar brute force, or finite differences.
"""
import itertools
import math

import numpy as np
import pytest
import torch

from oracle import attention_fwd, attention_bwd, allowed_mask
from workloads import dense_case, alibi_slopes

F64 = torch.float64


def _t(x):
    return torch.as_tensor(np.asarray(x, dtype=np.float64))


# --------------------------------------------------------------- masks ----
def test_mask_hand_derived():
    # causal with Sq == Sk: lower triangle
    m = allowed_mask(np.arange(4), 4, 4, causal=True)
    assert (m == np.array([[1, 0, 0, 0], [1, 1, 0, 0], [1, 1, 1, 0], [1, 1, 1, 1]], bool)).all()
    # causal with Sq < Sk aligns to the bottom-right: the last query sees every key
    m = allowed_mask(np.arange(2), 2, 5, causal=True)
    assert (m == np.array([[1, 1, 1, 1, 0], [1, 1, 1, 1, 1]], bool)).all()
    # causal with Sq > Sk: the first rows see nothing
    m = allowed_mask(np.arange(4), 4, 2, causal=True)
    assert (m == np.array([[0, 0], [0, 0], [1, 0], [1, 1]], bool)).all()
    # sliding window (1, 1), non-causal: a band of width 3
    m = allowed_mask(np.arange(4), 4, 4, window=(1, 1))
    assert (m == np.array([[1, 1, 0, 0], [1, 1, 1, 0], [0, 1, 1, 1], [0, 0, 1, 1]], bool)).all()
    # window (2, 0) with causal: at most 3 keys ending at the diagonal
    m = allowed_mask(np.arange(5), 5, 5, causal=True, window=(2, 0))
    assert (m == np.array([[1, 0, 0, 0, 0], [1, 1, 0, 0, 0], [1, 1, 1, 0, 0],
                           [0, 1, 1, 1, 0], [0, 0, 1, 1, 1]], bool)).all()
    # (-1, -1) is the unbounded window; causal overrides the right bound
    assert allowed_mask(np.arange(3), 3, 3, window=(-1, -1)).all()
    assert (allowed_mask(np.arange(3), 3, 3, causal=True, window=(-1, 5)) ==
            allowed_mask(np.arange(3), 3, 3, causal=True)).all()


# ------------------------------------------------- library routine (SDPA) --
def _sdpa_ref(q, k, v, scale, causal, window, slopes):
    """torch float64 SDPA with the mask and ALiBi given as an additive bias."""
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    g = Hq // Hkv
    qt = q.to(F64).permute(0, 2, 1, 3)
    kt = k.to(F64).repeat_interleave(g, dim=2).permute(0, 2, 1, 3)
    vt = v.to(F64).repeat_interleave(g, dim=2).permute(0, 2, 1, 3)
    ok = torch.from_numpy(allowed_mask(np.arange(Sq), Sq, Sk, causal, window))
    bias = torch.zeros(Hq, Sq, Sk, dtype=F64)
    if slopes is not None:
        ip = torch.arange(Sq)[:, None] + (Sk - Sq)
        dist = (ip - torch.arange(Sk)[None, :]).abs().to(F64)
        bias = bias - slopes.to(F64)[:, None, None] * dist
    bias = bias.masked_fill(~ok, float("-inf"))
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=bias[None], scale=scale)
    lse = torch.logsumexp(scale * qt @ kt.transpose(-1, -2) + bias[None], dim=-1)
    return out.permute(0, 2, 1, 3).numpy(), lse.numpy()


@pytest.mark.parametrize("causal,window,alibi", [
    (False, (-1, -1), False), (True, (-1, -1), False), (False, (5, 3), False),
    (True, (7, 0), True), (False, (-1, -1), True), (True, (-1, -1), True)])
@pytest.mark.parametrize("Sq,Sk", [(37, 37), (19, 45)])
def test_fwd_matches_torch_sdpa(causal, window, alibi, Sq, Sk):
    c = dense_case(2, Sq, Sk, 4, 2, 16, "bf16", seed=11, causal=causal, window=window, alibi=alibi)
    out, lse = attention_fwd(c.q, c.k, c.v, c.scale, causal, window, 0.0, c.alibi_slopes)
    ro, rl = _sdpa_ref(c.q, c.k, c.v, c.scale, causal, window, c.alibi_slopes)
    rows = np.isfinite(rl[0, 0])  # rows with at least one key
    np.testing.assert_allclose(out[:, rows], ro[:, rows], atol=1e-12, rtol=1e-12)
    np.testing.assert_allclose(lse[..., rows], rl[..., rows], atol=1e-12, rtol=1e-12)


# ------------------------------------------------------- closed forms ----
def test_zero_query_uniform_average():
    # q = 0 makes every logit equal: O_i = mean of the allowed values,
    # LSE_i = ln(number of allowed keys).
    S, w = 12, 3
    c = dense_case(1, S, S, 2, 2, 8, "bf16", seed=3)
    q = torch.zeros_like(c.q)
    v = c.v.to(F64).numpy()
    for causal, window, count in [
        (True, (-1, -1), lambda i: i + 1),
        (True, (w, 0), lambda i: min(i, w) + 1),
        (False, (w, 2), lambda i: min(i, w) + min(S - 1 - i, 2) + 1),
        (False, (-1, -1), lambda i: S),
    ]:
        out, lse = attention_fwd(q, c.k, c.v, c.scale, causal, window)
        for i in range(S):
            n = count(i)
            assert lse[0, 0, i] == pytest.approx(math.log(n), abs=1e-14)
            lo = i - w if window[0] >= 0 else 0
            lo = max(lo, 0)
            hi = i if causal else (min(S - 1, i + window[1]) if window[1] >= 0 else S - 1)
            np.testing.assert_allclose(out[0, i, 0], v[0, lo:hi + 1, 0].mean(axis=0), atol=1e-14)


def test_zero_query_alibi_geometric():
    # q = 0 with ALiBi, causal: z_ij = -m (i - j), so
    # LSE_i = ln sum_{d=0..i} e^{-m d} = ln((1 - e^{-m(i+1)}) / (1 - e^{-m})).
    S, H = 10, 4
    c = dense_case(1, S, S, H, H, 8, "bf16", seed=4, causal=True, alibi=True)
    q = torch.zeros_like(c.q)
    out, lse = attention_fwd(q, c.k, c.v, c.scale, True, (-1, -1), 0.0, c.alibi_slopes)
    v = c.v.to(F64).numpy()[0]
    for h in range(H):
        m = float(c.alibi_slopes[h])
        for i in range(S):
            ref = math.log((1 - math.exp(-m * (i + 1))) / (1 - math.exp(-m)))
            assert lse[0, h, i] == pytest.approx(ref, abs=1e-13)
        # row 1: weights e^{-m} on v_0 and 1 on v_1
        w0 = math.exp(-m)
        np.testing.assert_allclose(out[0, 1, h], (w0 * v[0, h] + v[1, h]) / (1 + w0), atol=1e-13)
    # the slope of query head h is 2^(-8(h+1)/H)
    assert [float(x) for x in alibi_slopes(4)] == [2 ** -2, 2 ** -4, 2 ** -6, 2 ** -8]


def test_single_key_and_first_causal_row():
    c = dense_case(2, 9, 1, 4, 2, 16, "bf16", seed=5)
    out, lse = attention_fwd(c.q, c.k, c.v, c.scale)
    q, k, v = (t.to(F64).numpy() for t in (c.q, c.k, c.v))
    for h in range(4):
        np.testing.assert_allclose(out[:, :, h], np.broadcast_to(v[:, 0:1, h // 2], out[:, :, h].shape), atol=0)
        s = c.scale * np.einsum("bsd,bd->bs", q[:, :, h], k[:, 0, h // 2])
        np.testing.assert_allclose(lse[:, h], s, atol=1e-13)
    # first row under causal masking sees only key 0
    c = dense_case(1, 6, 6, 2, 2, 8, "bf16", seed=6, causal=True)
    out, lse = attention_fwd(c.q, c.k, c.v, c.scale, causal=True)
    np.testing.assert_allclose(out[0, 0], c.v.to(F64).numpy()[0, 0], atol=0)


def test_softcap_closed_forms():
    # one key: LSE = c * tanh(s / c); two keys: P_0 = 1 / (1 + e^{z_1 - z_0})
    cap = 2.5
    c = dense_case(1, 5, 2, 1, 1, 8, "bf16", seed=7)
    q, k, v = (t.to(F64).numpy()[0, :, 0] for t in (c.q, c.k, c.v))
    out1, lse1 = attention_fwd(c.q, c.k[:, :1], c.v[:, :1], c.scale, softcap=cap)
    for i in range(5):
        s = c.scale * float(q[i] @ k[0])
        assert lse1[0, 0, i] == pytest.approx(cap * math.tanh(s / cap), abs=1e-14)
    out2, _ = attention_fwd(c.q, c.k, c.v, c.scale, softcap=cap)
    for i in range(5):
        z0 = cap * math.tanh(c.scale * float(q[i] @ k[0]) / cap)
        z1 = cap * math.tanh(c.scale * float(q[i] @ k[1]) / cap)
        p0 = 1.0 / (1.0 + math.exp(z1 - z0))
        np.testing.assert_allclose(out2[0, i, 0], p0 * v[0] + (1 - p0) * v[1], atol=1e-14)


def test_constant_values_and_empty_rows():
    c = dense_case(1, 7, 7, 2, 1, 8, "bf16", seed=8, causal=True)
    v = torch.full_like(c.v, 0.75)
    out, _ = attention_fwd(c.q, c.k, v, c.scale, causal=True)
    np.testing.assert_allclose(out, 0.75, atol=1e-15)
    # Sq > Sk with causal: rows 0..Sq-Sk-1 see no key -> O = 0, LSE = +inf
    c = dense_case(1, 5, 3, 1, 1, 8, "bf16", seed=9, causal=True)
    out, lse = attention_fwd(c.q, c.k, c.v, c.scale, causal=True)
    assert (out[0, :2] == 0).all() and np.isposinf(lse[0, 0, :2]).all()
    assert np.isfinite(lse[0, 0, 2:]).all()
    # no keys at all (Sk = 0): every row is empty, and so are the gradients
    c = dense_case(2, 3, 1, 2, 1, 8, "bf16", seed=10)
    k0, v0 = c.k[:, :0], c.v[:, :0]
    for causal in (False, True):
        out, lse = attention_fwd(c.q, k0, v0, c.scale, causal=causal)
        assert out.shape == (2, 3, 2, 8) and (out == 0).all() and np.isposinf(lse).all()
        dq, dk, dv = attention_bwd(c.q, k0, v0, c.dout, c.scale, causal=causal)
        assert (dq == 0).all() and dk.shape == (2, 0, 1, 8) and dv.shape == (2, 0, 1, 8)


# ---------------------------------------------------------- invariants ----
def test_rows_of_p_sum_to_one():
    # with V = identity (Sk = D), row i of O is row i of P
    S, D = 16, 16
    c = dense_case(1, S, S, 2, 2, D, "bf16", seed=10, causal=True, window=(5, 0), alibi=True)
    eye = torch.eye(D, dtype=torch.float32)[None, :, None, :].expand(1, S, 2, D).contiguous()
    out, _ = attention_fwd(c.q, c.k, eye, c.scale, True, (5, 0), 3.0, c.alibi_slopes)
    np.testing.assert_allclose(out.sum(axis=-1), 1.0, atol=1e-14)
    assert (out >= 0).all()
    assert (out[0, 10, :, :5] == 0).all() and (out[0, 10, :, 11:] == 0).all()


def test_key_permutation_invariance():
    c = dense_case(2, 11, 13, 4, 2, 16, "bf16", seed=12)
    perm = torch.from_numpy(np.random.default_rng(0).permutation(13))
    o1, l1 = attention_fwd(c.q, c.k, c.v, c.scale, softcap=4.0)
    o2, l2 = attention_fwd(c.q, c.k[:, perm], c.v[:, perm], c.scale, softcap=4.0)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)
    do = c.dout
    g1 = attention_bwd(c.q, c.k, c.v, do, c.scale)
    g2 = attention_bwd(c.q, c.k[:, perm], c.v[:, perm], do, c.scale)
    np.testing.assert_allclose(g1[0], g2[0], atol=1e-12)
    np.testing.assert_allclose(g1[1][:, perm.numpy()], g2[1], atol=1e-12)
    np.testing.assert_allclose(g1[2][:, perm.numpy()], g2[2], atol=1e-12)


def test_gqa_equals_repeated_mha():
    c = dense_case(1, 10, 10, 6, 2, 8, "bf16", seed=13, causal=True, alibi=True)
    kr = c.k.repeat_interleave(3, dim=2)
    vr = c.v.repeat_interleave(3, dim=2)
    o1, l1 = attention_fwd(c.q, c.k, c.v, c.scale, True, (-1, -1), 0.0, c.alibi_slopes)
    o2, l2 = attention_fwd(c.q, kr, vr, c.scale, True, (-1, -1), 0.0, c.alibi_slopes)
    np.testing.assert_allclose(o1, o2, atol=0)
    np.testing.assert_allclose(l1, l2, atol=0)
    g1 = attention_bwd(c.q, c.k, c.v, c.dout, c.scale, True, (-1, -1), 0.0, c.alibi_slopes)
    g2 = attention_bwd(c.q, kr, vr, c.dout, c.scale, True, (-1, -1), 0.0, c.alibi_slopes)
    np.testing.assert_allclose(g1[0], g2[0], atol=1e-13)
    np.testing.assert_allclose(g1[1], g2[1].reshape(1, 10, 2, 3, 8).sum(3), atol=1e-13)
    np.testing.assert_allclose(g1[2], g2[2].reshape(1, 10, 2, 3, 8).sum(3), atol=1e-13)


def test_window_and_softcap_limits():
    c = dense_case(1, 9, 9, 2, 2, 8, "bf16", seed=14)
    base = attention_fwd(c.q, c.k, c.v, c.scale)
    wide = attention_fwd(c.q, c.k, c.v, c.scale, window=(9, 9))
    big_cap = attention_fwd(c.q, c.k, c.v, c.scale, softcap=1e7)
    np.testing.assert_allclose(base[0], wide[0], atol=0)
    np.testing.assert_allclose(base[0], big_cap[0], atol=1e-10)


def test_alibi_distance_vs_column_form():
    # Under causal masking -m|i'-j| = -m i' + m j: the row constant shifts LSE
    # by exactly -m i' and leaves O unchanged.
    S, H = 8, 2
    c = dense_case(1, S, S, H, H, 8, "bf16", seed=15, causal=True, alibi=True)
    o1, l1 = attention_fwd(c.q, c.k, c.v, c.scale, True, (-1, -1), 0.0, c.alibi_slopes)
    q, k, v = (t.to(F64).numpy()[0] for t in (c.q, c.k, c.v))
    for h in range(H):
        m = float(c.alibi_slopes[h])
        s = c.scale * q[:, h] @ k[:, h].T + m * np.arange(S)[None, :]
        s = np.where(np.tril(np.ones((S, S), bool)), s, -np.inf)
        lse_col = np.log(np.exp(s - s.max(1, keepdims=True)).sum(1)) + s.max(1)
        np.testing.assert_allclose(l1[0, h], lse_col - m * np.arange(S), atol=1e-13)


# ---------------------------------------------------------- brute force ----
def _brute(q, k, v, scale, causal, window, softcap, slopes):
    """Scalar loops over (b, h, i, j, d) in plain Python."""
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    out = np.zeros((B, Sq, Hq, D))
    lse = np.zeros((B, Hq, Sq))
    for b in range(B):
        for h in range(Hq):
            kh = h * Hkv // Hq
            for i in range(Sq):
                ip = i + Sk - Sq
                zs = {}
                for j in range(Sk):
                    if causal and j > ip:
                        continue
                    if window[0] >= 0 and j < ip - window[0]:
                        continue
                    if not causal and window[1] >= 0 and j > ip + window[1]:
                        continue
                    s = 0.0
                    for d in range(D):
                        s += float(q[b, i, h, d]) * float(k[b, j, kh, d])
                    s *= scale
                    if softcap > 0:
                        s = softcap * math.tanh(s / softcap)
                    if slopes is not None:
                        s -= float(slopes[h]) * abs(ip - j)
                    zs[j] = s
                if not zs:
                    lse[b, h, i] = math.inf
                    continue
                mx = max(zs.values())
                tot = sum(math.exp(z - mx) for z in zs.values())
                lse[b, h, i] = mx + math.log(tot)
                for j, z in zs.items():
                    p = math.exp(z - mx) / tot
                    for d in range(D):
                        out[b, i, h, d] += p * float(v[b, j, kh, d])
    return out, lse


@pytest.mark.parametrize("causal,window,softcap,alibi", list(itertools.product(
    [False, True], [(-1, -1), (2, 1)], [0.0, 1.5], [False, True])))
def test_brute_force_tiny(causal, window, softcap, alibi):
    c = dense_case(2, 5, 7, 4, 2, 3, "bf16", seed=16, causal=causal, window=window,
                   softcap=softcap, alibi=alibi)
    q, k, v = (t.to(F64).numpy() for t in (c.q, c.k, c.v))
    ro, rl = _brute(q, k, v, c.scale, causal, window, softcap, c.alibi_slopes)
    out, lse = attention_fwd(c.q, c.k, c.v, c.scale, causal, window, softcap, c.alibi_slopes)
    np.testing.assert_allclose(out, ro, atol=1e-13)
    np.testing.assert_allclose(lse, rl, atol=1e-13)


# ------------------------------------------------------------ backward ----
def _torch_autograd(c, causal, window, softcap):
    """Gradients of a naive float64 torch expression via autograd."""
    q = c.q.to(F64).requires_grad_(True)
    k = c.k.to(F64).requires_grad_(True)
    v = c.v.to(F64).requires_grad_(True)
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    g = Hq // Hkv
    kk = k.repeat_interleave(g, dim=2)
    vv = v.repeat_interleave(g, dim=2)
    s = torch.einsum("bihd,bjhd->bhij", q, kk) * c.scale
    if softcap > 0:
        s = softcap * torch.tanh(s / softcap)
    if c.alibi_slopes is not None:
        ip = torch.arange(Sq)[:, None] + (Sk - Sq)
        s = s - c.alibi_slopes.to(F64)[None, :, None, None] * (ip - torch.arange(Sk)[None, :]).abs().to(F64)
    ok = torch.from_numpy(allowed_mask(np.arange(Sq), Sq, Sk, causal, window))
    s = s.masked_fill(~ok, float("-inf"))
    p = torch.softmax(s, dim=-1)
    o = torch.einsum("bhij,bjhd->bihd", p, vv)
    (o * c.dout.to(F64)).sum().backward()
    return q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


@pytest.mark.parametrize("causal,window,softcap,alibi", [
    (False, (-1, -1), 0.0, False), (True, (-1, -1), 0.0, False), (True, (4, 0), 2.0, True),
    (False, (3, 2), 0.0, True), (False, (-1, -1), 1.0, False)])
def test_bwd_matches_torch_autograd(causal, window, softcap, alibi):
    c = dense_case(2, 13, 13, 4, 2, 8, "bf16", seed=17, causal=causal, window=window,
                   softcap=softcap, alibi=alibi)
    ref = _torch_autograd(c, causal, window, softcap)
    got = attention_bwd(c.q, c.k, c.v, c.dout, c.scale, causal, window, softcap, c.alibi_slopes)
    for a, b in zip(got, ref):
        np.testing.assert_allclose(a, b, atol=1e-12, rtol=1e-10)


def test_bwd_finite_differences():
    # central differences of f = sum(O * dO) through the oracle's own forward
    c = dense_case(1, 6, 7, 2, 1, 4, "bf16", seed=18, causal=True, softcap=1.5, alibi=True)
    args = dict(causal=True, window=(-1, -1), softcap=1.5, alibi_slopes=c.alibi_slopes)
    do = c.dout.to(F64).numpy()
    dq, dk, dv = attention_bwd(c.q, c.k, c.v, c.dout, c.scale, **args)
    base = {n: t.to(F64).numpy() for n, t in (("q", c.q), ("k", c.k), ("v", c.v))}
    eps = 1e-6
    rng = np.random.default_rng(0)
    for name, grad in (("q", dq), ("k", dk), ("v", dv)):
        for _ in range(6):
            idx = tuple(int(rng.integers(0, n)) for n in base[name].shape)
            vals = []
            for sgn in (+1, -1):
                x = {n: a.copy() for n, a in base.items()}
                x[name][idx] += sgn * eps
                o, _ = attention_fwd(x["q"], x["k"], x["v"], c.scale, **args)
                vals.append((o * do).sum())
            fd = (vals[0] - vals[1]) / (2 * eps)
            assert fd == pytest.approx(grad[idx], abs=1e-7, rel=1e-6)


def test_bwd_zero_dout_and_key_gradient_sum():
    c = dense_case(1, 9, 9, 2, 1, 8, "bf16", seed=19, causal=True, alibi=True)
    z = attention_bwd(c.q, c.k, c.v, torch.zeros_like(c.dout), c.scale, causal=True,
                      alibi_slopes=c.alibi_slopes)
    for g in z:
        assert np.abs(g).max() == 0
    # without softcap, sum_j dk_j = scale * sum_i (sum_j dS_ij) q_i = 0
    _, dk, _ = attention_bwd(c.q, c.k, c.v, c.dout, c.scale, causal=True, alibi_slopes=c.alibi_slopes)
    np.testing.assert_allclose(dk.sum(axis=1), 0.0, atol=1e-12)


def test_sampled_modes_match_full():
    c = dense_case(1, 40, 40, 4, 2, 8, "bf16", seed=20, causal=True, window=(9, 0), softcap=3.0,
                   alibi=True)
    args = (c.scale, True, (9, 0), 3.0, c.alibi_slopes)
    o, l = attention_fwd(c.q, c.k, c.v, *args)
    rows = [0, 7, 39]
    os_, ls = attention_fwd(c.q, c.k, c.v, *args, heads=[1, 3], q_rows=rows)
    np.testing.assert_allclose(os_[:, rows][:, :, [1, 3]], o[:, rows][:, :, [1, 3]], atol=1e-14)
    np.testing.assert_allclose(ls[:, [1, 3]][:, :, rows], l[:, [1, 3]][:, :, rows], atol=1e-14)
    dq, dk, dv = attention_bwd(c.q, c.k, c.v, c.dout, *args)
    kr = [0, 5, 38]
    _, dks, dvs = attention_bwd(c.q, c.k, c.v, c.dout, *args, k_rows=kr)
    np.testing.assert_allclose(dks[:, kr], dk[:, kr], atol=1e-12)
    np.testing.assert_allclose(dvs[:, kr], dv[:, kr], atol=1e-12)
    qr = [1, 20, 39]
    dqs, _, _ = attention_bwd(c.q, c.k, c.v, c.dout, *args, heads=[0, 2], q_rows=qr)
    np.testing.assert_allclose(dqs[:, qr][:, :, [0, 2]], dq[:, qr][:, :, [0, 2]], atol=1e-12)
