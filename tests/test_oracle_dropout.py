"""Pins for the attention-dropout oracle (CPU only).

The generator is pinned against numpy's own Philox (a library routine; numpy
ships the 4 x 64-bit variant, which shares the round structure) and against
the published known-answer vectors of Philox4x32.  The mask is checked for
its statistics and structure, and dropout attention against torch float64
(softmax, products and autograd) with the same mask.
"""
import os

import numpy as np
import pytest
import torch

from oracle import attention_fwd, attention_bwd, varlen_fwd, varlen_bwd
from oracle.dropout import philox4, keep_mask, keep_scale, threshold
from workloads import dense_case

F64 = torch.float64
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "philox4x32_kat.txt")


def test_philox4x64_matches_numpy():
    # numpy's Philox bit generator increments the counter before each block
    for ctr, key in [([0, 0, 0, 0], [0, 0]), ([5, 7, 11, 13], [0x243F6A8885A308D3, 0x13198A2E03707344]),
                     ([2 ** 63, 3, 2 ** 64 - 1, 9], [2 ** 64 - 1, 12345])]:
        bg = np.random.Philox(counter=np.array(ctr, dtype=np.uint64), key=np.array(key, dtype=np.uint64))
        raw = [int(x) for x in bg.random_raw(4)]
        nxt = [ctr[0] + 1] + ctr[1:]
        assert philox4(nxt, key, width=64) == raw


def test_philox4x32_known_answers():
    rows = [ln.split() for ln in open(GOLDEN) if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 4
    for r in rows:
        rounds = int(r[0])
        ctr = [int(x, 16) for x in r[1:5]]
        key = [int(x, 16) for x in r[5:7]]
        want = [int(x, 16) for x in r[7:11]]
        got = philox4([np.array([c]) for c in ctr], key, width=32, rounds=rounds)
        assert [int(x[0]) for x in got] == want


def test_philox4x32_vectorised_equals_scalar_words():
    rng = np.random.default_rng(3)
    ctr = [rng.integers(0, 2 ** 32, size=50) for _ in range(4)]
    key = [int(rng.integers(0, 2 ** 32)), int(rng.integers(0, 2 ** 32))]
    vec = philox4(ctr, key)
    for n in range(50):
        one = philox4([np.array([c[n]]) for c in ctr], key)
        assert [int(w[0]) for w in one] == [int(w[n]) for w in vec]


def test_threshold_and_scale():
    assert threshold(0.0) == 0 and keep_scale(0.0) == 1.0
    assert threshold(0.1) == 26 and keep_scale(0.1) == 256.0 / 230.0
    assert threshold(0.5) == 128 and keep_scale(0.5) == 2.0
    assert threshold(1.5 / 256) == 2 and threshold(2.5 / 256) == 2  # ties to even
    with pytest.raises(ValueError):
        threshold(1.0)
    with pytest.raises(ValueError):
        threshold(-0.01)


def test_mask_statistics():
    rows, cols = np.arange(512), np.arange(512)
    for p in (0.1, 0.25, 0.5):
        m = keep_mask(p, 2024, 7, 3, rows, cols)
        q = threshold(p) / 256.0
        n = m.size
        drop = 1.0 - m.mean()
        assert abs(drop - q) < 5.0 * np.sqrt(q * (1 - q) / n)
        # no structure along rows or columns: every row/column drops near q
        per_row = 1.0 - m.mean(axis=1)
        assert abs(per_row.mean() - q) < 0.01 and per_row.std() < 3 * np.sqrt(q * (1 - q) / 512)
    assert keep_mask(0.0, 1, 2, 3, rows, cols).all()


def test_mask_is_a_function_of_the_pair():
    """A sub-block computed on its own equals the slice of a larger mask, and
    every input of the counter or key changes the mask."""
    big = keep_mask(0.3, 99, 5, 11, np.arange(40), np.arange(70))
    sub = keep_mask(0.3, 99, 5, 11, np.arange(13, 29), np.arange(3, 61))
    assert (sub == big[13:29, 3:61]).all()
    base = keep_mask(0.3, 99, 5, 11, np.arange(64), np.arange(64))
    for other in (keep_mask(0.3, 100, 5, 11, np.arange(64), np.arange(64)),
                  keep_mask(0.3, 99 + (1 << 40), 5, 11, np.arange(64), np.arange(64)),
                  keep_mask(0.3, 99, 6, 11, np.arange(64), np.arange(64)),
                  keep_mask(0.3, 99, 5, 12, np.arange(64), np.arange(64))):
        assert (other != base).mean() > 0.2


def test_mask_block_layout():
    """One generator call per 4 x 4 block: word i % 4, byte j % 4."""
    seed, off, bh = 0x0123456789ABCDEF, 77, 5
    t = threshold(0.5)
    m = keep_mask(0.5, seed, off, bh, np.arange(8), np.arange(8))
    for I in range(2):
        for J in range(2):
            w = philox4([np.array([J]), np.array([I]), np.array([bh]), np.array([off])],
                        (seed & 0xFFFFFFFF, seed >> 32))
            for a in range(4):
                for c in range(4):
                    byte = (int(w[a][0]) >> (8 * c)) & 0xFF
                    assert m[4 * I + a, 4 * J + c] == (byte >= t)


def _naive_dropout(q, k, v, scale, causal, p, seed, off, do=None):
    """torch float64 softmax attention with the oracle's keep mask applied."""
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    g = Hq // Hkv
    qt = q.to(F64).permute(0, 2, 1, 3).clone().requires_grad_(True)
    kt = k.to(F64).permute(0, 2, 1, 3).clone().requires_grad_(True)
    vt = v.to(F64).permute(0, 2, 1, 3).clone().requires_grad_(True)
    kr = kt.repeat_interleave(g, dim=1)
    vr = vt.repeat_interleave(g, dim=1)
    s = scale * (qt @ kr.transpose(-1, -2))
    if causal:
        ok = torch.ones(Sq, Sk, dtype=torch.bool).tril(Sk - Sq)
        s = s.masked_fill(~ok, float("-inf"))
    P = torch.softmax(s, dim=-1)
    M = torch.zeros(B, Hq, Sq, Sk, dtype=F64)
    for b in range(B):
        for h in range(Hq):
            M[b, h] = torch.from_numpy(keep_mask(p, seed, off, b * Hq + h, np.arange(Sq), np.arange(Sk)).astype(np.float64))
    o = (P * M * keep_scale(p)) @ vr
    grads = None
    if do is not None:
        o.backward(do.to(F64).permute(0, 2, 1, 3))
        grads = [x.grad.permute(0, 2, 1, 3).numpy() for x in (qt, kt, vt)]
    return o.detach().permute(0, 2, 1, 3).numpy(), grads


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_fwd_bwd_match_torch(causal):
    c = dense_case(B=2, Sq=12, Sk=12, Hq=4, Hkv=2, D=8, dtype="fp16", seed=31)
    drop = (0.2, 4242, 3)
    o, lse = attention_fwd(c.q, c.k, c.v, c.scale, causal, dropout=drop)
    o0, lse0 = attention_fwd(c.q, c.k, c.v, c.scale, causal)
    ref, grads = _naive_dropout(c.q, c.k, c.v, c.scale, causal, *drop, do=c.dout)
    np.testing.assert_allclose(o, ref, atol=1e-12)
    np.testing.assert_array_equal(lse, lse0)  # LSE of the undropped weights
    dq, dk, dv = attention_bwd(c.q, c.k, c.v, c.dout, c.scale, causal, dropout=drop)
    for got, want in zip((dq, dk, dv), grads):
        np.testing.assert_allclose(got, want, atol=1e-11)


def test_dropout_sampled_modes_match_full():
    c = dense_case(B=1, Sq=40, Sk=40, Hq=2, Hkv=1, D=8, dtype="fp16", seed=32)
    drop = (0.3, 11, 0)
    dq, dk, dv = attention_bwd(c.q, c.k, c.v, c.dout, c.scale, True, dropout=drop)
    dq_r, _, _ = attention_bwd(c.q, c.k, c.v, c.dout, c.scale, True, q_rows=[0, 17, 39], dropout=drop)
    np.testing.assert_allclose(dq_r[0, [0, 17, 39]], dq[0, [0, 17, 39]], atol=1e-12)
    _, dk_r, dv_r = attention_bwd(c.q, c.k, c.v, c.dout, c.scale, True, k_rows=[1, 20, 38], dropout=drop)
    np.testing.assert_allclose(dk_r[0, [1, 20, 38]], dk[0, [1, 20, 38]], atol=1e-12)
    np.testing.assert_allclose(dv_r[0, [1, 20, 38]], dv[0, [1, 20, 38]], atol=1e-12)


def test_dropout_zero_is_identity_and_mean_is_unbiased():
    c = dense_case(B=1, Sq=6, Sk=6, Hq=1, Hkv=1, D=4, dtype="fp16", seed=33)
    o0, _ = attention_fwd(c.q, c.k, c.v, c.scale)
    o, _ = attention_fwd(c.q, c.k, c.v, c.scale, dropout=(0.0, 5, 0))
    np.testing.assert_array_equal(o, o0)
    # E[K * scale] = 1 elementwise: the mean over many seeds approaches O
    acc = np.zeros_like(o0)
    n = 400
    for s in range(n):
        acc += attention_fwd(c.q, c.k, c.v, c.scale, dropout=(0.5, s, 0))[0]
    assert np.abs(acc / n - o0).max() < 0.15 * np.abs(o0).max() + 0.05


def test_varlen_dropout_uses_sequence_index():
    """Equal-length packed sequences draw the same masks as the dense batch."""
    c = dense_case(B=3, Sq=9, Sk=9, Hq=2, Hkv=2, D=8, dtype="fp16", seed=34)
    drop = (0.25, 8, 1)
    cu = [0, 9, 18, 27]
    pq = c.q.reshape(27, 2, 8)
    pk = c.k.reshape(27, 2, 8)
    pv = c.v.reshape(27, 2, 8)
    pdo = c.dout.reshape(27, 2, 8)
    o, _ = attention_fwd(c.q, c.k, c.v, c.scale, True, dropout=drop)
    ov, _ = varlen_fwd(pq, pk, pv, cu, cu, c.scale, True, dropout=drop)
    np.testing.assert_allclose(ov, o.reshape(27, 2, 8), atol=1e-13)
    g = attention_bwd(c.q, c.k, c.v, c.dout, c.scale, True, dropout=drop)
    gv = varlen_bwd(pq, pk, pv, pdo, cu, cu, c.scale, True, dropout=drop)
    for a, b in zip(gv, g):
        np.testing.assert_allclose(a, b.reshape(27, 2, 8), atol=1e-12)
