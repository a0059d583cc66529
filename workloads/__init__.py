"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests,
``bench.py`` and ``__graft_entry__.smoke()``.

This module draws random numbers and builds index structures (sequence
lengths, page tables, rotary tables).  It holds none of the attention
arithmetic: every value it returns is an *input* to the method.

Recipes (the shapes follow the pages' workloads):

* dense tensors: ``torch.Generator('cpu').manual_seed(seed)`` then
  ``torch.randn(shape, dtype=float32).to(dtype)``; q, k, v, dO are drawn in
  that order from one generator, so one seed fixes all four.
* integer draws (varlen lengths, cache lengths, page permutation):
  ``numpy.random.default_rng(seed)``.
* rotary tables: angle(pos, i) = pos * base**(-2i/rotary_dim) evaluated in
  float64, stored as float32 ``cos``/``sin`` of shape (max_pos, rotary_dim/2).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

DTYPES = {"fp16": torch.float16, "bf16": torch.bfloat16}


def randn(gen: torch.Generator, shape, dtype: torch.dtype) -> torch.Tensor:
    """N(0,1) float32 draw rounded once to ``dtype`` (CPU tensor)."""
    return torch.randn(*shape, generator=gen, dtype=torch.float32).to(dtype)


def make_gen(seed: int) -> torch.Generator:
    g = torch.Generator("cpu")
    g.manual_seed(int(seed))
    return g


@dataclass
class DenseCase:
    """Inputs for one dense (B, S, H, D) forward/backward call."""

    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    dout: torch.Tensor | None
    scale: float
    causal: bool = False
    window: tuple[int, int] = (-1, -1)
    softcap: float = 0.0
    alibi_slopes: torch.Tensor | None = None  # float32 (Hq,)
    name: str = ""


def dense_case(B, Sq, Sk, Hq, Hkv, D, dtype="bf16", seed=0, causal=False,
               window=(-1, -1), softcap=0.0, alibi=False, with_dout=True,
               scale=None, name="") -> DenseCase:
    dt = DTYPES[dtype] if isinstance(dtype, str) else dtype
    g = make_gen(seed)
    q = randn(g, (B, Sq, Hq, D), dt)
    k = randn(g, (B, Sk, Hkv, D), dt)
    v = randn(g, (B, Sk, Hkv, D), dt)
    do = randn(g, (B, Sq, Hq, D), dt) if with_dout else None
    slopes = alibi_slopes(Hq) if alibi else None
    return DenseCase(q, k, v, do, (1.0 / math.sqrt(D)) if scale is None else float(scale),
                     causal, tuple(window), float(softcap), slopes, name)


def alibi_slopes(Hq: int) -> torch.Tensor:
    """Slopes 2^(-8 i / Hq) for i = 1..Hq (float32, one per query head)."""
    return torch.tensor([2.0 ** (-8.0 * (i + 1) / Hq) for i in range(Hq)], dtype=torch.float32)


# ---------------------------------------------------------------- configs ---
# Forward-only fp16 example: (2, 512, 16, 64), causal, scale 1/8.
def cfg1(seed=1) -> DenseCase:
    return dense_case(2, 512, 512, 16, 16, 64, "fp16", seed, causal=True, scale=1.0 / 8,
                      with_dout=False, name="cfg1_fwd_fp16_b2_s512_h16_d64_causal")


# Forward+backward bf16 at hidden 2048, B*S = 16384 tokens.
CFG2_SEQLENS = (512, 1024, 2048, 4096, 8192, 16384)
CFG2_HEADS = ((16, 128), (32, 64))


def cfg2(S: int, H: int = 16, D: int = 128, causal: bool = False, seed=2) -> DenseCase:
    B = 16384 // S
    return dense_case(B, S, S, H, H, D, "bf16", seed, causal=causal,
                      name=f"cfg2_b{B}_s{S}_h{H}_d{D}_{'causal' if causal else 'full'}")


# GQA + window + softcap + ALiBi, bf16.
def cfg3(seed=3, S=8192) -> DenseCase:
    return dense_case(1, S, S, 32, 8, 128, "bf16", seed, causal=True, window=(4096, 0),
                      softcap=30.0, alibi=True, name=f"cfg3_gqa_s{S}_win4096_softcap30_alibi")


# Varlen packed sequences.
def varlen_lengths(total=32768, lo=128, hi=4096, seed=4) -> list[int]:
    """Integers in [lo, hi] drawn until the running sum reaches ``total``; the
    last one is truncated so the lengths sum exactly to ``total``."""
    rng = np.random.default_rng(seed)
    out, s = [], 0
    while s < total:
        L = int(rng.integers(lo, hi + 1))
        L = min(L, total - s)
        if L > 0:
            out.append(L)
        s += L
    return out


@dataclass
class VarlenCase:
    q: torch.Tensor  # (total_q, Hq, D)
    k: torch.Tensor  # (total_k, Hkv, D)
    v: torch.Tensor
    dout: torch.Tensor | None
    cu_seqlens_q: torch.Tensor  # int32 (nseq+1)
    cu_seqlens_k: torch.Tensor
    max_seqlen_q: int
    max_seqlen_k: int
    scale: float
    causal: bool = True
    window: tuple[int, int] = (-1, -1)
    softcap: float = 0.0
    alibi_slopes: torch.Tensor | None = None
    name: str = ""


def varlen_case(lengths_q, lengths_k=None, Hq=16, Hkv=16, D=128, dtype="bf16", seed=4,
                causal=True, window=(-1, -1), softcap=0.0, alibi=False, with_dout=True,
                name="") -> VarlenCase:
    lengths_k = list(lengths_q) if lengths_k is None else list(lengths_k)
    dt = DTYPES[dtype] if isinstance(dtype, str) else dtype
    cq = np.concatenate([[0], np.cumsum(lengths_q)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lengths_k)]).astype(np.int32)
    g = make_gen(seed)
    tq, tk = int(cq[-1]), int(ck[-1])
    q = randn(g, (tq, Hq, D), dt)
    k = randn(g, (tk, Hkv, D), dt)
    v = randn(g, (tk, Hkv, D), dt)
    do = randn(g, (tq, Hq, D), dt) if with_dout else None
    return VarlenCase(q, k, v, do, torch.from_numpy(cq), torch.from_numpy(ck),
                      int(max(lengths_q)), int(max(lengths_k)), 1.0 / math.sqrt(D), causal,
                      tuple(window), float(softcap), alibi_slopes(Hq) if alibi else None, name)


def cfg4(seed=4) -> VarlenCase:
    lens = varlen_lengths(32768, 128, 4096, seed)
    return varlen_case(lens, Hq=16, Hkv=16, D=128, seed=seed, causal=True,
                       name=f"cfg4_varlen_{len(lens)}seqs_32768tok_h16_d128_causal")


# Paged KV-cache decode.
def rotary_tables(max_pos: int, rotary_dim: int, base: float = 10000.0):
    """float32 cos/sin tables (max_pos, rotary_dim/2) from float64 angles."""
    half = rotary_dim // 2
    inv = base ** (-np.arange(0, half, dtype=np.float64) * 2.0 / rotary_dim)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv[None, :]
    return (torch.from_numpy(np.cos(ang).astype(np.float32)),
            torch.from_numpy(np.sin(ang).astype(np.float32)))


@dataclass
class DecodeCase:
    q: torch.Tensor          # (B, Sq_new, Hq, D)
    k_new: torch.Tensor      # (B, Sq_new, Hkv, D)
    v_new: torch.Tensor
    k_cache: torch.Tensor    # (n_pages, page, Hkv, D) or (B, cap, Hkv, D) when block_table is None
    v_cache: torch.Tensor
    cache_seqlens: torch.Tensor  # int32 (B,)
    block_table: torch.Tensor | None  # int32 (B, max_blocks), -1 padded
    page_size: int
    rotary_cos: torch.Tensor | None
    rotary_sin: torch.Tensor | None
    rotary_dim: int
    scale: float
    causal: bool = True
    name: str = ""
    poison: float = 1.0e4


def decode_case(B=8, Hq=32, Hkv=8, D=128, page=256, seqlens=None, lo=1024, hi=65536,
                seed=5, dtype="bf16", rotary_dim=None, paged=True, poison=1.0e4,
                max_pos=None, name="", sq_new=1) -> DecodeCase:
    """Decode inputs.  Sequence b owns ceil((L_b+sq_new)/page) pages (room for
    the appended tokens); pages come from a seeded permutation of the pool and
    are handed to the sequences in order.  Slots past L_b are filled with
    +/-poison so that any read of them shows up in the output."""
    dt = DTYPES[dtype] if isinstance(dtype, str) else dtype
    rng = np.random.default_rng(seed)
    if seqlens is None:
        L = rng.integers(lo, hi + 1, size=B)
    else:
        L = np.asarray(seqlens, dtype=np.int64)
    L = L.astype(np.int64)
    need = [(int(x) + sq_new + page - 1) // page for x in L]
    n_pages = int(sum(need))
    perm = rng.permutation(n_pages)
    max_blocks = max(need) if seqlens is not None else (hi + 1 + page - 1) // page
    max_blocks = max(max_blocks, max(need))
    bt = np.full((B, max_blocks), -1, dtype=np.int32)
    pos = 0
    for b in range(B):
        bt[b, :need[b]] = perm[pos:pos + need[b]]
        pos += need[b]
    g = make_gen(seed)
    if paged:
        k_cache = randn(g, (n_pages, page, Hkv, D), dt)
        v_cache = randn(g, (n_pages, page, Hkv, D), dt)
    else:
        cap = max_blocks * page
        k_cache = randn(g, (B, cap, Hkv, D), dt)
        v_cache = randn(g, (B, cap, Hkv, D), dt)
    q = randn(g, (B, sq_new, Hq, D), dt)
    k_new = randn(g, (B, sq_new, Hkv, D), dt)
    v_new = randn(g, (B, sq_new, Hkv, D), dt)
    # poison every slot at or past L_b (slot L_b is overwritten by the append)
    sign = torch.where(torch.arange(D) % 2 == 0, 1.0, -1.0).to(dt) * poison
    for b in range(B):
        for j in range(int(L[b]), need[b] * page):
            if paged:
                p, s = int(bt[b, j // page]), j % page
                k_cache[p, s] = sign
                v_cache[p, s] = sign
            else:
                k_cache[b, j] = sign
                v_cache[b, j] = sign
    rd = D if rotary_dim is None else rotary_dim
    if rd > 0:
        mp = int(L.max()) + sq_new + 1 if max_pos is None else max_pos
        cos, sin = rotary_tables(mp, rd)
    else:
        cos = sin = None
    return DecodeCase(q, k_new, v_new, k_cache, v_cache, torch.from_numpy(L.astype(np.int32)),
                      torch.from_numpy(bt) if paged else None, page, cos, sin, rd,
                      1.0 / math.sqrt(D), True, name, poison)


def cfg5(seed=5) -> DecodeCase:
    return decode_case(B=8, Hq=32, Hkv=8, D=128, page=256, seed=seed, max_pos=65537 + 1,
                       name="cfg5_decode_b8_hq32_hkv8_d128_page256")
