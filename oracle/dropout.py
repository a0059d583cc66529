"""Attention-dropout mask oracle — test infrastructure only.

The pages pass ``dropout_p`` to the attention call in their usage examples
(page "FlashAttention 实战指南：如何把训练内存省 20 倍、速度提 4 倍", section
"上手 FlashAttention 的三步走", and the interface listing of page
"终极指南：如何通过FlashAttention实现Transformer模型的4倍加速与20倍内存优化")
but define neither the random generator nor which element gets which
random number.  The readings taken here:

* dropout acts on the normalised attention weights: O = (P * K / (1 - p)) V
  with K_ij in {0, 1}; the log-sum-exp stays that of the undropped P;
* the random numbers come from the counter-based generator Philox4x32-10
  (J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel random
  numbers: as easy as 1, 2, 3", SC 2011), keyed by the 64-bit seed;
* one generator call covers a 4 x 4 block of (query row, key) pairs of one
  (batch entry, query head): counter = (j // 4, i // 4, b * Hq + h,
  offset mod 2^32); word i % 4 of the output holds the block's query row,
  byte j % 4 of that word (bits 8 (j % 4) .. 8 (j % 4) + 7) the key;
* a pair is dropped when its byte is below t = round(256 p) (ties to even),
  so the drop probability is t / 256 and kept weights are scaled by
  256 / (256 - t); 0 <= p < 255.5 / 256.

For packed variable-length batches b is the sequence index and i, j are
positions within the sequence.
"""
from __future__ import annotations

import numpy as np

# Philox multipliers and Weyl key increments (Salmon et al., 2011), for 32-
# and 64-bit words.
PHILOX_M = {32: (0xD2511F53, 0xCD9E8D57), 64: (0xD2E7470EE14C6C93, 0xCA5A826395121157)}
PHILOX_W = {32: (0x9E3779B9, 0xBB67AE85), 64: (0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B)}


def philox4(counter, key, width=32, rounds=10):
    """Philox4xW-R on four counter words and two key words.

    Each round multiplies counter words 0 and 2 by the two multipliers; the
    new words are (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0), and the key
    advances by the Weyl increments between rounds.  width 32 takes numpy
    arrays of counters (products formed exactly in uint64); width 64 takes
    Python integers.  Returns the four output words."""
    m0, m1 = PHILOX_M[width]
    w0, w1 = PHILOX_W[width]
    mask = (1 << width) - 1
    if width == 32:
        c = [np.asarray(x, dtype=np.uint64) & np.uint64(mask) for x in counter]
        k0, k1 = np.uint64(key[0] & mask), np.uint64(key[1] & mask)
        m0, m1 = np.uint64(m0), np.uint64(m1)
        sh, mk = np.uint64(32), np.uint64(mask)
        for _ in range(rounds):
            p0 = m0 * c[0]
            p1 = m1 * c[2]
            c = [(p1 >> sh) ^ c[1] ^ k0, p1 & mk, (p0 >> sh) ^ c[3] ^ k1, p0 & mk]
            k0 = np.uint64((int(k0) + w0) & mask)
            k1 = np.uint64((int(k1) + w1) & mask)
        return [x.astype(np.uint32) for x in c]
    c = [int(x) & mask for x in counter]
    k0, k1 = key[0] & mask, key[1] & mask
    for _ in range(rounds):
        p0 = m0 * c[0]
        p1 = m1 * c[2]
        c = [(p1 >> width) ^ c[1] ^ k0, p1 & mask, (p0 >> width) ^ c[3] ^ k1, p0 & mask]
        k0 = (k0 + w0) & mask
        k1 = (k1 + w1) & mask
    return c


def threshold(p):
    """Byte threshold t = round(256 p), ties to even."""
    p = float(p)
    if not (0.0 <= p < 255.5 / 256.0):
        raise ValueError("dropout_p must lie in [0, 255.5/256)")
    return int(np.rint(p * 256.0))


def keep_scale(p):
    """Scale of kept weights, 256 / (256 - t)."""
    return 256.0 / (256.0 - threshold(p))


def keep_mask(p, seed, offset, bh, rows, cols):
    """Boolean (len(rows), len(cols)) keep mask of one (batch entry, query
    head) pair, bh = b * Hq + h, for query rows ``rows`` and keys ``cols``."""
    t = threshold(p)
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    if t == 0:
        return np.ones((len(rows), len(cols)), dtype=bool)
    i = rows[:, None]
    j = cols[None, :]
    shape = np.broadcast_shapes(i.shape, j.shape)
    c0 = np.broadcast_to(j // 4, shape)
    c1 = np.broadcast_to(i // 4, shape)
    c2 = np.full(shape, bh, dtype=np.int64)
    c3 = np.full(shape, int(offset) & 0xFFFFFFFF, dtype=np.int64)
    seed = int(seed) & ((1 << 64) - 1)
    words = philox4([c0, c1, c2, c3], (seed & 0xFFFFFFFF, seed >> 32))
    wsel = np.broadcast_to(i % 4, shape)
    word = np.choose(wsel, words)
    byte = (word >> (8 * np.broadcast_to(j % 4, shape)).astype(np.uint32)) & np.uint32(0xFF)
    return byte >= t
