"""Dropout keep masks from a counter-based generator, in integers -- TEST
INFRASTRUCTURE ONLY (see the package docstring for who may import it).

The pages name dropout among the element-wise steps attention fuses
([IO-aware] "Attention is memory-bound"; [Why-faster] "Extra computation can
still finish sooner") but give no generator.  Random numbers that the method
draws inside the kernel cannot be passed in, so both sides implement one
published counter-based generator: Philox4x32-10 (Salmon, Moraes, Dror and
Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011), written here
from that definition:

* state: four 32-bit counter words (c0, c1, c2, c3) and two key words
  (k0, k1);
* one round: (hi0, lo0) = 0xD2511F53 * c0 and (hi1, lo1) = 0xCD9E8D57 * c2 as
  64-bit products split into halves; the new state is
  (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0);
* the key is bumped by (0x9E3779B9, 0xBB67AE85) between rounds; ten rounds.

Readings (the pages give none of this):

* the 64-bit seed is the key (k0 = low word, k1 = high word);
* one generator call serves a 4 x 4 block of (query, key) positions of one
  (b, h): counter = (key // 4, query // 4, h, b); its 16 output bytes, taken
  little-endian from the four words in order, belong to (query 4 qq + r,
  key 4 kq + c) at byte 4 r + c;
* the drop probability is quantised to 1/256: p8 = floor(256 p + 1/2), an
  element is kept when its byte is >= p8, and kept probabilities are scaled
  by 256 / (256 - p8), so the expectation of the dropped output equals the
  undropped one exactly.
"""
from __future__ import annotations

import numpy as np

M0, M1 = 0xD2511F53, 0xCD9E8D57
W0, W1 = 0x9E3779B9, 0xBB67AE85
MASK32 = 0xFFFFFFFF


def philox4x32_10(c0, c1, c2, c3, k0: int, k1: int):
    """Philox4x32-10 on broadcastable uint32 counter arrays; returns the four
    output words as uint64 arrays holding 32-bit values."""
    c = [np.asarray(x, dtype=np.uint64) & MASK32 for x in (c0, c1, c2, c3)]
    c = np.broadcast_arrays(*c)
    c = [x.copy() for x in c]
    k0, k1 = int(k0) & MASK32, int(k1) & MASK32
    for rnd in range(10):
        if rnd:
            k0 = (k0 + W0) & MASK32
            k1 = (k1 + W1) & MASK32
        p0 = np.uint64(M0) * c[0]
        p1 = np.uint64(M1) * c[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & np.uint64(MASK32)
        hi1, lo1 = p1 >> np.uint64(32), p1 & np.uint64(MASK32)
        c = [hi1 ^ c[1] ^ np.uint64(k0), lo1, hi0 ^ c[3] ^ np.uint64(k1), lo0]
    return c


def quantize_p(p: float) -> int:
    """p8 = floor(256 p + 1/2); p must give 0 <= p8 <= 255."""
    if not (0.0 <= p < 1.0):
        raise ValueError("dropout probability must be in [0, 1)")
    p8 = int(np.floor(256.0 * p + 0.5))
    if p8 > 255:
        raise ValueError("dropout probability rounds to 1")
    return p8


def drop_scale(p8: int) -> float:
    return 256.0 / (256 - p8)


def keep_bytes(b: int, h: int, nq: int, nk: int, seed: int,
               q_rows=None) -> np.ndarray:
    """uint8 [rows, nk]: the generator byte of every (query, key) of head
    (b, h)."""
    rows = np.arange(nq) if q_rows is None else np.asarray(q_rows)
    cols = np.arange(nk)
    qq, kq = rows[:, None] // 4, cols[None, :] // 4
    words = philox4x32_10(kq, qq, h, b, seed & MASK32, (seed >> 32) & MASK32)
    r, c = (rows[:, None] % 4), (cols[None, :] % 4)
    byte = 4 * r + c                     # byte index inside the 16 bytes
    w = byte // 4                        # = r
    out = np.zeros((rows.size, nk), dtype=np.uint64)
    for i in range(4):
        out = np.where(w == i, words[i], out)
    shift = (8 * (byte % 4)).astype(np.uint64)
    return ((out >> shift) & np.uint64(0xFF)).astype(np.uint8)


def keep_mask(b: int, h: int, nq: int, nk: int, p8: int, seed: int,
              q_rows=None) -> np.ndarray:
    """Boolean [rows, nk]: True where the element is kept."""
    return keep_bytes(b, h, nq, nk, seed, q_rows) >= p8
