"""The tiled online-softmax recurrence, in float64, for checking the oracle.

Test infrastructure only.  [IO-aware] ("Tiling: never materialise S" and
"Online softmax") computes one row's softmax-weighted sum of values tile by
tile, carrying a running maximum and a running sum that are rescaled
whenever the maximum grows.  Restated here through the state of a row over
a set of keys,

    m = the largest score,   l = sum exp(s - m),   a = sum exp(s - m) v,

(an empty set: m = -inf, l = 0, a = 0).  The states of two disjoint key
sets combine exactly: with M = max(m1, m2),

    l = l1 exp(m1 - M) + l2 exp(m2 - M),   a = a1 exp(m1 - M) + a2 exp(m2 - M),

where a set with m = -inf contributes nothing (its factor is taken as 0,
never as exp(-inf - (-inf))).  Folding the key tiles one at a time into the
running state is the recurrence of the page; the same combination merges the
partial results of independent key runs in Flash-Decoding ([IO-aware], "In
practice").  After the last tile O = a / l and L = m + ln l (the delayed
normalisation and single statistic of [IO-aware], "FlashAttention-2").

Query rows are taken in blocks of Br and keys in tiles of Bc; either last
block may be short.  The function exists to show, on small inputs, that the
tiled computation reproduces ``attention.forward_head``; the GPU path is
compared with ``attention.forward_head`` directly.
"""
from __future__ import annotations

import numpy as np

from .attention import keep_matrix


def empty_state(rows: int, d: int):
    """The state of an empty key set for `rows` query rows."""
    return np.full(rows, -np.inf), np.zeros(rows), np.zeros((rows, d))


def tile_state(s: np.ndarray, v: np.ndarray):
    """State of one key tile: s [rows, c] scaled scores (-inf where
    masked), v [c, d] its values."""
    m = s.max(axis=1)
    seen = np.isfinite(m)
    e = np.exp(s - np.where(seen, m, 0.0)[:, None])   # 0 where s = -inf
    return m, e.sum(axis=1), e @ v


def merge(x, y):
    """The state of the union of two disjoint key sets."""
    (m1, l1, a1), (m2, l2, a2) = x, y
    m = np.maximum(m1, m2)
    ref = np.where(np.isfinite(m), m, 0.0)
    f1 = np.where(np.isfinite(m1), np.exp(m1 - ref), 0.0)
    f2 = np.where(np.isfinite(m2), np.exp(m2 - ref), 0.0)
    return m, l1 * f1 + l2 * f2, a1 * f1[:, None] + a2 * f2[:, None]


def online_forward_head(q, k, v, scale, Br=64, Bc=64, causal=False,
                        block_mask=None, mask_block=128, trace=None):
    """O and L by folding key tiles into a running state.  If ``trace`` is
    a list, (row block start, key tile start, m, l, a) is appended after
    each tile."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    n, d = q.shape
    nk = k.shape[0]
    O = np.zeros((n, d))
    L = np.zeros(n)
    for i0 in range(0, n, Br):
        rows = np.arange(i0, min(n, i0 + Br))
        keep = keep_matrix(n, nk, causal, block_mask, mask_block, q_rows=rows)
        state = empty_state(rows.size, d)
        for j0 in range(0, nk, Bc):
            cols = slice(j0, min(nk, j0 + Bc))
            s = np.where(keep[:, cols], scale * (q[rows] @ k[cols].T),
                         -np.inf)
            state = merge(state, tile_state(s, v[cols]))
            if trace is not None:
                trace.append((i0, j0) + tuple(x.copy() for x in state))
        m, l, a = state
        seen = l > 0
        O[rows] = np.where(seen[:, None],
                           a / np.where(seen, l, 1.0)[:, None], 0.0)
        L[rows] = np.where(seen, m + np.log(np.where(seen, l, 1.0)), -np.inf)
    return O, L
