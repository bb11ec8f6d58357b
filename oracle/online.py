"""The tiled online-softmax recurrence, in float64, for checking the oracle.

Test infrastructure only.  This is the algorithm of [IO-aware] ("Tiling: never
materialise S", "Online softmax", and the plain-code forward pass after "In
practice"), restated with whole-tile numpy operations:

* queries are processed in blocks of Br rows, keys/values in blocks of Bc
  columns; the last block of either may be short (ragged tail);
* each query row carries a running maximum m (starting at -inf), a running
  sum l of exp(s - m) and an unnormalised output acc;
* for every key tile the new maximum is m_new = max(m, rowmax(S_tile)), the
  correction exp(m - m_new) shrinks l and acc, and the tile's exp(S - m_new)
  are added to l and, weighted by V, to acc;
* after the last tile O = acc / l and L = m + ln l (the delayed normalisation
  and single statistic of [IO-aware], "FlashAttention-2").

Masked scores are -inf.  A row that has seen no unmasked key yet keeps
m = -inf; its correction is taken as 0 rather than evaluating
exp(-inf - (-inf)).  The function exists to show, on tiny inputs, that this
recurrence reproduces ``attention.forward_head``; the GPU path is compared with
``attention.forward_head`` directly.
"""
from __future__ import annotations

import numpy as np

from .attention import keep_matrix


def online_forward_head(q, k, v, scale, Br=64, Bc=64, causal=False,
                        block_mask=None, mask_block=128, trace=None):
    """O and L by the tiled recurrence.  If ``trace`` is a list, the state
    (row block start, key block start, m, l, acc) after each tile is appended.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    N, d = q.shape
    Nk = k.shape[0]
    O = np.zeros((N, d))
    L = np.zeros(N)
    for i0 in range(0, N, Br):
        rows = np.arange(i0, min(N, i0 + Br))
        m = np.full(rows.size, -np.inf)
        l = np.zeros(rows.size)
        acc = np.zeros((rows.size, d))
        for j0 in range(0, Nk, Bc):
            cols = np.arange(j0, min(Nk, j0 + Bc))
            s = scale * (q[rows] @ k[cols].T)
            keep = keep_matrix(N, Nk, causal, block_mask, mask_block,
                               q_rows=rows)[:, cols]
            s = np.where(keep, s, -np.inf)
            m_new = np.maximum(m, s.max(axis=1))
            seen = np.isfinite(m_new)
            ref = np.where(seen, m_new, 0.0)
            correction = np.where(np.isfinite(m), np.exp(m - ref), 0.0)
            p = np.exp(s - ref[:, None])
            l = l * correction + p.sum(axis=1)
            acc = acc * correction[:, None] + p @ v[cols]
            m = m_new
            if trace is not None:
                trace.append((i0, j0, m.copy(), l.copy(), acc.copy()))
        nonempty = l > 0
        O[rows] = np.where(nonempty[:, None],
                           acc / np.where(nonempty, l, 1.0)[:, None], 0.0)
        L[rows] = np.where(nonempty, m + np.log(np.where(nonempty, l, 1.0)),
                           -np.inf)
    return O, L
