"""Split-KV forward by the merge rule, in float64, for checking the oracle.

Test infrastructure only.  [IO-aware] "In practice" describes
Flash-Decoding: the keys of one query row are split into runs processed
independently, and the partial results are combined with the logsumexp
rescaling of the online softmax.  For runs s with partial (normalised)
outputs O_s and logsumexps L_s over their own keys,

    L = ln sum_s exp(L_s),      O = sum_s exp(L_s - L) O_s,

because exp(L_s) is run s's share of the row's softmax denominator.  A run
with no unmasked key for a row has L_s = -inf and weighs zero.

``split_forward_head`` takes these steps with ``attention.forward_head`` on
each run; the tests show it reproduces ``forward_head`` over all keys (and the
worked example of ``tests/golden``).  The GPU split-KV path is compared with
``forward_head`` directly, since the split result is exact up to rounding.
"""
from __future__ import annotations

import numpy as np

from .attention import forward_head


def split_forward_head(q, k, v, scale, bounds, causal=False,
                       causal_offset=0):
    """O and L over all keys, from the runs of keys [bounds[i], bounds[i+1]).

    Each run keeps its keys' absolute positions for the causal rule
    (k <= q + causal_offset).  Returns (O, L, parts) with parts the list of
    per-run (O_s, L_s).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    nq = q.shape[0]
    parts = []
    for a, b in zip(bounds[:-1], bounds[1:]):
        # Keys a..b-1 only: causal position k <= q + off becomes
        # (k - a) <= q + (off - a) on the run's own key index.
        O_s, L_s = forward_head(q, k[a:b], v[a:b], scale, causal,
                                causal_offset=causal_offset - a)
        parts.append((O_s, L_s))
    Ls = np.stack([p[1] for p in parts])             # [runs, nq]
    m = Ls.max(axis=0)
    seen = np.isfinite(m)
    w = np.where(seen[None, :], np.exp(Ls - np.where(seen, m, 0.0)[None, :]),
                 0.0)                                  # [runs, nq]
    tot = w.sum(axis=0)
    L = np.where(seen, m + np.log(np.where(seen, tot, 1.0)), -np.inf)
    O = np.zeros((nq, v.shape[1]))
    for (O_s, _), w_s in zip(parts, w):
        O += w_s[:, None] * O_s
    O = np.where(seen[:, None], O / np.where(seen, tot, 1.0)[:, None], 0.0)
    return O, L, parts
