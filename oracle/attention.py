"""The definition of exact softmax attention and its gradient, in float64.

Test infrastructure only (see the package docstring for who may import it).

For one head with queries Q (Nq x d), keys K (Nk x d), values V (Nk x d):

* S = scale * Q K^T.  [IO-aware, "Attention is memory-bound"] names the three
  steps (scores, softmax, weighted values); the formulas themselves did not
  survive in the page text, so the reading is the one [Why-faster] states in
  words ("Why is FlashAttention faster on long sequences?": S is Q times K
  transposed, P is softmax of S, O is P times V) with the 1/sqrt(d) scale of
  the plain-code forward listing of [IO-aware] and of [IO-algos] section 4.3.
* Masked positions get S = -inf: causal keeps key <= query; a block mask
  keeps (q, k) when mask[q // mb][k // mb] != 0 (row = query block).  Whole
  masked tiles are what [IO-aware] "Counting the IO" (block-sparse) and
  "FlashAttention-2" (causal) skip.
* P = row softmax of S, computed with the row maximum subtracted
  ([IO-aware], "Online softmax").
* O = P V.
* L = m + ln(sum_k exp(S_qk - m)), the natural-log logsumexp of the scaled
  scores ([IO-aware], "The backward pass: recompute, don't store", and the
  listing's final line, which uses the natural logarithm).
* A row whose keys are all masked has no softmax; the reading taken here is
  O = 0, L = -inf, and no gradient flows through it.

Backward, for the loss sum(O * dO) (the pages print no backward formulas; these
follow from the definition above by the chain rule):

* dV = P^T dO
* dP = dO V^T
* D_q = sum_k P_qk dP_qk          (softmax Jacobian row term)
* dS = P * (dP - D 1^T)
* dQ = scale * dS K,  dK = scale * dS^T Q

[IO-aware] "The backward pass" states that the row term has a closed form from
vectors the forward already produced; ``delta_closed_form`` is that form,
D = rowsum(dO * O), and the tests pin the identity with the definition above.
"""
from __future__ import annotations

import numpy as np


def keep_matrix(nq: int, nk: int, causal: bool = False, block_mask=None,
                mask_block: int = 128, q_rows=None,
                causal_offset: int = 0, kv_len=None) -> np.ndarray:
    """Boolean [len(q_rows), nk]: True where query q may attend to key k.

    Causal keeps k <= q + causal_offset.  With equal query and key lengths
    the offset is 0; when fewer queries than keys are given (decoding against
    a key/value cache) the reading taken is that the queries are the last
    positions of the key sequence, offset = nk - nq.
    """
    rows = np.arange(nq) if q_rows is None else np.asarray(q_rows)
    cols = np.arange(nk)
    keep = np.ones((rows.size, nk), dtype=bool)
    if causal:
        keep &= cols[None, :] <= rows[:, None] + causal_offset
    if block_mask is not None:
        bm = np.asarray(block_mask).astype(bool)
        keep &= bm[rows[:, None] // mask_block, cols[None, :] // mask_block]
    if kv_len is not None:
        keep &= cols[None, :] < kv_len      # key padding: keys >= kv_len
    return keep


def softmax_rows(S: np.ndarray):
    """Row softmax with the row max subtracted; all -inf rows give zeros.

    Returns (P, m, l) with m the row max (-inf for empty rows) and
    l = sum_k exp(S_qk - m).
    """
    m = S.max(axis=1)
    nonempty = np.isfinite(m)
    m_shift = np.where(nonempty, m, 0.0)
    E = np.exp(S - m_shift[:, None])
    l = E.sum(axis=1)
    P = E / np.where(nonempty, l, 1.0)[:, None]
    return P, m, l


def forward_head(q, k, v, scale, causal=False, block_mask=None,
                 mask_block=128, q_rows=None, causal_offset=0, kv_len=None,
                 drop_keep=None, drop_scale=1.0):
    """O (rows x d) and L (rows) for one head.

    ``q_rows`` selects which query rows to compute (default: all).  Rows are
    independent, so a subset is computed exactly as in the full call.
    ``causal_offset``, ``kv_len``: see ``keep_matrix``.

    Dropout (``drop_keep``: boolean [rows, Nk], True = kept): applied to the
    normalised probabilities, O = ((P * keep) * drop_scale) V; L is the
    logsumexp of the scores, unaffected.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    rows = np.arange(q.shape[0]) if q_rows is None else np.asarray(q_rows)
    S = scale * (q[rows] @ k.T)
    keep = keep_matrix(q.shape[0], k.shape[0], causal, block_mask, mask_block,
                       q_rows=rows, causal_offset=causal_offset, kv_len=kv_len)
    S = np.where(keep, S, -np.inf)
    P, m, l = softmax_rows(S)
    if drop_keep is not None:
        O = (np.where(drop_keep, P, 0.0) * drop_scale) @ v
    else:
        O = P @ v
    nonempty = np.isfinite(m)
    L = np.where(nonempty, m + np.log(np.where(nonempty, l, 1.0)), -np.inf)
    return O, L


def backward_head(q, k, v, do, scale, causal=False, block_mask=None,
                  mask_block=128, kv_len=None, drop_keep=None,
                  drop_scale=1.0):
    """(dQ, dK, dV, D) for one head, from the definition (no recomputation
    tricks: P is formed explicitly, D from P and dP).

    With dropout (O = (P * Z * s) V for the keep matrix Z and scale s):
    dV = (P * Z * s)^T dO; the gradient reaching P is dP = (dO V^T) * Z * s;
    D_q = sum_k P_qk dP_qk; dS = P * (dP - D), and dQ, dK as without it.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    S = scale * (q @ k.T)
    keep = keep_matrix(q.shape[0], k.shape[0], causal, block_mask, mask_block,
                       kv_len=kv_len)
    S = np.where(keep, S, -np.inf)
    P, _, _ = softmax_rows(S)
    if drop_keep is not None:
        Z = np.where(drop_keep, drop_scale, 0.0)
        dV = (P * Z).T @ do
        dP = (do @ v.T) * Z
    else:
        dV = P.T @ do
        dP = do @ v.T
    D = (P * dP).sum(axis=1)
    dS = P * (dP - D[:, None])
    dQ = scale * (dS @ k)
    dK = scale * (dS.T @ q)
    return dQ, dK, dV, D


def delta_closed_form(o, do):
    """D_q = sum_j dO_qj O_qj, the closed form the backward uses
    ([IO-aware], "The backward pass: recompute, don't store")."""
    return (np.asarray(o, np.float64) * np.asarray(do, np.float64)).sum(-1)


def forward(q, k, v, scale, causal=False, block_mask=None, mask_block=128,
            heads=None, row_chunk=None):
    """O [B,H,N,d] and L [B,H,N] over every head (or the (b, h) pairs in
    ``heads``, others left NaN).  ``row_chunk`` bounds memory by computing
    query rows in independent groups."""
    B, H, N, d = q.shape
    O = np.full((B, H, N, d), np.nan)
    L = np.full((B, H, N), np.nan)
    todo = heads if heads is not None else [(b, h) for b in range(B)
                                           for h in range(H)]
    for b, h in todo:
        if row_chunk is None:
            O[b, h], L[b, h] = forward_head(q[b, h], k[b, h], v[b, h], scale,
                                            causal, block_mask, mask_block)
        else:
            for r0 in range(0, N, row_chunk):
                rows = np.arange(r0, min(N, r0 + row_chunk))
                O[b, h, rows], L[b, h, rows] = forward_head(
                    q[b, h], k[b, h], v[b, h], scale, causal, block_mask,
                    mask_block, q_rows=rows)
    return O, L


def backward(q, k, v, do, scale, causal=False, block_mask=None,
             mask_block=128, heads=None):
    """dQ, dK, dV [B,H,N,d] over every head (or the listed (b, h) pairs)."""
    B, H, N, d = q.shape
    dQ = np.full((B, H, N, d), np.nan)
    dK = np.full((B, H, N, d), np.nan)
    dV = np.full((B, H, N, d), np.nan)
    todo = heads if heads is not None else [(b, h) for b in range(B)
                                           for h in range(H)]
    for b, h in todo:
        dQ[b, h], dK[b, h], dV[b, h], _ = backward_head(
            q[b, h], k[b, h], v[b, h], do[b, h], scale, causal, block_mask,
            mask_block)
    return dQ, dK, dV
