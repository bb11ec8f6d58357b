"""Work and traffic counting for the attention workloads (counting only).

FLOP convention (per head, sequence length N, head dimension d):

* forward:  4 N^2 d -- the two N x N x d contractions S = Q K^T and O = P V;
* backward: 10 N^2 d -- five contractions (S recomputed, dV = P^T dO,
  dP = dO V^T, dQ = dS K, dK = dS^T Q);
* causal work is exactly half of the dense count; block-sparse work is the
  kept fraction of the mask's blocks times the dense count.

Compulsory HBM bytes are the bytes the method must move at least once: the
forward reads Q, K, V and writes O and L; the backward reads Q, K, V, O, dO, L
and writes dQ, dK, dV, plus the row term D (written once, read once).  dQ is
accumulated in registers by a query-outer kernel and written once, so no fp32
accumulator travels through memory.

``naive_intermediate_bytes`` is the traffic a pipeline that materialises S and
P would add: write S, read S, write P, read P ("Why is FlashAttention faster?",
"The 4K-token traffic FlashAttention avoids").
"""
from __future__ import annotations

ELT = {"bf16": 2, "fp32": 4}


def work_fraction(N: int, causal: bool, block_mask=None, mask_block: int = 128):
    if block_mask is not None:
        import numpy as np
        bm = np.asarray(block_mask).astype(bool)
        nb = bm.shape[0]
        if N != nb * mask_block:
            raise ValueError("work_fraction expects N to be a multiple of the "
                             "mask block")
        frac = bm.sum() / bm.size
        if causal:
            raise ValueError("causal + block mask work is not counted here")
        return float(frac)
    return 0.5 if causal else 1.0


def fwd_flops(B, H, N, d, causal=False, block_mask=None, mask_block=128):
    return 4.0 * N * N * d * B * H * work_fraction(N, causal, block_mask,
                                                   mask_block)


def bwd_flops(B, H, N, d, causal=False, block_mask=None, mask_block=128):
    return 10.0 * N * N * d * B * H * work_fraction(N, causal, block_mask,
                                                    mask_block)


def fwd_bytes(B, H, N, d, dtype):
    e = ELT[dtype]
    return B * H * (4 * N * d * e + 4 * N)


def bwd_bytes(B, H, N, d, dtype):
    """Q, K, V, O, dO read and dQ, dK, dV written (8 N d elements), L read,
    D written and read (4 N + 8 N bytes), per head."""
    e = ELT[dtype]
    per_head = 8 * N * d * e + 4 * N + 8 * N
    return B * H * per_head


def naive_intermediate_bytes(N: int, dtype: str) -> int:
    """Write S, read S, write P, read P for one head."""
    return 4 * N * N * ELT[dtype]
