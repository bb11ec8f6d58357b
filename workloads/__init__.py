"""Seeded synthetic inputs for exact attention, shared by the tests, the benchmark
and the smoke check.

This module holds no attention arithmetic.  It only draws random numbers, rounds
them once to the storage dtype, and builds the block-sparsity mask.  Both the
fp64 oracle and the HIP path receive the arrays it returns; neither side's
results ever flow back into it.

Workloads (scale 1/sqrt(d) everywhere, Q/K/V/dO drawn in that order from
``numpy.random.Generator(PCG64(seed))`` as iid N(0,1) fp64, then rounded once
with round-to-nearest-even to the storage dtype):

* ``c1``  B=1  H=1  N=256   d=64  fp32, dense
* ``c2``  B=4  H=16 N=1024  d=64  bf16, dense
* ``c3``  B=2  H=32 N=4096  d=128 bf16, causal (the headline workload)
* ``c4f`` B=1  H=16 N=16384 d=128 bf16, causal, K scaled x3, forward only
* ``c4b`` B=1  H=16 N=8192  d=128 bf16, causal, K scaled x3, forward+backward
* ``c5``  B=2  H=16 N=8192  d=64  bf16, 128x128 block mask: the |i-j|<=1 band
  plus exactly floor(0.25 * off-band) other blocks chosen uniformly without
  replacement, drawn after dO from the same generator; one mask shared by all
  (b, h).

The sizes mirror the shapes the pages discuss: the 4K-token, d=128, bf16 head of
"Why is FlashAttention faster?" ("The 4K-token traffic FlashAttention avoids"),
the N=1024, d=64, 16-head A100 experiment of the same page ("Extra computation
can still finish sooner"), long sequences with sharp softmax rows, and the
block-sparse variant of "FlashAttention: making attention IO-aware" ("Counting
the IO").
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "get", "round_to_dtype", "round_bf16",
    "bf16_bits", "make_inputs", "band_random_block_mask", "small_case",
    "KvWorkload", "KV_WORKLOADS", "make_kv_inputs", "make_varlen_inputs",
    "varlen_lengths", "hadamard_signs", "outlier_inputs",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    D: int
    dtype: str            # "fp32" or "bf16"
    causal: bool
    seed: int
    k_scale: float = 1.0  # K multiplied by this in fp64 before rounding
    mask_block: int = 0   # 0 = no block mask
    mask_band: int = 0    # |i - j| <= band blocks always kept
    mask_frac: float = 0.0  # fraction of the off-band blocks kept
    backward: bool = True
    softmax_scale: Optional[float] = None  # None: 1/sqrt(D)

    @property
    def scale(self) -> float:
        if self.softmax_scale is not None:
            return float(self.softmax_scale)
        return 1.0 / math.sqrt(self.D)

    @property
    def shape(self):
        return (self.B, self.H, self.N, self.D)

    @property
    def has_mask(self) -> bool:
        return self.mask_block > 0


WORKLOADS = {
    "c1": Workload("c1", 1, 1, 256, 64, "fp32", False, 1),
    "c2": Workload("c2", 4, 16, 1024, 64, "bf16", False, 2),
    "c3": Workload("c3", 2, 32, 4096, 128, "bf16", True, 3),
    "c4f": Workload("c4f", 1, 16, 16384, 128, "bf16", True, 4, k_scale=3.0,
                    backward=False),
    "c4b": Workload("c4b", 1, 16, 8192, 128, "bf16", True, 40, k_scale=3.0),
    "c5": Workload("c5", 2, 16, 8192, 64, "bf16", False, 5, mask_block=128,
                   mask_band=1, mask_frac=0.25),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def small_case(name: str, B: int, H: int, N: int, D: int, dtype: str,
               causal: bool, seed: int, k_scale: float = 1.0,
               mask_block: int = 0, mask_band: int = 0,
               mask_frac: float = 0.0,
               scale: Optional[float] = None) -> Workload:
    """A reduced workload with the same recipe (used by parity tests);
    ``scale`` overrides the softmax scale 1/sqrt(D)."""
    return Workload(name, B, H, N, D, dtype, causal, seed, k_scale,
                    mask_block, mask_band, mask_frac, softmax_scale=scale)


# ----------------------------------------------------------------- rounding

def round_bf16(x) -> np.ndarray:
    """Round fp64 values once, to nearest-even, onto the bfloat16 grid.

    bfloat16 keeps 8 significant bits.  With x = m * 2**e and 0.5 <= |m| < 1,
    the nearest representable value is rint(m * 2**8) * 2**(e - 8); numpy's
    rint rounds halves to even.  Inputs must be finite and inside the normal
    bf16 range (true for every workload here).
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("round_bf16: non-finite input")
    ax = np.abs(x[x != 0])
    if ax.size and (ax.min() < 2.0 ** -126 or ax.max() >= 2.0 ** 127):
        raise ValueError("round_bf16: value outside the normal bf16 range")
    m, e = np.frexp(x)
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def round_to_dtype(x, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "fp32":
        return np.asarray(x, np.float64).astype(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype}")


def bf16_bits(x_rounded: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of values already on the bf16 grid (exact)."""
    f = np.ascontiguousarray(x_rounded, dtype=np.float64).astype(np.float32)
    bits = f.view(np.uint32)
    if np.any(bits & 0xFFFF):
        raise ValueError("bf16_bits: value is not on the bf16 grid")
    return (bits >> 16).astype(np.uint16)


# ------------------------------------------------------------ block mask

def band_random_block_mask(n_blocks: int, band: int, frac: float,
                           rng: np.random.Generator) -> np.ndarray:
    """uint8 [n_blocks, n_blocks] mask, row = query block, column = key block.

    Keeps every block with |i - j| <= band, plus exactly floor(frac * n_off)
    of the n_off other blocks, chosen uniformly without replacement.
    """
    i = np.arange(n_blocks)[:, None]
    j = np.arange(n_blocks)[None, :]
    band_keep = np.abs(i - j) <= band
    off = np.flatnonzero(~band_keep.ravel())
    n_pick = int(math.floor(frac * off.size))
    picked = rng.choice(off, size=n_pick, replace=False)
    mask = band_keep.ravel().copy()
    mask[picked] = True
    return mask.reshape(n_blocks, n_blocks).astype(np.uint8)


# ---------------------------------------------------------------- inputs

def make_inputs(w: Workload, with_grad: Optional[bool] = None) -> dict:
    """Draw the workload's inputs.

    Returns a dict of fp64 numpy arrays whose values lie exactly on the
    storage dtype's grid: ``q``, ``k``, ``v``, ``do`` (shape [B,H,N,D]) and
    ``block_mask`` (uint8 [nb, nb] or None).  The draw order is fixed
    (Q, K, V, dO, then the mask), so the mask of a workload does not depend
    on whether dO is used.
    """
    rng = np.random.Generator(np.random.PCG64(w.seed))
    shape = w.shape
    q = rng.standard_normal(shape)
    k = rng.standard_normal(shape) * w.k_scale
    v = rng.standard_normal(shape)
    do = rng.standard_normal(shape)
    mask = None
    if w.has_mask:
        nb = -(-w.N // w.mask_block)
        mask = band_random_block_mask(nb, w.mask_band, w.mask_frac, rng)
    out = {
        "q": round_to_dtype(q, w.dtype),
        "k": round_to_dtype(k, w.dtype),
        "v": round_to_dtype(v, w.dtype),
        "do": round_to_dtype(do, w.dtype),
        "block_mask": mask,
    }
    return out


@dataclasses.dataclass(frozen=True)
class KvWorkload:
    """Queries against a longer key/value sequence (decoding against a
    cache, "FlashAttention: making attention IO-aware", "In practice")."""
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    D: int
    causal: bool          # keys <= query + (Nk - Nq)
    seed: int
    num_splits: int = 16
    dtype: str = "bf16"
    k_scale: float = 1.0
    softmax_scale: Optional[float] = None  # None: 1/sqrt(D)

    @property
    def scale(self) -> float:
        if self.softmax_scale is not None:
            return float(self.softmax_scale)
        return 1.0 / math.sqrt(self.D)


# A decode step of a batch of 4 sequences, 32 heads of d = 128, one new
# query each against a 16384-token key/value cache.
KV_WORKLOADS = {
    "dec": KvWorkload("dec", 4, 32, 1, 16384, 128, True, 6, num_splits=4),
}


def make_kv_inputs(w: KvWorkload) -> dict:
    """Q [B,H,Nq,D], K and V [B,H,Nk,D], drawn in that order as iid N(0,1)
    fp64 from PCG64(seed) (K times k_scale), rounded once to the dtype."""
    rng = np.random.Generator(np.random.PCG64(w.seed))
    q = rng.standard_normal((w.B, w.H, w.Nq, w.D))
    k = rng.standard_normal((w.B, w.H, w.Nk, w.D)) * w.k_scale
    v = rng.standard_normal((w.B, w.H, w.Nk, w.D))
    return {"q": round_to_dtype(q, w.dtype), "k": round_to_dtype(k, w.dtype),
            "v": round_to_dtype(v, w.dtype)}


def varlen_lengths(n_seqs: int, lo: int, hi: int, seed: int) -> list:
    """A seeded mix of sequence lengths, uniform on [lo, hi]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return [int(x) for x in rng.integers(lo, hi + 1, size=n_seqs)]


def padding_workload() -> "Workload":
    """Batch 64, 16 heads, N = 1024, d = 64, bf16, no causal mask: the shape
    of the key-padding experiment in "Why is FlashAttention faster?" ("Extra
    computation can still finish sooner")."""
    return small_case("pad", 64, 16, 1024, 64, "bf16", False, seed=11)


def padding_lengths(B: int, N: int, seed: int = 12) -> list:
    """Seeded valid-key counts per batch entry for the key-padding workload:
    uniform on [N/4, N] (the page does not give its padding distribution)."""
    return varlen_lengths(B, N // 4, N, seed)


def make_varlen_inputs(lengths, H: int, D: int, seed: int,
                       dtype: str = "bf16") -> dict:
    """A packed batch of sequences of the given lengths: Q, K, V, dO as
    [total, H, D] iid N(0,1) fp64 (drawn in that order from PCG64(seed)),
    rounded once to the dtype, and the int32 row offsets ``cu_seqlens``."""
    rng = np.random.Generator(np.random.PCG64(seed))
    total = int(sum(lengths))
    out = {}
    for name in ("q", "k", "v", "do"):
        out[name] = round_to_dtype(rng.standard_normal((total, H, D)), dtype)
    out["cu_seqlens"] = np.concatenate(
        [[0], np.cumsum(lengths)]).astype(np.int32)
    return out


def hadamard_signs(D: int, seed: int) -> np.ndarray:
    """The random sign vector of a rotation diag(signs) H_D: D values of +-1,
    each -1 with probability 1/2, from PCG64(seed)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return np.where(rng.random(D) < 0.5, -1.0, 1.0)


def outlier_inputs(N: int, D: int, seed: int, B: int = 1, H: int = 1,
                   frac: float = 0.001, std: float = 10.0,
                   dtype: str = "bf16") -> dict:
    """Q, K, V [B,H,N,D] with outliers: iid N(0,1) plus, at a fraction
    ``frac`` of the entries (chosen independently), an extra N(0, std^2)
    term; drawn in the order Q, K, V (for each: base, selection, extra) from
    PCG64(seed), rounded once to the dtype.  Also returns the rotation signs
    drawn afterwards from the same generator.  The mix is the kind of
    heavy-tailed activation that "FlashAttention-3: Hopper asynchrony and
    FP8" says FP8 handles badly."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = {}
    shape = (B, H, N, D)
    for name in ("q", "k", "v"):
        x = rng.standard_normal(shape)
        pick = rng.random(shape) < frac
        x = x + pick * rng.standard_normal(shape) * std
        out[name] = round_to_dtype(x, dtype)
    out["signs"] = np.where(rng.random(D) < 0.5, -1.0, 1.0)
    return out


def to_torch(x: np.ndarray, dtype: str, device="cpu"):
    """Exact conversion of grid values to a torch tensor of the storage dtype."""
    import torch
    if dtype == "bf16":
        bits = bf16_bits(x)
        t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    elif dtype == "fp32":
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    else:
        raise ValueError(dtype)
    return t.to(device)
