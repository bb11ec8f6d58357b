"""FP8 forward with incoherent processing, in float64 -- TEST INFRASTRUCTURE ONLY.

Who may import this: see the package docstring.  Nothing here is shared with
the HIP path.

[IO-aware] "FlashAttention-3: Hopper asynchrony and FP8" describes the method
in one item: FP8 halves the cost of the matrix products again but suffers from
outliers, so the inputs are quantised per block, and Q and K are first
multiplied by a random orthogonal matrix built from a Hadamard matrix, which
spreads an outlier's mass over all dimensions; the result is reported as 2.6x
less error than plain FP8 attention.  The page gives no formulas.  The
readings taken here (each one is listed with its reason in the design notes):

* FP8 = the OCP E4M3 format without infinities ("E4M3FN"): 1 sign bit, 4
  exponent bits (bias 7), 3 mantissa bits, largest finite value 448,
  subnormals m * 2^-9.  Conversion rounds to nearest, ties to even.
* Rotation: M = diag(signs) H_d with H_d the d x d Sylvester Hadamard matrix
  (entries +-1) and `signs` a caller-drawn vector of +-1; Q' = Q M and
  K' = K M.  M M^T = d I, so Q' K'^T = d Q K^T and the softmax scale is
  divided by d (a power of two: exact).  V is not rotated (the page rotates
  Q and K only).
* Blocks: 64 consecutive rows of one head (the last block of a head may be
  shorter) share one scale.  The scale is a power of two, 2^e with e the
  smallest integer such that the block's largest magnitude is <= 448 * 2^e
  (e >= -127, so an all-zero block gets 2^-127); codes = E4M3(x / 2^e).
* Both products run on the quantised operands: S = scale' (Qd Kd^T) with
  Qd = codes * 2^e (likewise Kd, Vd); P = exp(S - m) with m the row maximum;
  P is itself rounded to E4M3 after multiplication by 2^p_shift (so that its
  small entries stay in the normal range; with p_shift = 4, 2^4 P <= 16),
  O = (E4M3(2^p_shift P) Vd) / (2^p_shift sum_k P).  The row sum uses the
  unrounded P.  L = m + ln(sum_k P) (natural log), as in the exact forward.

With rotate=False the same steps give "baseline FP8 attention", the page's
point of comparison.
"""
from __future__ import annotations

import numpy as np

from .attention import keep_matrix

E4M3_MAX = 448.0
BLOCK_ROWS = 64


def e4m3_round(x) -> np.ndarray:
    """Round float64 values to the nearest E4M3FN value, ties to even.

    A binade [2^e, 2^(e+1)) with e >= -6 holds 8 values spaced 2^(e-3); below
    2^-6 the spacing is the subnormal step 2^-9.  So the grid step of x is
    2^(max(e, -6) - 3), and x rounds to the multiple of that step nearest to
    it (np.rint rounds halves to even, i.e. to an even multiple, which is an
    even mantissa).  Magnitudes that would round above 448 raise: the method
    never produces them.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, ex = np.frexp(a)            # a = f 2^ex, f in [0.5, 1)
    e = np.maximum(ex - 1, -6)     # floor(log2 a), clamped to the subnormals
    step = np.ldexp(1.0, e - 3)
    r = np.rint(a / step) * step
    r = np.where(a == 0, 0.0, r)
    if np.any(r > E4M3_MAX):
        raise ValueError("value outside the E4M3FN range")
    return np.copysign(r, x)


def hadamard(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order d (a power of two), entries +-1.

    H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]].
    """
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def rotation(d: int, signs=None) -> np.ndarray:
    """M = diag(signs) H_d (signs default to all +1)."""
    s = np.ones(d) if signs is None else np.asarray(signs, dtype=np.float64)
    if s.shape != (d,) or not np.all(np.abs(s) == 1):
        raise ValueError("signs must be d values of +-1")
    return s[:, None] * hadamard(d)


def block_exponent(amax: float) -> int:
    """Smallest integer e with amax <= 448 * 2^e, and at least -127."""
    amax = float(amax)
    if amax == 0.0:
        return -127
    e = int(np.ceil(np.log2(amax / E4M3_MAX)))
    while amax > E4M3_MAX * 2.0 ** e:       # correct any log2 rounding
        e += 1
    while amax <= E4M3_MAX * 2.0 ** (e - 1):
        e -= 1
    return max(e, -127)


def quantize_blocks(x, block: int = BLOCK_ROWS):
    """Per-block E4M3 quantisation of the rows of x (n x d).

    Returns (codes, exps): codes are the E4M3 values (float64, before the
    block scale is applied back), exps[i] the exponent of rows
    block*i .. block*(i+1)-1.  x = codes * 2^exps[row // block] up to the
    rounding of E4M3.
    """
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[0]
    nblk = (n + block - 1) // block
    codes = np.zeros_like(x)
    exps = np.zeros(nblk, dtype=np.int64)
    for i in range(nblk):
        rows = slice(i * block, min(n, (i + 1) * block))
        e = block_exponent(np.max(np.abs(x[rows]), initial=0.0))
        exps[i] = e
        codes[rows] = e4m3_round(x[rows] * 2.0 ** (-e))
    return codes, exps


def dequantize(codes, exps, block: int = BLOCK_ROWS) -> np.ndarray:
    rows = np.arange(codes.shape[0]) // block
    return np.asarray(codes) * np.ldexp(1.0, np.asarray(exps)[rows])[:, None]


def quantize_head(q, k, v, signs=None, rotate: bool = True,
                  block: int = BLOCK_ROWS) -> dict:
    """The quantisation step for one head: rotate Q, K, then quantise Q, K, V
    per block.  Returns the codes, exponents and the dequantised operands."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    d = q.shape[1]
    if rotate:
        m = rotation(d, signs)
        q = q @ m
        k = k @ m
    out = {}
    for name, x in (("q", q), ("k", k), ("v", v)):
        c, e = quantize_blocks(x, block)
        out[name + "_codes"] = c
        out[name + "_exps"] = e
        out[name + "_deq"] = dequantize(c, e, block)
        out[name + "_in"] = x           # the values that were quantised
    out["score_div"] = float(d) if rotate else 1.0
    return out


def fp8_forward_head(q, k, v, scale: float, causal: bool = False, signs=None,
                     rotate: bool = True, block: int = BLOCK_ROWS,
                     p_shift: int = 4, causal_offset: int = 0) -> dict:
    """FP8 forward of one head; returns O, L and the intermediate terms the
    tests use (dequantised operands, P, the row sums)."""
    qz = quantize_head(q, k, v, signs, rotate, block)
    nq, nk = qz["q_deq"].shape[0], qz["k_deq"].shape[0]
    s = (scale / qz["score_div"]) * (qz["q_deq"] @ qz["k_deq"].T)
    keep = keep_matrix(nq, nk, causal, causal_offset=causal_offset)
    s = np.where(keep, s, -np.inf)
    m = np.max(s, axis=1, initial=-np.inf)
    live = np.isfinite(m)
    m_safe = np.where(live, m, 0.0)
    p = np.where(keep, np.exp(s - m_safe[:, None]), 0.0)
    ell = p.sum(axis=1)
    shift = 2.0 ** p_shift
    p8 = e4m3_round(p * shift)
    o = np.zeros((nq, qz["v_deq"].shape[1]))
    o[live] = (p8[live] @ qz["v_deq"]) / (shift * ell[live])[:, None]
    lse = np.where(live, m_safe + np.log(np.where(live, ell, 1.0)), -np.inf)
    return {"O": o, "L": lse, "P": p, "ell": ell, "p_shift": p_shift, **qz}


def p_rounding_bound(res: dict) -> np.ndarray:
    """Elementwise bound on how far two evaluations of the FP8 forward may
    differ when they round P to E4M3 against different row references.

    Each side rounds 2^p_shift P_qk to E4M3 after multiplying it by some
    factor >= 1 (exp of the gap between the row maximum and the reference
    maximum that side subtracted), and divides the factor out again later:
    relative error <= 2^-4 in the normal range, absolute <= 2^-10 below it,
    i.e. each side's P is within max(2^-4 P, 2^-10 2^-p_shift) of P.  Two
    sides differ by at most twice that, so O differs by at most
    sum_k 2 max(2^-4 P_qk, 2^-10-p_shift) |Vd_kc| / sum_k P_qk.
    """
    p, ell, vd = res["P"], res["ell"], res["v_deq"]
    eps = np.maximum(2.0 ** -4 * p, 2.0 ** (-10 - res["p_shift"]))
    eps = np.where(p > 0, eps, 0.0)
    with np.errstate(invalid="ignore", divide="ignore"):
        b = 2.0 * (eps @ np.abs(vd)) / ell[:, None]
    return np.where(ell[:, None] > 0, b, 0.0)
