"""GPU parity of the FP8 forward with incoherent processing ("FlashAttention:
making attention IO-aware", section "FlashAttention-3: Hopper asynchrony and
FP8") against the fp64 FP8 oracle (oracle/fp8.py).

* Quantisation (integer work): the E4M3 codes and E8M0 block scales the
  library writes equal the oracle's bit for bit without rotation.  With
  rotation the library transforms in fp32 and the oracle in fp64, so a code
  (or a block exponent) may differ only where the exact value lies within
  the fp32 transform's rounding of a rounding boundary; every such element
  is checked to be one, and the rest must be equal.
* Forward: L within 1e-3 of the oracle's; O within the bound that follows
  from both sides rounding P to E4M3 against different row references
  (oracle.fp8.p_rounding_bound) plus the bf16 rounding of the output; and
  the library's error against exact attention matches the method's own.
* The rotation lowers the error against exact attention on inputs with
  outliers, as the page reports.
"""
import math

import numpy as np
import pytest
import torch

import io_aware_exact_04_amd as fa
import oracle
from oracle import fp8 as F
import workloads as W
from tests import _parity as P

pytestmark = pytest.mark.gpu

TOL_L = P.TOL_L


def _key_position(r):
    """Position of key r of a 64-key group in the transposed V codes (the
    formula the library's header documents)."""
    r = np.asarray(r)
    return 32 * ((r >> 2) & 1) + 16 * (r >> 5) + 4 * ((r >> 3) & 3) + (r & 3)


def _decode(u8: torch.Tensor) -> np.ndarray:
    return u8.cpu().view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _gpu_sections(ws, q_shape, bh, n):
    s = fa.fp8_sections(ws, q_shape)
    rows = s["rows"]
    vt = s["v_codes"][bh].cpu()                         # [d, rows]
    pos = np.arange(rows)
    perm = 64 * (pos // 64) + _key_position(pos % 64)   # key r -> column
    v_codes = vt[:, torch.as_tensor(perm)].T.contiguous()  # [rows, d]
    return {
        "q": (_decode(s["q_codes"][bh]), s["q_scales"][bh].cpu().numpy() - 127),
        "k": (_decode(s["k_codes"][bh]), s["k_scales"][bh].cpu().numpy() - 127),
        "v": (_decode(v_codes), s["v_scales"][bh].cpu().numpy() - 127),
        "rows": rows,
    }


def _check_codes(name, gpu_codes, gpu_exps, ref, n, rotated, x_in):
    """Compare one operand's codes and exponents of one head."""
    rc, re = ref
    rows = gpu_codes.shape[0]
    assert not gpu_codes[n:].any(), f"{name}: padded rows not zero"
    gc = gpu_codes[:n]
    if not rotated:
        np.testing.assert_array_equal(gpu_exps, re, err_msg=name)
        np.testing.assert_array_equal(gc, rc, err_msg=name)
        return 0
    # fp32 transform error per output: log2(d) <= 7 butterfly stages, each
    # rounding a partial sum bounded by the input row's L1 norm, which is at
    # most the rotated row's: <= 7 2^-24 |x|_1 < 2^-20 |x_rot|_1.
    slack = 2.0 ** -20 * np.abs(x_in).sum(axis=1, keepdims=True)
    flips = 0
    for blk in range(len(re)):
        rs = slice(64 * blk, min(n, 64 * (blk + 1)))
        xs, sl = x_in[rs], slack[rs]
        amax = np.abs(xs).max()
        eg = int(gpu_exps[blk])
        if eg != re[blk]:
            lo = F.block_exponent(max(amax - sl.max(), 0.0))
            hi = F.block_exponent(amax + sl.max())
            assert lo <= eg <= hi, f"{name} block {blk}: exponent {eg} vs {re[blk]}"
        scaled = xs * 2.0 ** -eg
        want = F.e4m3_round(scaled)
        near = (F.e4m3_round(np.clip(scaled + sl * 2.0 ** -eg, -448, 448)) !=
                F.e4m3_round(np.clip(scaled - sl * 2.0 ** -eg, -448, 448)))
        got = gc[rs]
        bad = (got != want) & ~near
        assert not bad.any(), f"{name} block {blk}: {int(bad.sum())} codes differ"
        flips += int(((got != want) & near).sum())
    return flips


def _quant_case(B, H, N, D, rotate, seed):
    w = W.small_case(f"fp8q{seed}", B, H, N, D, "bf16", False, seed)
    inp = W.make_inputs(w, with_grad=False)
    signs = W.hadamard_signs(D, seed + 1)
    P.say(f"[gpu] fp8 quantise B={B} H={H} N={N} d={D} rotate={rotate}")
    q, k, v = (W.to_torch(inp[x], "bf16", "cuda") for x in ("q", "k", "v"))
    ws = fa.fa_fp8_quantize(q, k, v, signs, rotate)
    torch.cuda.synchronize()
    flips = 0
    for b in range(B):
        for h in range(H):
            ref = F.quantize_head(inp["q"][b, h], inp["k"][b, h],
                                  inp["v"][b, h], signs, rotate)
            g = _gpu_sections(ws, q.shape, b * H + h, N)
            for name in ("q", "k", "v"):
                flips += _check_codes(
                    name, g[name][0], g[name][1],
                    (ref[name + "_codes"], ref[name + "_exps"]), N,
                    rotate and name != "v", ref[name + "_in"])
    return flips, B * H * N * D * 2


QCASES = [(1, 2, 1, 128), (1, 2, 100, 128), (2, 2, 257, 128), (1, 3, 64, 64),
          (1, 2, 300, 64)]


@pytest.mark.parametrize("rotate", [False, True])
@pytest.mark.parametrize("case", QCASES, ids=[f"N{c[2]}_d{c[3]}" for c in QCASES])
def test_fp8_quantize_codes(case, rotate):
    B, H, N, D = case
    flips, total = _quant_case(B, H, N, D, rotate, 300 + N + D)
    P.say(f"  codes at a rounding boundary that differ: {flips} of {total}")
    assert flips <= max(2, total // 10000)


def _fwd_case(w, inp, signs, rotate, heads, rows=None):
    q, k, v = (W.to_torch(inp[x], "bf16", "cuda") for x in ("q", "k", "v"))
    P.say(f"[gpu] fp8 forward {w.name} B={w.B} H={w.H} N={w.N} d={w.D} "
          f"causal={w.causal} rotate={rotate}")
    o, lse = fa.fa_fwd_fp8(q, k, v, w.scale, w.causal, signs, rotate)
    torch.cuda.synchronize()
    worst = {"L": 0.0, "O/bound": 0.0}
    ratio = []
    for b, h in heads:
        r = F.fp8_forward_head(inp["q"][b, h], inp["k"][b, h], inp["v"][b, h],
                               w.scale, w.causal, signs, rotate)
        go, gl = P.head(o, b, h), P.head(lse, b, h)
        assert np.isfinite(go).all() and np.isfinite(gl).all(), (b, h)
        dl = np.abs(gl - r["L"])
        worst["L"] = max(worst["L"], float(dl.max()))
        bound = (F.p_rounding_bound(r) + 2.0 ** -8 * np.abs(r["O"]) + 2e-5)
        worst["O/bound"] = max(worst["O/bound"],
                               float((np.abs(go - r["O"]) / bound).max()))
        ex = oracle.forward_head(inp["q"][b, h], inp["k"][b, h],
                                 inp["v"][b, h], w.scale, w.causal)[0]
        e_gpu = np.sqrt(((go - ex) ** 2).mean())
        e_ref = np.sqrt(((r["O"] - ex) ** 2).mean())
        ratio.append(e_gpu / e_ref if e_ref > 0 else 1.0)
    P.say(f"  max|dL|={worst['L']:.3e} (tol {TOL_L}) "
          f"max|dO|/bound={worst['O/bound']:.3f} (<= 1) "
          f"error vs exact, library/oracle = {min(ratio):.3f}..{max(ratio):.3f}")
    assert worst["L"] <= TOL_L
    assert worst["O/bound"] <= 1.0
    assert 0.8 <= min(ratio) and max(ratio) <= 1.25
    return o, lse


FCASES = [
    # name, B, H, N, D, causal
    ("one_row_d128", 1, 2, 1, 128, False),
    ("ragged_causal_d128", 1, 2, 257, 128, True),
    ("three_blocks_d128", 2, 2, 384, 128, False),
    ("ragged_causal_d64", 1, 2, 200, 64, True),
    ("dense_d64", 1, 3, 320, 64, False),
]


@pytest.mark.parametrize("rotate", [True, False])
@pytest.mark.parametrize("case", FCASES, ids=[c[0] for c in FCASES])
def test_fp8_forward_small_every_head(case, rotate):
    name, B, H, N, D, causal = case
    w = W.small_case(name, B, H, N, D, "bf16", causal, 500 + N + D)
    inp = W.make_inputs(w, with_grad=False)
    signs = W.hadamard_signs(D, 501 + N)
    _fwd_case(w, inp, signs, rotate,
              [(b, h) for b in range(B) for h in range(H)])


def test_fp8_forward_headline_shape_sampled_heads():
    """B=2, H=32, N=4096, d=128, causal: two whole heads against the oracle,
    and their quantised codes."""
    w = W.get("c3")
    inp = W.make_inputs(w, with_grad=False)
    signs = W.hadamard_signs(w.D, 33)
    heads = [(0, 5), (1, 30)]
    _fwd_case(w, inp, signs, True, heads)
    q, k, v = (W.to_torch(inp[x], "bf16", "cuda") for x in ("q", "k", "v"))
    ws = fa.fa_fp8_quantize(q, k, v, signs, True)
    torch.cuda.synchronize()
    for b, h in heads:
        ref = F.quantize_head(inp["q"][b, h], inp["k"][b, h], inp["v"][b, h],
                              signs, True)
        g = _gpu_sections(ws, q.shape, b * w.H + h, w.N)
        flips = 0
        for name in ("q", "k", "v"):
            flips += _check_codes(name, g[name][0], g[name][1],
                                  (ref[name + "_codes"], ref[name + "_exps"]),
                                  w.N, name != "v", ref[name + "_in"])
        assert flips <= w.N * w.D * 2 // 10000


def test_fp8_split_call_equals_fused_call():
    """fa_fp8_quantize + fa_fwd_fp8_quantized is fa_fwd_fp8, bit for bit."""
    w = W.small_case("split", 1, 2, 200, 128, "bf16", True, 61)
    inp = W.make_inputs(w, with_grad=False)
    signs = W.hadamard_signs(128, 62)
    q, k, v = (W.to_torch(inp[x], "bf16", "cuda") for x in ("q", "k", "v"))
    o1, l1 = fa.fa_fwd_fp8(q, k, v, w.scale, True, signs, True)
    ws = fa.fa_fp8_quantize(q, k, v, signs, True)
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
    fa.fa_fwd_fp8_quantized(ws, o2, l2, w.scale, True, True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fp8_rotation_lowers_error_with_outliers():
    """Same draw as the oracle's pin: the library's errors against exact
    attention, with and without the rotation, are the method's own (within
    10%), and the rotation lowers the error."""
    x = W.outlier_inputs(1024, 128, seed=21, B=1, H=2)
    q, k, v = (W.to_torch(x[n], "bf16", "cuda") for n in ("q", "k", "v"))
    scale = 1 / math.sqrt(128)
    err, ref = {}, {}
    for rotate in (False, True):
        P.say(f"[gpu] fp8 outliers rotate={rotate}")
        o, _ = fa.fa_fwd_fp8(q, k, v, scale, False, x["signs"], rotate)
        torch.cuda.synchronize()
        e2 = r2 = 0.0
        for h in range(2):
            args = (x["q"][0, h], x["k"][0, h], x["v"][0, h], scale, False)
            ex = oracle.forward_head(*args)[0]
            e2 += ((P.head(o, 0, h) - ex) ** 2).mean()
            r2 += ((F.fp8_forward_head(*args, x["signs"], rotate)["O"] - ex)
                   ** 2).mean()
        err[rotate], ref[rotate] = math.sqrt(e2 / 2), math.sqrt(r2 / 2)
    P.say(f"  rmse plain {err[False]:.3e} (oracle {ref[False]:.3e}), "
          f"rotated {err[True]:.3e} (oracle {ref[True]:.3e}), "
          f"ratio {err[False] / err[True]:.2f}")
    for rotate in (False, True):
        assert 0.9 <= err[rotate] / ref[rotate] <= 1.1
    assert err[False] / err[True] > 1.5
