"""Shared helpers for the GPU parity tests (not collected by pytest)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import io_aware_exact_04_amd as fa
import oracle
import workloads as W

# Tolerances against the fp64 oracle.
TOL_F32 = 1e-4        # max |delta| on O, L, dQ, dK, dV (fp32 storage)
TOL_O_BF16 = 2e-2     # max |delta| on O (bf16 storage)
TOL_L = 1e-3          # max |delta| on L
TOL_G_BF16 = 5e-2     # max |delta| / max |ref| on dQ, dK, dV (bf16 storage)
# Floor of that denominator: a gradient that vanishes identically (one key
# per row: P = 1, so dP = D and dS = 0) has no scale of its own; the
# kernels' rounding residue is then measured against 1e-3, far below the
# gradients' size for the unit-variance inputs here.
GRAD_FLOOR = 1e-3


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(inp, w):
    q, k, v, do = (W.to_torch(inp[x], w.dtype, "cuda") for x in
                   ("q", "k", "v", "do"))
    mask = None
    if inp["block_mask"] is not None:
        mask = torch.from_numpy(inp["block_mask"]).cuda()
    return q, k, v, do, mask


def run_gpu(w, inp, backward=True):
    say(f"[gpu] {w.name} B={w.B} H={w.H} N={w.N} d={w.D} {w.dtype} "
        f"causal={w.causal} mask={w.has_mask} backward={backward}")
    q, k, v, do, mask = to_dev(inp, w)
    mb = w.mask_block if w.has_mask else 128
    o, lse = fa.fa_fwd(q, k, v, w.scale, w.causal, mask, mb)
    out = {"o": o, "lse": lse}
    if backward:
        dq, dk, dv = fa.fa_bwd(q, k, v, o, lse, do, w.scale, w.causal, mask,
                               mb)
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return out


def head(t: torch.Tensor, b: int, h: int, rows=None) -> np.ndarray:
    x = t[b, h] if rows is None else t[b, h][torch.as_tensor(rows).cuda()]
    return x.float().cpu().numpy().astype(np.float64)


def check_forward(w, inp, out, heads, rows=None):
    """O and L of the listed heads (optionally only some query rows)."""
    worst = {"o": 0.0, "lse": 0.0}
    for b, h in heads:
        O, L = oracle.forward_head(inp["q"][b, h], inp["k"][b, h],
                                   inp["v"][b, h], w.scale, w.causal,
                                   inp["block_mask"], w.mask_block or 128,
                                   q_rows=rows)
        go = head(out["o"], b, h, rows)
        gl = head(out["lse"], b, h, rows)
        assert np.array_equal(np.isneginf(L), np.isneginf(gl)), (b, h)
        fin = np.isfinite(L)
        eo = float(np.abs(go - O).max()) if O.size else 0.0
        el = float(np.abs(gl[fin] - L[fin]).max()) if fin.any() else 0.0
        assert np.isfinite(go).all(), (b, h)
        worst["o"] = max(worst["o"], eo)
        worst["lse"] = max(worst["lse"], el)
    tol_o = TOL_F32 if w.dtype == "fp32" else TOL_O_BF16
    tol_l = TOL_F32 if w.dtype == "fp32" else TOL_L
    say(f"  fwd max|dO|={worst['o']:.3e} (tol {tol_o}) "
        f"max|dL|={worst['lse']:.3e} (tol {tol_l})")
    assert worst["o"] <= tol_o, worst
    assert worst["lse"] <= tol_l, worst
    return worst


def check_backward(w, inp, out, heads):
    worst = {}
    for b, h in heads:
        dQ, dK, dV, _ = oracle.backward_head(
            inp["q"][b, h], inp["k"][b, h], inp["v"][b, h], inp["do"][b, h],
            w.scale, w.causal, inp["block_mask"], w.mask_block or 128)
        for name, ref in (("dq", dQ), ("dk", dK), ("dv", dV)):
            got = head(out[name], b, h)
            assert np.isfinite(got).all(), (name, b, h)
            err = float(np.abs(got - ref).max())
            if w.dtype == "fp32":
                val = err
            else:
                val = err / max(float(np.abs(ref).max()), GRAD_FLOOR)
            worst[name] = max(worst.get(name, 0.0), val)
    tol = TOL_F32 if w.dtype == "fp32" else TOL_G_BF16
    kind = "max|d|" if w.dtype == "fp32" else "max|d|/max|ref|"
    say("  bwd " + " ".join(f"{k} {kind}={v:.3e}" for k, v in worst.items())
        + f" (tol {tol})")
    for k, v in worst.items():
        assert v <= tol, (k, v)
    return worst
