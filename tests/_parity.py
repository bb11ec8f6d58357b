"""Shared helpers for the GPU parity tests (not collected by pytest)."""
from __future__ import annotations

import concurrent.futures
import os
import sys
import time

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
# Query rows per oracle evaluation of one head's forward (bounds memory of
# the explicit score matrix at long sequence lengths).
ROW_CHUNK = 2048


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def workers() -> int:
    """Host threads for oracle evaluations: the CPUs this process may use,
    at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - non-Linux
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def to_dev(inp, w):
    q, k, v, do = (W.to_torch(inp[x], w.dtype, "cuda") for x in
                   ("q", "k", "v", "do"))
    mask = None
    if inp["block_mask"] is not None:
        mask = torch.from_numpy(inp["block_mask"]).cuda()
    return q, k, v, do, mask


def nan_like(t: torch.Tensor) -> torch.Tensor:
    """A tensor laid out like t, filled with NaN: an output element the
    library fails to write stays NaN and fails every comparison."""
    x = torch.empty_strided(t.shape, t.stride(), dtype=t.dtype,
                            device=t.device)
    return x.fill_(float("nan"))


def run_gpu(w, inp, backward=True):
    """Forward (and backward) through the C ABI into NaN-filled outputs."""
    say(f"[gpu] {w.name} B={w.B} H={w.H} N={w.N} d={w.D} {w.dtype} "
        f"causal={w.causal} mask={w.has_mask} scale={w.scale:.6g} "
        f"backward={backward}")
    q, k, v, do, mask = to_dev(inp, w)
    mb = w.mask_block if w.has_mask else 128
    o = nan_like(q)
    lse = torch.full((w.B, w.H, w.N), float("nan"), device=q.device)
    fa.fa_fwd(q, k, v, w.scale, w.causal, mask, mb, out=o, lse=lse)
    out = {"o": o, "lse": lse}
    if backward:
        grads = tuple(nan_like(q) for _ in range(3))
        fa.fa_bwd(q, k, v, o, lse, do, w.scale, w.causal, mask, mb,
                  out=grads)
        out.update(dq=grads[0], dk=grads[1], dv=grads[2])
    torch.cuda.synchronize()
    return out


def host_copy(out: dict) -> dict:
    """GPU outputs as float32 host tensors (exact for bf16 and fp32)."""
    return {name: t.float().cpu() for name, t in out.items()}


def head(t: torch.Tensor, b: int, h: int, rows=None) -> np.ndarray:
    x = t[b, h]
    if rows is not None:
        x = x[torch.as_tensor(rows, device=x.device)]
    return x.float().cpu().numpy().astype(np.float64)


def _forward_errors(w, inp, host, b, h, rows=None):
    """max |dO| and max |dL| of one head (rows: a subset of query rows)."""
    mb = w.mask_block or 128
    all_rows = np.arange(w.N) if rows is None else np.asarray(rows)
    eo, el = 0.0, 0.0
    for r0 in range(0, all_rows.size, ROW_CHUNK):
        rr = all_rows[r0:r0 + ROW_CHUNK]
        O, L = oracle.forward_head(inp["q"][b, h], inp["k"][b, h],
                                   inp["v"][b, h], w.scale, w.causal,
                                   inp["block_mask"], mb, q_rows=rr)
        go = head(host["o"], b, h, rr)
        gl = head(host["lse"], b, h, rr)
        # Every element written, -inf exactly where the oracle has it.
        if not np.isfinite(go).all():
            return float("inf"), float("inf")
        if not np.array_equal(np.isneginf(L), np.isneginf(gl)):
            return eo, float("inf")
        fin = np.isfinite(L)
        if not np.isfinite(gl[fin]).all():
            return eo, float("inf")
        if O.size:
            eo = max(eo, float(np.abs(go - O).max()))
        if fin.any():
            el = max(el, float(np.abs(gl[fin] - L[fin]).max()))
    return eo, el


def _backward_errors(w, inp, host, b, h, f32_relative=False):
    """Gradient errors of one head: max|d| (fp32) or max|d|/max|ref|.  For
    fp32, f32_relative divides by max(1, max|ref|) instead: the fp32
    bound is absolute at the unit scale of the workloads' data, and a case
    whose gradients are larger (a softmax scale far above 1/sqrt(d)) keeps
    the same relative bar."""
    mb = w.mask_block or 128
    dQ, dK, dV, _ = oracle.backward_head(
        inp["q"][b, h], inp["k"][b, h], inp["v"][b, h], inp["do"][b, h],
        w.scale, w.causal, inp["block_mask"], mb)
    errs = {}
    for name, ref in (("dq", dQ), ("dk", dK), ("dv", dV)):
        got = head(host[name], b, h)
        if not np.isfinite(got).all():
            errs[name] = float("inf")
            continue
        err = float(np.abs(got - ref).max()) if ref.size else 0.0
        top = float(np.abs(ref).max()) if ref.size else 0.0
        if w.dtype != "fp32":
            err /= max(top, GRAD_FLOOR)
        elif f32_relative:
            err /= max(top, 1.0)
        errs[name] = err
    return errs


def _map_heads(fn, heads, label):
    """fn(b, h) over the heads on a thread pool (numpy releases the GIL in
    its array operations; BLAS is held to one thread per worker)."""
    from threadpoolctl import threadpool_limits
    n = workers()
    t0 = time.time()
    res = {}
    with threadpool_limits(limits=1, user_api="blas"):
        with concurrent.futures.ThreadPoolExecutor(max_workers=n) as ex:
            futs = {ex.submit(fn, b, h): (b, h) for b, h in heads}
            done = 0
            for f in concurrent.futures.as_completed(futs):
                res[futs[f]] = f.result()
                done += 1
                if done % max(1, len(heads) // 4) == 0 or done == len(heads):
                    say(f"  {label}: {done}/{len(heads)} heads checked "
                        f"({time.time() - t0:.0f} s, {n} threads)")
    return res


def check_forward(w, inp, out, heads, rows=None):
    """O and L of the listed heads (optionally only some query rows)."""
    host = host_copy({"o": out["o"], "lse": out["lse"]})
    res = _map_heads(lambda b, h: _forward_errors(w, inp, host, b, h, rows),
                     heads, f"{w.name} fwd")
    worst = {"o": max(r[0] for r in res.values()),
             "lse": max(r[1] for r in res.values())}
    tol_o = TOL_F32 if w.dtype == "fp32" else TOL_O_BF16
    tol_l = TOL_F32 if w.dtype == "fp32" else TOL_L
    say(f"  fwd max|dO|={worst['o']:.3e} (tol {tol_o}) "
        f"max|dL|={worst['lse']:.3e} (tol {tol_l}) over {len(heads)} heads")
    bad = [bh for bh, r in res.items() if not (r[0] <= tol_o and
                                                r[1] <= tol_l)]
    assert not bad, (worst, bad[:8])
    return worst


def check_backward(w, inp, out, heads, f32_relative=False):
    """dQ, dK, dV of the listed heads.  f32_relative: fp32 gradients are
    measured against max(1, max|ref|) (only for cases whose gradients are
    far above unit scale; the workloads keep the absolute bound)."""
    host = host_copy({k: out[k] for k in ("dq", "dk", "dv")})
    res = _map_heads(lambda b, h: _backward_errors(w, inp, host, b, h,
                                                   f32_relative),
                     heads, f"{w.name} bwd")
    tol = TOL_F32 if w.dtype == "fp32" else TOL_G_BF16
    worst = {k: max(r[k] for r in res.values()) for k in ("dq", "dk", "dv")}
    kind = ("max|d|/max(1, max|ref|)" if w.dtype == "fp32" and f32_relative
            else "max|d|" if w.dtype == "fp32" else "max|d|/max|ref|")
    say("  bwd " + " ".join(f"{k} {kind}={v:.3e}" for k, v in worst.items())
        + f" (tol {tol}) over {len(heads)} heads")
    bad = [bh for bh, r in res.items() if not all(v <= tol
                                                  for v in r.values())]
    assert not bad, (worst, bad[:8])
    return worst


def all_heads(w):
    return [(b, h) for b in range(w.B) for h in range(w.H)]
