"""Guard regions: no entry point writes outside the memory it was given.

Every output tensor is a strided view inside a larger NaN-filled buffer:
rows are padded (sn > d), heads and batches carry gaps, and guard regions
sit before and after the whole view.  Every workspace is a slice of a larger
buffer of sentinel bytes.  After each call the NaN (or sentinel) outside the
views must be untouched, and no element inside an output view may be left
NaN.  The kernels rely on buffer range checks to drop stores past the last
row of a head; these checks pin that they also never reach the padding
between rows, heads and batches, nor the bytes around a workspace.
"""
import numpy as np
import pytest
import torch

import io_aware_exact_04_amd as fa
import workloads as W
from tests import _parity as P

pytestmark = pytest.mark.gpu

NAN = float("nan")
SENTINEL = 0xA5
LEAD = 64          # guard elements before a view (16-byte multiple)
TRAIL = 1000       # guard elements after it


class Guarded:
    """A [..., d] view with padded strides inside a NaN-filled buffer."""

    def __init__(self, shape, dtype, strides=None, fill=None):
        elt = torch.empty((), dtype=dtype).element_size()
        step = 16 // elt                      # elements per 16 bytes
        if strides is None:                   # padded rows, gaps between heads
            strides = [1]
            inner = shape[-1] + 3 * step
            for n in reversed(shape[:-1]):
                strides.insert(0, inner)
                inner = inner * n + 5 * step
        self.strides = tuple(strides)
        span = 1 + sum((n - 1) * s for n, s in zip(shape, strides))
        self.buf = torch.full((LEAD + span + TRAIL,), NAN, dtype=dtype,
                              device="cuda")
        self.view = self.buf.as_strided(shape, self.strides, LEAD)
        if fill is not None:
            self.view.copy_(fill)

    def check(self, name, written=True):
        n = self.buf.numel()
        idx = torch.arange(n, device="cuda").as_strided(
            self.view.shape, self.view.stride(), LEAD)
        inside = torch.zeros(n, dtype=torch.bool, device="cuda")
        inside[idx.reshape(-1)] = True
        out = self.buf[~inside].float()
        assert torch.isnan(out).all(), f"{name}: written outside its view"
        if written:
            assert not torch.isnan(self.buf[inside].float()).any(), \
                f"{name}: element of the view left unwritten"


class GuardedBytes:
    """A workspace slice of exactly `nbytes` inside sentinel bytes."""

    def __init__(self, nbytes):
        self.n = max(int(nbytes), 16)
        self.buf = torch.full((256 + self.n + 4096,), SENTINEL,
                              dtype=torch.uint8, device="cuda")
        self.view = self.buf[256:256 + self.n]

    def check(self, name):
        assert bool((self.buf[:256] == SENTINEL).all()), \
            f"{name}: wrote before its workspace"
        assert bool((self.buf[256 + self.n:] == SENTINEL).all()), \
            f"{name}: wrote past its workspace"


def _inputs(w, strides=None):
    inp = W.make_inputs(w)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    t = {x: Guarded(w.shape, dt, strides,
                    W.to_torch(inp[x], w.dtype, "cuda")) for x in
         ("q", "k", "v", "do")}
    mask = (torch.from_numpy(inp["block_mask"]).cuda()
            if inp["block_mask"] is not None else None)
    return t, mask


CASES = [
    # name, B, H, N, D, dtype, causal, mask_block, frac
    ("bf16_d128_causal", 2, 3, 300, 128, "bf16", True, 0, 0.0),
    ("bf16_d64_mask", 1, 2, 640, 64, "bf16", False, 128, 0.5),
    ("bf16_d64_dense", 2, 2, 129, 64, "bf16", False, 0, 0.0),
    ("fp32_d64_causal", 1, 2, 200, 64, "fp32", True, 0, 0.0),
    ("fp32_d128_mask", 1, 1, 384, 128, "fp32", False, 128, 0.5),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fwd_bwd_guards(case):
    name, B, H, N, D, dtype, causal, mb, frac = case
    w = W.small_case(f"guard_{name}", B, H, N, D, dtype, causal, seed=8100 + N,
                     mask_block=mb, mask_frac=frac)
    P.say(f"[gpu] guards fa_fwd/fa_bwd {name}")
    t, mask = _inputs(w)
    dt = t["q"].view.dtype
    strides = t["q"].strides
    o = Guarded(w.shape, dt, strides)
    lse = Guarded((B, H, N), torch.float32, (H * N, N, 1))
    grads = [Guarded(w.shape, dt, strides) for _ in range(3)]
    ws = GuardedBytes(fa.workspace_bytes(t["q"].view))
    q, k, v, do = (t[x].view for x in ("q", "k", "v", "do"))
    fa.fa_fwd(q, k, v, w.scale, causal, mask, mb or 128, out=o.view,
              lse=lse.view)
    fa.fa_bwd(q, k, v, o.view, lse.view, do, w.scale, causal, mask, mb or 128,
              workspace=ws.view, out=tuple(g.view for g in grads))
    torch.cuda.synchronize()
    o.check("O")
    lse.check("L")
    for g, n in zip(grads, ("dQ", "dK", "dV")):
        g.check(n)
    ws.check("fa_bwd workspace")
    for x in ("q", "k", "v", "do"):
        t[x].check(x, written=True)   # inputs: untouched guards, still set
    # The padded layout computes what the dense layout does.
    o2, l2 = fa.fa_fwd(q.contiguous(), k.contiguous(), v.contiguous(),
                       w.scale, causal, mask, mb or 128)
    g2 = fa.fa_bwd(q.contiguous(), k.contiguous(), v.contiguous(), o2, l2,
                   do.contiguous(), w.scale, causal, mask, mb or 128)
    torch.cuda.synchronize()
    assert torch.equal(o.view, o2) and torch.equal(lse.view, l2)
    for a, b in zip(grads, g2):
        assert torch.equal(a.view, b)


@pytest.mark.parametrize("Nq", [5, 1])
def test_splitkv_guards(Nq):
    B, H, Nk, D = 2, 2, 700, 128
    w = W.KvWorkload(f"guard_kv_{Nq}", B, H, Nq, Nk, D, True, seed=8200,
                     num_splits=3)
    inp = W.make_kv_inputs(w)
    P.say("[gpu] guards fa_fwd_splitkv")
    q = Guarded((B, H, Nq, D), torch.bfloat16, None,
                W.to_torch(inp["q"], "bf16", "cuda"))
    k = Guarded((B, H, Nk, D), torch.bfloat16, None,
                W.to_torch(inp["k"], "bf16", "cuda"))
    v = Guarded((B, H, Nk, D), torch.bfloat16, k.strides,
                W.to_torch(inp["v"], "bf16", "cuda"))
    o = Guarded((B, H, Nq, D), torch.bfloat16, q.strides)
    lse = Guarded((B, H, Nq), torch.float32, (H * Nq, Nq, 1))
    ws = GuardedBytes(fa.splitkv_workspace_bytes(q.view, k.view, 3))
    fa.fa_fwd_splitkv(q.view, k.view, v.view, w.scale, True, 3, out=o.view,
                      lse=lse.view, workspace=ws.view)
    torch.cuda.synchronize()
    o.check("O")
    lse.check("L")
    ws.check("split-KV workspace")


def test_varlen_guards():
    lengths, H, D = [1, 130, 0, 257], 2, 64
    inp = W.make_varlen_inputs(lengths, H, D, seed=8300)
    total = sum(lengths)
    P.say("[gpu] guards fa_fwd_varlen/fa_bwd_varlen")
    st = (H * D + 24, D + 8, 1)           # padded rows and heads
    t = {x: Guarded((total, H, D), torch.bfloat16, st,
                    W.to_torch(inp[x], "bf16", "cuda")) for x in
         ("q", "k", "v", "do")}
    cu = torch.from_numpy(inp["cu_seqlens"]).cuda()
    mx = max(lengths)
    o = Guarded((total, H, D), torch.bfloat16, st)
    lse = Guarded((H, total), torch.float32, (total, 1))
    grads = [Guarded((total, H, D), torch.bfloat16, st) for _ in range(3)]
    q, k, v, do = (t[x].view for x in ("q", "k", "v", "do"))
    fa.fa_fwd_varlen(q, k, v, cu, mx, causal=True, out=o.view, lse=lse.view)
    desc = fa._varlen_desc(q, cu, mx, [])
    need = int(fa.load_library().fa_bwd_varlen_workspace_bytes(
        fa.ctypes.byref(desc)))
    ws = GuardedBytes(need)
    fa.fa_bwd_varlen(q, k, v, o.view, lse.view, do, cu, mx, causal=True,
                     out=tuple(g.view for g in grads), workspace=ws.view)
    torch.cuda.synchronize()
    o.check("O")
    lse.check("L")
    for g, n in zip(grads, ("dQ", "dK", "dV")):
        g.check(n)
    ws.check("varlen workspace")


def test_dropout_padding_guards():
    B, H, N, D = 3, 2, 257, 128
    w = W.small_case("guard_ex", B, H, N, D, "bf16", True, seed=8400)
    P.say("[gpu] guards fa_fwd_ex/fa_bwd_ex")
    t, _ = _inputs(w)
    st = t["q"].strides
    kl = torch.tensor([0, 100, 257], dtype=torch.int32, device="cuda")
    o = Guarded(w.shape, torch.bfloat16, st)
    lse = Guarded((B, H, N), torch.float32, (H * N, N, 1))
    grads = [Guarded(w.shape, torch.bfloat16, st) for _ in range(3)]
    ws = GuardedBytes(fa.workspace_bytes(t["q"].view))
    q, k, v, do = (t[x].view for x in ("q", "k", "v", "do"))
    fa.fa_fwd_ex(q, k, v, w.scale, True, 0.2, 99, kl, out=o.view,
                 lse=lse.view)
    fa.fa_bwd_ex(q, k, v, o.view, lse.view, do, w.scale, True, 0.2, 99, kl,
                 workspace=ws.view, out=tuple(g.view for g in grads))
    torch.cuda.synchronize()
    o.check("O")
    lse.check("L")
    for g, n in zip(grads, ("dQ", "dK", "dV")):
        g.check(n)
    ws.check("fa_bwd_ex workspace")


def test_fp8_guards():
    B, H, N, D = 1, 2, 200, 128
    w = W.small_case("guard_fp8", B, H, N, D, "bf16", True, seed=8500)
    P.say("[gpu] guards fa_fwd_fp8")
    t, _ = _inputs(w)
    o = Guarded(w.shape, torch.bfloat16, t["q"].strides)
    lse = Guarded((B, H, N), torch.float32, (H * N, N, 1))
    ws = GuardedBytes(fa.fp8_layout(t["q"].view).bytes)
    signs = W.hadamard_signs(D, 3)
    fa.fa_fwd_fp8(t["q"].view, t["k"].view, t["v"].view, w.scale, True,
                  signs, True, workspace=ws.view, out=o.view, lse=lse.view)
    torch.cuda.synchronize()
    o.check("O")
    lse.check("L")
    ws.check("fp8 workspace")
    assert np.isfinite(o.view.float().cpu().numpy()).all()
