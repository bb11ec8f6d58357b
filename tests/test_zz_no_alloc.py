"""The allocation-free backward (fa_bwd_noalloc: the row term D in the
library's static device scratch instead of a caller workspace) against the
workspace backward fa_bwd on the same inputs, through the C ABI.  Both run
the same kernels, so the gradients must be bitwise equal; one case is also
checked against the fp64 oracle.  Consecutive calls reuse the same scratch:
the second call has a smaller input."""
import numpy as np
import pytest
import torch

import io_aware_exact_04_amd as fa
import workloads as W
from tests import _parity as P

pytestmark = pytest.mark.gpu

# name, B, H, N, D, dtype, causal, mask_block, frac
SEQUENCE = [
    ("bf16_d128_causal", 2, 3, 700, 128, "bf16", True, 0, 0.0),
    ("bf16_d64_mask_smaller", 1, 2, 300, 64, "bf16", False, 128, 0.5),
    ("fp32_d64_causal_smaller", 1, 1, 130, 64, "fp32", True, 0, 0.0),
]


def _case(c, seed):
    name, B, H, N, D, dtype, causal, mb, frac = c
    return W.small_case(f"noalloc_{name}", B, H, N, D, dtype, causal, seed,
                        mask_block=mb, mask_frac=frac)


def test_noalloc_equals_workspace_backward_in_sequence():
    for i, c in enumerate(SEQUENCE):
        w = _case(c, 9100 + i)
        inp = W.make_inputs(w)
        P.say(f"[gpu] fa_bwd_noalloc call {i}: {w.name} B={w.B} H={w.H} "
              f"N={w.N} d={w.D} {w.dtype}")
        q, k, v, do, mask = P.to_dev(inp, w)
        mb = w.mask_block or 128
        o, lse = fa.fa_fwd(q, k, v, w.scale, w.causal, mask, mb)
        ref = fa.fa_bwd(q, k, v, o, lse, do, w.scale, w.causal, mask, mb)
        out = tuple(P.nan_like(q) for _ in range(3))
        got = fa.fa_bwd_noalloc(q, k, v, o, lse, do, w.scale, w.causal, mask,
                                mb, out=out)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(a, b), (w.name, name)
        if i == 0:
            P.check_backward(w, inp, dict(zip(("dq", "dk", "dv"), got)),
                             P.all_heads(w))


def test_noalloc_rejects_more_rows_than_its_scratch():
    rows = fa.noalloc_max_rows()
    # One head of 64 rows more than the scratch holds, d = 64 (0.5 GiB per
    # tensor); the call must be rejected before any launch.
    n = rows + 64
    q = torch.zeros(1, 1, n, 64, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(1, 1, n, dtype=torch.float32, device="cuda")
    outs = tuple(P.nan_like(q) for _ in range(3))
    P.say(f"[gpu] fa_bwd_noalloc with {n} rows (limit {rows})")
    with pytest.raises(fa.FaError) as e:
        fa.fa_bwd_noalloc(q, q, q, q, lse, q, 0.125, False, out=outs)
    assert e.value.status_name == "FA_ERR_WORKSPACE"
    torch.cuda.synchronize()
    for t in outs:              # nothing was launched
        assert bool(torch.isnan(t.float()).all())


def test_noalloc_backward_replays_from_a_captured_graph():
    # The use the entry point exists for: the backward captured in a graph
    # (no allocation inside the capture) and replayed.  The first call runs
    # eagerly, outside the capture.  Each replay follows eager work on new
    # inputs and a synchronisation, and must equal an eager call bitwise.
    w = W.small_case("noalloc_graph", 1, 2, 333, 128, "bf16", True, 9200)
    inp = W.make_inputs(w)
    q, k, v, do, _ = P.to_dev(inp, w)
    o, lse = fa.fa_fwd(q, k, v, w.scale, True)
    out = tuple(torch.empty_like(q) for _ in range(3))
    ref = tuple(torch.empty_like(q) for _ in range(3))
    P.say("[gpu] fa_bwd_noalloc under graph capture, 3 replays")
    fa.fa_bwd_noalloc(q, k, v, o, lse, do, w.scale, True, out=out)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            fa.fa_bwd_noalloc(q, k, v, o, lse, do, w.scale, True, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    gen = torch.Generator(device="cuda").manual_seed(5)
    for rep in range(3):
        # New dO (and so new gradients) written in place, eagerly.
        do.copy_(torch.randn(do.shape, device="cuda",
                             generator=gen).to(do.dtype))
        for t in out:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        fa.fa_bwd(q, k, v, o, lse, do, w.scale, True, out=ref)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), out, ref):
            assert torch.equal(a, b), (rep, name)
