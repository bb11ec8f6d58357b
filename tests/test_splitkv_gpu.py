"""GPU parity of the split-KV forward (Flash-Decoding, "FlashAttention: making
attention IO-aware", "In practice") against the fp64 definition: queries
against a longer key/value sequence, keys split into runs whose partial
results the library merges by their logsumexp.  Every head is checked on the
small cases and of the decode workload.
"""
import numpy as np
import pytest
import torch

import io_aware_exact_04_amd as fa
import oracle
import workloads as W
from tests import _parity as P

pytestmark = pytest.mark.gpu

CASES = [
    # name, B, H, Nq, Nk, D, causal, splits, k_scale
    ("one_query_d128", 1, 3, 1, 1000, 128, True, 4, 1.0),
    ("sixteen_queries_d64", 2, 2, 16, 777, 64, False, 7, 1.0),
    ("two_query_blocks_causal", 1, 2, 130, 4100, 128, True, 3, 3.0),
    ("equal_lengths_causal", 1, 2, 300, 300, 128, True, 5, 1.0),
    ("one_split", 1, 2, 8, 513, 64, True, 1, 1.0),
    ("more_splits_than_tiles", 1, 2, 4, 100, 128, False, 16, 1.0),
    ("single_key", 1, 1, 1, 1, 64, True, 3, 1.0),
    ("many_splits", 1, 4, 2, 8191, 128, True, 64, 1.0),
    # One query row takes the streaming decode pass (vector ALUs, 16 lanes
    # per key row, 64-key batches per wave): ragged key counts against the
    # batches, one split and many, both head sizes.
    ("one_query_d64_ragged", 2, 3, 1, 3001, 64, False, 5, 3.0),
    ("one_query_d128_many_splits", 1, 2, 1, 4097, 128, True, 32, 1.0),
    ("one_query_d64_one_split", 1, 2, 1, 200, 64, True, 1, 1.0),
    ("one_query_d128_short_splits", 1, 2, 1, 130, 128, False, 2, 1.0),
    # sharp rows (K x 8: logits of standard deviation 8, nearly one-hot)
    ("one_query_d128_sharp", 1, 2, 1, 2000, 128, True, 4, 8.0),
    ("one_query_d64_sharp", 2, 2, 1, 999, 64, False, 3, 8.0),
]


def _run(w, inp):
    P.say(f"[gpu] splitkv {w.name} B={w.B} H={w.H} Nq={w.Nq} Nk={w.Nk} "
          f"d={w.D} causal={w.causal} splits={w.num_splits} "
          f"scale={w.scale:.6g}")
    q, k, v = (W.to_torch(inp[x], "bf16", "cuda") for x in ("q", "k", "v"))
    o, lse = fa.fa_fwd_splitkv(q, k, v, w.scale, w.causal, w.num_splits)
    torch.cuda.synchronize()
    return q, k, v, o, lse


def _check(w, inp, o, lse, heads):
    worst_o = worst_l = 0.0
    for b, h in heads:
        O, L = oracle.forward_head(inp["q"][b, h], inp["k"][b, h],
                                   inp["v"][b, h], w.scale, w.causal,
                                   causal_offset=w.Nk - w.Nq)
        go, gl = P.head(o, b, h), P.head(lse, b, h)
        assert np.isfinite(go).all() and np.isfinite(gl).all(), (b, h)
        worst_o = max(worst_o, float(np.abs(go - O).max()))
        worst_l = max(worst_l, float(np.abs(gl - L).max()))
    P.say(f"  max|dO|={worst_o:.3e} (tol {P.TOL_O_BF16}) "
          f"max|dL|={worst_l:.3e} (tol {P.TOL_L})")
    assert worst_o <= P.TOL_O_BF16 and worst_l <= P.TOL_L


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_splitkv_small_every_head(case):
    name, B, H, Nq, Nk, D, causal, splits, ks = case
    w = W.KvWorkload(name, B, H, Nq, Nk, D, causal, seed=2000 + len(name),
                     num_splits=splits, k_scale=ks)
    inp = W.make_kv_inputs(w)
    _, _, _, o, lse = _run(w, inp)
    _check(w, inp, o, lse, [(b, h) for b in range(B) for h in range(H)])


@pytest.mark.parametrize("scale", [0.3, 0.05, 1.0])
@pytest.mark.parametrize("D", [64, 128])
def test_splitkv_non_default_scale(D, scale):
    # The scale argument reaches the partial scores and logsumexps.
    w = W.KvWorkload(f"scaled_{D}_{scale}", 1, 2, 5, 900, D, True,
                     seed=2100 + D, num_splits=3, softmax_scale=scale)
    inp = W.make_kv_inputs(w)
    _, _, _, o, lse = _run(w, inp)
    _check(w, inp, o, lse, [(0, 0), (0, 1)])


def test_splitkv_equals_forward_at_equal_lengths():
    # With as many keys as queries the split path computes what fa_fwd does
    # (up to rounding); both are within tolerance of the definition.
    w = W.KvWorkload("eq", 1, 2, 512, 512, 128, True, seed=77, num_splits=4)
    inp = W.make_kv_inputs(w)
    q, k, v, o, lse = _run(w, inp)
    o2, lse2 = fa.fa_fwd(q, k, v, w.scale, True)
    torch.cuda.synchronize()
    assert float((o.float() - o2.float()).abs().max()) <= 2 * P.TOL_O_BF16
    assert float((lse - lse2).abs().max()) <= P.TOL_L
    _check(w, inp, o, lse, [(0, 0), (0, 1)])


def test_splitkv_decode_workload_every_head():
    w = W.KV_WORKLOADS["dec"]
    inp = W.make_kv_inputs(w)
    _, _, _, o, lse = _run(w, inp)
    _check(w, inp, o, lse, [(b, h) for b in range(w.B) for h in range(w.H)])


@pytest.mark.parametrize("nq", [3, 1])
def test_splitkv_split_count_does_not_change_the_result_beyond_rounding(nq):
    w = W.KvWorkload(f"splits_{nq}", 1, 2, nq, 2000, 64, True, seed=91)
    inp = W.make_kv_inputs(w)
    q, k, v = (W.to_torch(inp[x], "bf16", "cuda") for x in ("q", "k", "v"))
    outs = [fa.fa_fwd_splitkv(q, k, v, w.scale, True, s) for s in (1, 2, 5, 32)]
    torch.cuda.synchronize()
    for o, lse in outs[1:]:
        assert float((o.float() - outs[0][0].float()).abs().max()) <= 1e-2
        assert float((lse - outs[0][1]).abs().max()) <= 1e-4
