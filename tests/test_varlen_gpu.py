"""GPU parity of packed variable-length batches ("FlashAttention: making
attention IO-aware", "In practice": concatenated sequences plus their offsets,
no padding) against the fp64 definition applied to each sequence on its own:
forward and backward, every (sequence, head) on the small mixes, sampled ones
on a larger mix, and agreement with the padded [B, H, N, d] path.
"""
import numpy as np
import pytest
import torch

import io_aware_exact_04_amd as fa
import oracle
import workloads as W
from tests import _parity as P

pytestmark = pytest.mark.gpu


def _run(inp, H, D, causal, backward=True):
    q, k, v, do = (W.to_torch(inp[x], "bf16", "cuda") for x in
                   ("q", "k", "v", "do"))
    cu_np = inp["cu_seqlens"]
    cu = torch.from_numpy(cu_np).cuda()
    max_len = int(np.diff(cu_np).max()) if cu_np.size > 1 else 0
    P.say(f"[gpu] varlen total={q.shape[0]} seqs={cu_np.size - 1} H={H} "
          f"d={D} causal={causal} max_len={max_len}")
    o, lse = fa.fa_fwd_varlen(q, k, v, cu, max_len, causal=causal)
    out = {"o": o, "lse": lse}
    if backward:
        dq, dk, dv = fa.fa_bwd_varlen(q, k, v, o, lse, do, cu, max_len,
                                      causal=causal)
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return {k_: x.float().cpu().numpy().astype(np.float64)
            for k_, x in out.items()}


def _check(inp, out, D, causal, pairs, backward=True):
    cu = inp["cu_seqlens"]
    scale = 1.0 / np.sqrt(D)
    # Gradient errors are relative to the largest reference value over the
    # whole packed tensor (a one-token sequence has dQ = dK = 0 exactly).
    worst = {"o": 0.0, "lse": 0.0, "dq": 0.0, "dk": 0.0, "dv": 0.0}
    gmax = {"dq": 0.0, "dk": 0.0, "dv": 0.0}
    for s, h in pairs:
        a, b = int(cu[s]), int(cu[s + 1])
        if b == a:
            continue
        q, k, v, do = (inp[x][a:b, h] for x in ("q", "k", "v", "do"))
        O, L = oracle.forward_head(q, k, v, scale, causal)
        worst["o"] = max(worst["o"], float(np.abs(out["o"][a:b, h] - O).max()))
        worst["lse"] = max(worst["lse"],
                           float(np.abs(out["lse"][h, a:b] - L).max()))
        if backward:
            dQ, dK, dV, _ = oracle.backward_head(q, k, v, do, scale, causal)
            for name, ref in (("dq", dQ), ("dk", dK), ("dv", dV)):
                worst[name] = max(worst[name], float(np.abs(
                    out[name][a:b, h] - ref).max()))
                gmax[name] = max(gmax[name], float(np.abs(ref).max()))
    for name in gmax:
        worst[name] /= max(gmax[name], P.GRAD_FLOOR)
    P.say("  " + " ".join(f"{k_}={v_:.3e}" for k_, v_ in worst.items()))
    assert worst["o"] <= P.TOL_O_BF16 and worst["lse"] <= P.TOL_L
    for name in ("dq", "dk", "dv"):
        assert worst[name] <= P.TOL_G_BF16, (name, worst[name])


MIXES = [
    # name, lengths, H, D, causal
    ("edges_d128_causal", [1, 17, 128, 129, 300, 0, 64, 255], 3, 128, True),
    ("edges_d128_dense", [129, 1, 0, 200, 64], 2, 128, False),
    ("edges_d64_causal", [5, 333, 256, 1, 70], 2, 64, True),
    ("edges_d64_dense", [100, 0, 0, 257], 2, 64, False),
]


@pytest.mark.parametrize("mix", MIXES, ids=[m[0] for m in MIXES])
def test_varlen_small_every_sequence(mix):
    name, lengths, H, D, causal = mix
    inp = W.make_varlen_inputs(lengths, H, D, seed=3000 + len(name))
    out = _run(inp, H, D, causal)
    _check(inp, out, D, causal,
           [(s, h) for s in range(len(lengths)) for h in range(H)])


def test_varlen_length_mix_sampled():
    lengths = W.varlen_lengths(12, 200, 3000, seed=31)
    H, D = 16, 128
    inp = W.make_varlen_inputs(lengths, H, D, seed=32)
    out = _run(inp, H, D, True)
    rng = np.random.default_rng(1)
    pairs = sorted({(int(rng.integers(len(lengths))), int(rng.integers(H)))
                    for _ in range(10)})
    _check(inp, out, D, True, pairs)


def test_varlen_equal_lengths_match_the_padded_path():
    B, N, H, D = 3, 384, 2, 128
    inp = W.make_varlen_inputs([N] * B, H, D, seed=33)
    out = _run(inp, H, D, True)
    q, k, v, do = (W.to_torch(inp[x], "bf16", "cuda")
                   .view(B, N, H, D).permute(0, 2, 1, 3) for x in
                   ("q", "k", "v", "do"))
    o, lse = fa.fa_fwd(q, k, v, causal=True)
    dq, dk, dv = fa.fa_bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    packed = lambda t: t.permute(0, 2, 1, 3).reshape(B * N, H, D).float().cpu().numpy()
    # The same kernels on the same rows: identical results.
    np.testing.assert_array_equal(out["o"], packed(o))
    np.testing.assert_array_equal(out["lse"],
                                  lse.permute(1, 0, 2).reshape(H, B * N).cpu().numpy())
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        np.testing.assert_array_equal(out[name], packed(t))
