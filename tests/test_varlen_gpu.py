"""GPU parity of packed variable-length batches ("FlashAttention: making
attention IO-aware", "In practice": concatenated sequences plus their offsets,
no padding) against the fp64 definition applied to each sequence on its own:
forward and backward, every (sequence, head) of the small mixes and of a
larger mix, and agreement with the padded [B, H, N, d] path.
"""
import numpy as np
import pytest
import torch

import io_aware_exact_04_amd as fa
import oracle
import workloads as W
from tests import _parity as P

pytestmark = pytest.mark.gpu


def _run(inp, H, D, causal, backward=True, scale=None):
    q, k, v, do = (W.to_torch(inp[x], "bf16", "cuda") for x in
                   ("q", "k", "v", "do"))
    cu_np = inp["cu_seqlens"]
    cu = torch.from_numpy(cu_np).cuda()
    max_len = int(np.diff(cu_np).max()) if cu_np.size > 1 else 0
    P.say(f"[gpu] varlen total={q.shape[0]} seqs={cu_np.size - 1} H={H} "
          f"d={D} causal={causal} max_len={max_len} scale={scale}")
    o, lse = fa.fa_fwd_varlen(q, k, v, cu, max_len, scale, causal=causal)
    out = {"o": o, "lse": lse}
    if backward:
        dq, dk, dv = fa.fa_bwd_varlen(q, k, v, o, lse, do, cu, max_len,
                                      scale, causal=causal)
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return {k_: x.float().cpu().numpy().astype(np.float64)
            for k_, x in out.items()}


def _check(inp, out, D, causal, pairs, backward=True, scale=None):
    cu = inp["cu_seqlens"]
    scale = 1.0 / np.sqrt(D) if scale is None else scale

    def pair(s, h):
        a, b = int(cu[s]), int(cu[s + 1])
        r = {"o": 0.0, "lse": 0.0, "dq": 0.0, "dk": 0.0, "dv": 0.0}
        g = {"dq": 0.0, "dk": 0.0, "dv": 0.0}
        if b == a:
            return r, g
        q, k, v, do = (inp[x][a:b, h] for x in ("q", "k", "v", "do"))
        O, L = oracle.forward_head(q, k, v, scale, causal)
        r["o"] = float(np.abs(out["o"][a:b, h] - O).max())
        r["lse"] = float(np.abs(out["lse"][h, a:b] - L).max())
        if backward:
            dQ, dK, dV, _ = oracle.backward_head(q, k, v, do, scale, causal)
            for name, ref in (("dq", dQ), ("dk", dK), ("dv", dV)):
                r[name] = float(np.abs(out[name][a:b, h] - ref).max())
                g[name] = float(np.abs(ref).max())
        return r, g

    res = P._map_heads(pair, pairs, "varlen").values()
    # Gradient errors are relative to the largest reference value over the
    # whole packed tensor (a one-token sequence has dQ = dK = 0 exactly).
    worst = {k_: max(r[k_] for r, _ in res)
             for k_ in ("o", "lse", "dq", "dk", "dv")}
    for name in ("dq", "dk", "dv"):
        gmax = max(g[name] for _, g in res)
        worst[name] /= max(gmax, P.GRAD_FLOOR)
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


@pytest.mark.parametrize("scale", [0.3, 0.05, 1.0])
def test_varlen_non_default_scale(scale):
    lengths, H, D = [77, 0, 300, 129], 2, 64
    inp = W.make_varlen_inputs(lengths, H, D, seed=3500)
    out = _run(inp, H, D, True, scale=scale)
    _check(inp, out, D, True,
           [(s, h) for s in range(len(lengths)) for h in range(H)],
           scale=scale)


def test_varlen_length_mix_every_sequence():
    lengths = W.varlen_lengths(12, 200, 3000, seed=31)
    H, D = 16, 128
    inp = W.make_varlen_inputs(lengths, H, D, seed=32)
    out = _run(inp, H, D, True)
    _check(inp, out, D, True,
           [(s, h) for s in range(len(lengths)) for h in range(H)])


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


def test_varlen_packed_qkv_slices():
    # q, k, v as slices of one packed [total, 3, H, d] buffer (strides
    # (3 H d, d, 1)): outputs come back with q's strides and the results
    # equal those of contiguous copies.
    lengths, H, D = [65, 200, 1], 2, 128
    inp = W.make_varlen_inputs(lengths, H, D, seed=3600)
    cu_np = inp["cu_seqlens"]
    cu = torch.from_numpy(cu_np).cuda()
    total, mx = int(cu_np[-1]), max(lengths)
    qkv = torch.stack([W.to_torch(inp[x], "bf16", "cuda") for x in
                       ("q", "k", "v")], dim=1)
    q, k, v = qkv[:, 0], qkv[:, 1], qkv[:, 2]
    P.say(f"[gpu] varlen packed-QKV slices total={total} H={H} d={D}")
    do = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype,
                             device=q.device)
    do.copy_(W.to_torch(inp["do"], "bf16", "cuda"))
    o, lse = fa.fa_fwd_varlen(q, k, v, cu, mx, causal=True)
    grads = fa.fa_bwd_varlen(q, k, v, o, lse, do, cu, mx, causal=True)
    qc, kc, vc, doc = (x.contiguous() for x in (q, k, v, do))
    o2, lse2 = fa.fa_fwd_varlen(qc, kc, vc, cu, mx, causal=True)
    grads2 = fa.fa_bwd_varlen(qc, kc, vc, o2, lse2, doc, cu, mx, causal=True)
    torch.cuda.synchronize()
    assert o.stride() == q.stride()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    for a, b in zip(grads, grads2):
        assert a.stride() == q.stride() and torch.equal(a, b)


def test_ex_entry_points_on_a_non_dense_q():
    # fa_fwd_ex / fa_bwd_ex allocate outputs with q's strides, too.
    B, N, H, D = 2, 150, 2, 64
    w = W.small_case("ex_strided", B, H, N, D, "bf16", True, seed=3700)
    inp = W.make_inputs(w)
    t = {x: W.to_torch(inp[x], "bf16", "cuda") for x in ("q", "k", "v", "do")}
    big = torch.stack([t["q"], t["k"], t["v"], t["do"]], dim=2)  # [B,H,4,N,D]
    q, k, v, do = (big[:, :, i] for i in range(4))
    assert not q.is_contiguous()
    P.say("[gpu] fa_fwd_ex / fa_bwd_ex on a non-dense q")
    kl = torch.tensor([150, 99], dtype=torch.int32, device="cuda")
    o, lse = fa.fa_fwd_ex(q, k, v, w.scale, True, 0.1, 5, kl)
    g = fa.fa_bwd_ex(q, k, v, o, lse, do, w.scale, True, 0.1, 5, kl)
    o2, lse2 = fa.fa_fwd_ex(t["q"], t["k"], t["v"], w.scale, True, 0.1, 5, kl)
    g2 = fa.fa_bwd_ex(t["q"], t["k"], t["v"], o2, lse2, t["do"], w.scale,
                      True, 0.1, 5, kl)
    torch.cuda.synchronize()
    assert o.stride() == q.stride() and torch.equal(o, o2)
    assert torch.equal(lse, lse2)
    for a, b in zip(g, g2):
        assert a.stride() == q.stride() and torch.equal(a, b)
