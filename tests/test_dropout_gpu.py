"""GPU parity of dropout and key padding (fa_fwd_ex / fa_bwd_ex) against the
fp64 oracle with the same Philox4x32-10 keep masks (oracle/dropout.py).

* The keep decisions themselves (integer work) are compared bit for bit:
  with V = identity the forward's O[q, k] = P Z s, and with dO = identity
  the dK/dV kernel's dV[k, q] = P Z s, so the masks the kernels used can be
  read off their outputs (all P > 0 on these non-causal cases).
* Forward and backward against the definition with dropout and/or padding,
  to the bf16 tolerances of the plain path.
"""
import numpy as np
import pytest
import torch

import io_aware_exact_04_amd as fa
import oracle
from oracle import dropout as Dr
import workloads as W
from tests import _parity as P

pytestmark = pytest.mark.gpu


def _identity_case(B, H, N, D, seed):
    """Q, K small (P nearly uniform, all > 0), V = dO = identity rows."""
    w = W.small_case("dropid", B, H, N, D, "bf16", False, seed)
    inp = W.make_inputs(w)
    eye = np.zeros((B, H, N, D))
    eye[:, :, np.arange(N), np.arange(N)] = 1.0
    return w, inp, eye


@pytest.mark.parametrize("N,D", [(100, 128), (64, 64), (128, 128)])
def test_keep_masks_bit_exact(N, D):
    B, H, seed, p = 2, 3, 0x1234ABCD5678, 0.5
    p8 = Dr.quantize_p(p)
    w, inp, eye = _identity_case(B, H, N, D, 900 + N)
    P.say(f"[gpu] dropout masks B={B} H={H} N={N} d={D} p={p}")
    q, k = (W.to_torch(inp[x], "bf16", "cuda") for x in ("q", "k"))
    v = W.to_torch(eye, "bf16", "cuda")
    scale = 0.05
    o, lse = fa.fa_fwd_ex(q, k, v, scale, False, p, seed)
    dq, dk, dv = fa.fa_bwd_ex(q, k, v, o, lse, v, scale, False, p, seed)
    torch.cuda.synchronize()
    for b in range(B):
        for h in range(H):
            want = Dr.keep_mask(b, h, N, N, p8, seed)
            got_fwd = P.head(o, b, h)[:, :N] != 0
            got_bwd = P.head(dv, b, h)[:, :N].T != 0
            assert np.array_equal(got_fwd, want), (b, h, "forward")
            assert np.array_equal(got_bwd, want), (b, h, "dK/dV kernel")
            assert 0.3 < want.mean() < 0.7


def _head_errors(w, inp, host, b, h, kv_lens, p8, seed):
    s = Dr.drop_scale(p8)
    kl = None if kv_lens is None else int(kv_lens[b])
    keep = Dr.keep_mask(b, h, w.N, w.N, p8, seed) if p8 else None
    args = (inp["q"][b, h], inp["k"][b, h], inp["v"][b, h])
    O, L = oracle.forward_head(*args, w.scale, w.causal, kv_len=kl,
                               drop_keep=keep, drop_scale=s)
    dQ, dK, dV, _ = oracle.backward_head(*args, inp["do"][b, h], w.scale,
                                         w.causal, kv_len=kl, drop_keep=keep,
                                         drop_scale=s)
    go, gl = P.head(host["o"], b, h), P.head(host["lse"], b, h)
    err = {"o": float("inf"), "lse": float("inf"), "dq": float("inf"),
           "dk": float("inf"), "dv": float("inf")}
    finite = np.isfinite(L)
    if not (np.isfinite(go).all() and
            np.array_equal(np.isfinite(gl), finite) and
            np.array_equal(np.isneginf(gl), np.isneginf(L))):
        return err
    err["o"] = float(np.abs(go - O).max())
    err["lse"] = (float(np.abs(gl[finite] - L[finite]).max())
                  if finite.any() else 0.0)
    for name, ref in (("dq", dQ), ("dk", dK), ("dv", dV)):
        g = P.head(host[name], b, h)
        if not np.isfinite(g).all():
            return err
        den = max(float(np.abs(ref).max()), P.GRAD_FLOOR)
        err[name] = float(np.abs(g - ref).max()) / den
    if kl is not None:      # padded keys: exactly zero gradients
        if (P.head(host["dk"], b, h)[kl:].any()
                or P.head(host["dv"], b, h)[kl:].any()):
            err["dk"] = err["dv"] = float("inf")
    return err


def _check(w, inp, out, heads, kv_lens, p8, seed):
    host = P.host_copy(out)
    res = P._map_heads(lambda b, h: _head_errors(w, inp, host, b, h,
                                                 kv_lens, p8, seed),
                       heads, w.name)
    worst = {k_: max(r[k_] for r in res.values())
             for k_ in ("o", "lse", "dq", "dk", "dv")}
    P.say("  " + " ".join(f"{k_}={v_:.3e}" for k_, v_ in worst.items())
          + f" over {len(heads)} heads")
    assert worst["o"] <= P.TOL_O_BF16 and worst["lse"] <= P.TOL_L, worst
    assert max(worst["dq"], worst["dk"], worst["dv"]) <= P.TOL_G_BF16, worst


def _run(w, inp, p, seed, kv_lens):
    P.say(f"[gpu] dropout/padding {w.name} B={w.B} H={w.H} N={w.N} d={w.D} "
          f"causal={w.causal} p={p} kv_lens={kv_lens} scale={w.scale:.6g}")
    q, k, v, do = (W.to_torch(inp[x], "bf16", "cuda") for x in
                   ("q", "k", "v", "do"))
    kl = (None if kv_lens is None else
          torch.tensor(kv_lens, dtype=torch.int32, device="cuda"))
    o, lse = fa.fa_fwd_ex(q, k, v, w.scale, w.causal, p, seed, kl)
    dq, dk, dv = fa.fa_bwd_ex(q, k, v, o, lse, do, w.scale, w.causal, p,
                              seed, kl)
    torch.cuda.synchronize()
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


CASES = [
    # name, B, H, N, D, causal, p, kv_lens
    ("drop_causal_d128", 1, 2, 200, 128, True, 0.1, None),
    ("drop_dense_d64", 2, 2, 257, 64, False, 0.3, None),
    ("drop_half_d128", 1, 2, 384, 128, False, 0.5, None),
    ("pad_only_d128", 4, 2, 300, 128, False, 0.0, [0, 1, 137, 300]),
    ("pad_causal_d64", 4, 2, 257, 64, True, 0.0, [257, 200, 64, 3]),
    ("drop_pad_causal_d128", 2, 2, 333, 128, True, 0.2, [333, 130]),
    ("drop_pad_dense_d64", 2, 2, 190, 64, False, 0.25, [5, 190]),
    # softmax scales other than 1/sqrt(d)
    ("drop_pad_causal_d128_s0.3", 2, 2, 260, 128, True, 0.2, [260, 77], 0.3),
    ("drop_dense_d64_s0.05", 1, 2, 200, 64, False, 0.1, None, 0.05),
    # sharp rows (scale 1: nearly one-hot softmax)
    ("drop_pad_causal_d64_s1", 2, 2, 230, 64, True, 0.2, [230, 101], 1.0),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_dropout_padding_every_head(case):
    name, B, H, N, D, causal, p, kv_lens = case[:8]
    scale = case[8] if len(case) > 8 else None
    w = W.small_case(name, B, H, N, D, "bf16", causal, 1100 + N + D,
                     scale=scale)
    inp = W.make_inputs(w)
    seed = 0x9E3779B97F4A7C15 ^ N
    out = _run(w, inp, p, seed, kv_lens)
    _check(w, inp, out, [(b, h) for b in range(B) for h in range(H)],
           kv_lens, Dr.quantize_p(p), seed)


def test_no_options_is_the_plain_path():
    w = W.small_case("plain", 2, 2, 200, 128, "bf16", True, 71)
    inp = W.make_inputs(w)
    q, k, v, do = (W.to_torch(inp[x], "bf16", "cuda") for x in
                   ("q", "k", "v", "do"))
    o1, l1 = fa.fa_fwd(q, k, v, w.scale, True)
    full = torch.full((2,), 200, dtype=torch.int32, device="cuda")
    o2, l2 = fa.fa_fwd_ex(q, k, v, w.scale, True, 0.0, 5, full)
    g1 = fa.fa_bwd(q, k, v, o1, l1, do, w.scale, True)
    g2 = fa.fa_bwd_ex(q, k, v, o2, l2, do, w.scale, True, 0.0, 5, full)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_dropout_headline_shape_sampled_head():
    """B=2, H=32, N=4096, d=128, causal, p = 0.1: one head against the
    oracle, forward and backward."""
    w = W.get("c3")
    inp = W.make_inputs(w)
    seed = 2024
    out = _run(w, inp, 0.1, seed, None)
    _check(w, inp, out, [(1, 17)], None, Dr.quantize_p(0.1), seed)


def test_padding_workload_every_head():
    """The key-padding bench workload at full size (B=64, H=16, N=1024,
    d=64, valid keys per batch entry uniform on [256, 1024]), as bench.py
    launches it; every head against the oracle, padded key rows of dK, dV
    exactly zero."""
    w = W.padding_workload()
    lens = W.padding_lengths(w.B, w.N)
    inp = W.make_inputs(w)
    out = _run(w, inp, 0.0, 0, lens)
    _check(w, inp, out, [(b, h) for b in range(w.B) for h in range(w.H)],
           lens, 0, 0)
