"""Largest memory spans the C ABI accepts.

A bf16 head may span up to 2^31 bytes: (N + 256) * sn * 2 < 2^31, since the
kernels address one head with 32-bit buffer offsets and descriptor ranges,
and a ragged last tile may load up to 256 rows past the end of a head.  An
fp32 head may span up to 2^31 elements ((N - 1) * sn + d < 2^31).  Heads and
batches may lie anywhere (64-bit offsets).  Each case below puts every head
at that limit. A row stride far above d keeps the arithmetic small, and
several heads make the later ones start past 4 GiB.  Every head is then
checked against the oracle.  The memory between the rows is NaN before
each call and must still be NaN after it, so no store may land between the
rows.  A packed variable-length batch puts its whole packed tensor at its
limit; a split-KV call puts its keys and values there; dropout with key
padding and the FP8 forward (which quantises straight from the strided bf16
inputs) run on heads at the limit too.
"""
import numpy as np
import pytest
import torch

import io_aware_exact_04_amd as fa
import oracle
import workloads as W
from tests import _parity as P

pytestmark = pytest.mark.gpu

LIMIT = 1 << 31
TRAIL = 4096       # guard elements after the last row


def largest_sn(rows: int, width: int, dtype: str) -> int:
    """The largest row stride (a 16-byte multiple) the library accepts for
    `rows` rows whose last row ends `width` elements after its start."""
    if dtype == "bf16":
        sn = (LIMIT - 1) // (2 * (rows + 256))
        step = 8
        assert (rows + 256) * (sn - sn % step + step) * 2 >= LIMIT
    else:
        sn = (LIMIT - 1 - width) // max(rows - 1, 1)
        step = 4
    return sn - sn % step


class Spread:
    """A view of `shape` (last dim contiguous) whose rows start `sn`
    elements apart inside a NaN-filled buffer: `rows` rows of `width` used
    elements, then the gap up to the next row, then TRAIL guard elements."""

    def __init__(self, shape, strides, rows, width, sn, dtype, src=None):
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.rows, self.width, self.sn = rows, width, sn
        self.buf = torch.full((rows * sn + TRAIL,), float("nan"), dtype=tdt,
                              device="cuda")
        self.view = self.buf.as_strided(shape, strides)
        if src is not None:
            self.view.copy_(W.to_torch(src, dtype, "cuda"))

    @classmethod
    def heads(cls, B, H, N, d, sn, dtype, src=None):
        """[B, H, N, d], heads one after another, each N rows of stride sn."""
        return cls((B, H, N, d), (H * N * sn, N * sn, sn, 1), B * H * N, d,
                   sn, dtype, src)

    def gaps_untouched(self) -> bool:
        gaps = self.buf.as_strided((self.rows, self.sn - self.width),
                                   (self.sn, 1), self.width)
        step = max(1, (1 << 28) // (self.sn - self.width))
        for r0 in range(0, self.rows, step):
            if not bool(torch.isnan(gaps[r0:r0 + step]).all()):
                return False
        return bool(torch.isnan(self.buf[self.rows * self.sn:]).all())

    def release(self):
        del self.view, self.buf


def _need(nbytes: int):
    """Skip (not fail) when the device lacks the memory a case needs: the
    cases here are about offsets, not about how much memory a box has."""
    free, _ = torch.cuda.mem_get_info()
    if free < nbytes * 1.1:
        pytest.skip(f"needs {nbytes / 2**30:.1f} GiB of device memory, "
                    f"{free / 2**30:.1f} GiB free")


def _free(*spreads):
    for s in spreads:
        s.release()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


CASES = [
    # name, B, H, N, d, dtype, causal
    ("bf16_d128_dense_ragged", 2, 2, 4000, 128, "bf16", False),
    ("bf16_d64_causal", 2, 2, 1000, 64, "bf16", True),
    ("fp32_d64_causal", 1, 1, 300, 64, "fp32", True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fwd_bwd_at_the_largest_head_span(case):
    name, B, H, N, D, dtype, causal = case
    sn = largest_sn(N, D, dtype)
    w = W.small_case(f"limit_{name}", B, H, N, D, dtype, causal,
                     seed=9100 + N + D)
    inp = W.make_inputs(w)
    elt = 2 if dtype == "bf16" else 4
    _need(8 * (B * H * N * sn + TRAIL) * elt)
    P.say(f"[gpu] limit {name} B={B} H={H} N={N} d={D} {dtype} "
          f"causal={causal} sn={sn}: head span "
          f"{((N - 1) * sn + D) * elt / 2**30:.3f} GiB, last head at "
          f"{(B * H - 1) * N * sn * elt / 2**30:.2f} GiB")
    q, k, v, do = (Spread.heads(B, H, N, D, sn, dtype, inp[x])
                   for x in ("q", "k", "v", "do"))
    o, dq, dk, dv = (Spread.heads(B, H, N, D, sn, dtype) for _ in range(4))
    lse = torch.full((B, H, N), float("nan"), device="cuda")
    fa.fa_fwd(q.view, k.view, v.view, w.scale, causal, out=o.view, lse=lse)
    fa.fa_bwd(q.view, k.view, v.view, o.view, lse, do.view, w.scale, causal,
              out=(dq.view, dk.view, dv.view))
    torch.cuda.synchronize()
    for t, nm in ((o, "o"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
        assert t.gaps_untouched(), f"{nm}: written between its rows"
    heads = P.all_heads(w)
    host = {"o": o.view.float().cpu(), "lse": lse.cpu(),
            "dq": dq.view.float().cpu(), "dk": dk.view.float().cpu(),
            "dv": dv.view.float().cpu()}
    _free(q, k, v, do, o, dq, dk, dv)
    P.check_forward(w, inp, host, heads)
    P.check_backward(w, inp, host, heads)


def test_varlen_packed_tensor_at_the_largest_span():
    lengths, H, D = [1000, 1, 1999, 0, 1000], 2, 128
    inp = W.make_varlen_inputs(lengths, H, D, seed=9200)
    total = int(sum(lengths))
    sn = largest_sn(total, H * D, "bf16")
    _need(8 * (total * sn + TRAIL) * 2)
    P.say(f"[gpu] limit varlen total={total} H={H} d={D} sn={sn}: packed "
          f"span {((total - 1) * sn + H * D) * 2 / 2**30:.3f} GiB")

    def packed(src=None):
        return Spread((total, H, D), (sn, D, 1), total, H * D, sn, "bf16",
                      src)
    q, k, v, do = (packed(inp[x]) for x in ("q", "k", "v", "do"))
    o, dq, dk, dv = (packed() for _ in range(4))
    cu = torch.from_numpy(inp["cu_seqlens"]).cuda()
    max_len = max(lengths)
    _, lse = fa.fa_fwd_varlen(q.view, k.view, v.view, cu, max_len,
                              causal=True, out=o.view)
    fa.fa_bwd_varlen(q.view, k.view, v.view, o.view, lse, do.view, cu,
                     max_len, causal=True, out=(dq.view, dk.view, dv.view))
    torch.cuda.synchronize()
    for t, nm in ((o, "o"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
        assert t.gaps_untouched(), f"{nm}: written between its rows"
    got = {nm: t.view.float().cpu().numpy().astype(np.float64)
           for nm, t in (("o", o), ("dq", dq), ("dk", dk), ("dv", dv))}
    got["lse"] = lse.cpu().numpy().astype(np.float64)
    _free(q, k, v, do, o, dq, dk, dv)
    cus = inp["cu_seqlens"]
    scale = 1.0 / np.sqrt(D)
    worst = {"o": 0.0, "lse": 0.0, "dq": 0.0, "dk": 0.0, "dv": 0.0}
    gmax = {"dq": 0.0, "dk": 0.0, "dv": 0.0}
    for s in range(len(lengths)):
        a, b = int(cus[s]), int(cus[s + 1])
        for h in range(H):
            if a == b:
                continue
            x = {nm: inp[nm][a:b, h] for nm in ("q", "k", "v", "do")}
            O, L = oracle.forward_head(x["q"], x["k"], x["v"], scale, True)
            worst["o"] = max(worst["o"], float(np.abs(got["o"][a:b, h] - O).max()))
            worst["lse"] = max(worst["lse"],
                               float(np.abs(got["lse"][h, a:b] - L).max()))
            refs = oracle.backward_head(x["q"], x["k"], x["v"], x["do"],
                                        scale, True)
            for nm, ref in zip(("dq", "dk", "dv"), refs[:3]):
                worst[nm] = max(worst[nm],
                                float(np.abs(got[nm][a:b, h] - ref).max()))
                gmax[nm] = max(gmax[nm], float(np.abs(ref).max()))
    for nm in gmax:
        worst[nm] /= max(gmax[nm], P.GRAD_FLOOR)
    P.say("  " + " ".join(f"{k_}={v_:.3e}" for k_, v_ in worst.items()))
    assert worst["o"] <= P.TOL_O_BF16 and worst["lse"] <= P.TOL_L
    for nm in gmax:
        assert worst[nm] <= P.TOL_G_BF16, (nm, worst[nm])


@pytest.mark.parametrize("nq", [1, 64], ids=["decode", "query_block"])
def test_splitkv_keys_at_the_largest_span(nq):
    B, H, Nk, D, splits = 2, 2, 5000, 128, 4
    w = W.KvWorkload(f"limit_kv_{nq}", B, H, nq, Nk, D, True,
                     seed=9300 + nq, num_splits=splits)
    inp = W.make_kv_inputs(w)
    sn = largest_sn(Nk, D, "bf16")
    _need(2 * (B * H * Nk * sn + TRAIL) * 2)
    P.say(f"[gpu] limit splitkv B={B} H={H} Nq={nq} Nk={Nk} d={D} "
          f"splits={splits} kv sn={sn}: head span "
          f"{((Nk - 1) * sn + D) * 2 / 2**30:.3f} GiB")
    q = W.to_torch(inp["q"], "bf16", "cuda")
    k, v = (Spread.heads(B, H, Nk, D, sn, "bf16", inp[x]) for x in ("k", "v"))
    o, lse = fa.fa_fwd_splitkv(q, k.view, v.view, w.scale, True, splits)
    torch.cuda.synchronize()
    assert k.gaps_untouched() and v.gaps_untouched()
    go = o.float().cpu().numpy().astype(np.float64)
    gl = lse.cpu().numpy().astype(np.float64)
    _free(k, v)
    worst_o = worst_l = 0.0
    for b in range(B):
        for h in range(H):
            O, L = oracle.forward_head(inp["q"][b, h], inp["k"][b, h],
                                       inp["v"][b, h], w.scale, True,
                                       causal_offset=Nk - nq)
            worst_o = max(worst_o, float(np.abs(go[b, h] - O).max()))
            worst_l = max(worst_l, float(np.abs(gl[b, h] - L).max()))
    P.say(f"  max|dO|={worst_o:.3e} max|dL|={worst_l:.3e}")
    assert worst_o <= P.TOL_O_BF16 and worst_l <= P.TOL_L


def test_dropout_padding_at_the_largest_head_span():
    """fa_fwd_ex / fa_bwd_ex with dropout and key padding, every head at the
    bf16 limit, against the oracle with the same Philox keep masks."""
    from oracle import dropout as Dr
    from tests.test_dropout_gpu import _check as check_dropout
    B, H, N, D, p, seed = 2, 2, 3000, 128, 0.1, 0x5EED0123
    kv_lens = [2411, 2963]
    w = W.small_case("limit_drop", B, H, N, D, "bf16", True, seed=9400)
    inp = W.make_inputs(w)
    sn = largest_sn(N, D, "bf16")
    _need(8 * (B * H * N * sn + TRAIL) * 2)
    P.say(f"[gpu] limit dropout/padding B={B} H={H} N={N} d={D} p={p} "
          f"kv_lens={kv_lens} sn={sn}: head span "
          f"{((N - 1) * sn + D) * 2 / 2**30:.3f} GiB")
    q, k, v, do = (Spread.heads(B, H, N, D, sn, "bf16", inp[x])
                   for x in ("q", "k", "v", "do"))
    o, dq, dk, dv = (Spread.heads(B, H, N, D, sn, "bf16") for _ in range(4))
    kl = torch.tensor(kv_lens, dtype=torch.int32, device="cuda")
    lse = torch.full((B, H, N), float("nan"), device="cuda")
    fa.fa_fwd_ex(q.view, k.view, v.view, w.scale, True, p, seed, kl,
                 out=o.view, lse=lse)
    fa.fa_bwd_ex(q.view, k.view, v.view, o.view, lse, do.view, w.scale, True,
                 p, seed, kl, out=(dq.view, dk.view, dv.view))
    torch.cuda.synchronize()
    for t, nm in ((o, "o"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
        assert t.gaps_untouched(), f"{nm}: written between its rows"
    host = {"o": o.view.float().cpu(), "lse": lse.cpu(),
            "dq": dq.view.float().cpu(), "dk": dk.view.float().cpu(),
            "dv": dv.view.float().cpu()}
    _free(q, k, v, do, o, dq, dk, dv)
    check_dropout(w, inp, host, P.all_heads(w), kv_lens, Dr.quantize_p(p),
                  seed)


@pytest.mark.parametrize("D,causal", [(128, True), (64, False)])
def test_fp8_forward_at_the_largest_head_span(D, causal):
    """The FP8 forward quantises straight from the strided bf16 inputs:
    every head at the limit against the FP8 oracle (L within the bf16
    tolerance, O within the P-rounding bound)."""
    from oracle import fp8 as F
    B, H, N = 2, 2, 3000
    w = W.small_case(f"limit_fp8_{D}", B, H, N, D, "bf16", causal,
                     seed=9500 + D)
    inp = W.make_inputs(w, with_grad=False)
    signs = W.hadamard_signs(D, 9501 + D)
    sn = largest_sn(N, D, "bf16")
    _need(4 * (B * H * N * sn + TRAIL) * 2)
    P.say(f"[gpu] limit fp8 forward B={B} H={H} N={N} d={D} causal={causal} "
          f"sn={sn}: head span {((N - 1) * sn + D) * 2 / 2**30:.3f} GiB")
    q, k, v = (Spread.heads(B, H, N, D, sn, "bf16", inp[x])
               for x in ("q", "k", "v"))
    o = Spread.heads(B, H, N, D, sn, "bf16")
    lse = torch.full((B, H, N), float("nan"), device="cuda")
    fa.fa_fwd_fp8(q.view, k.view, v.view, w.scale, causal, signs, True,
                  out=o.view, lse=lse)
    torch.cuda.synchronize()
    assert o.gaps_untouched(), "o: written between its rows"
    go_all, gl_all = o.view.float().cpu(), lse.cpu()
    _free(q, k, v, o)

    def head_errors(b, h):
        r = F.fp8_forward_head(inp["q"][b, h], inp["k"][b, h],
                               inp["v"][b, h], w.scale, causal, signs, True)
        go, gl = P.head(go_all, b, h), P.head(gl_all, b, h)
        if not (np.isfinite(go).all() and np.isfinite(gl).all()):
            return float("inf"), float("inf")
        bound = F.p_rounding_bound(r) + 2.0 ** -8 * np.abs(r["O"]) + 2e-5
        return (float(np.abs(gl - r["L"]).max()),
                float((np.abs(go - r["O"]) / bound).max()))
    res = P._map_heads(head_errors, P.all_heads(w), w.name).values()
    dl = max(r[0] for r in res)
    ob = max(r[1] for r in res)
    P.say(f"  max|dL|={dl:.3e} (tol {P.TOL_L}) max|dO|/bound={ob:.3f} (<= 1)")
    assert dl <= P.TOL_L and ob <= 1.0
