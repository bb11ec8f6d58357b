"""GPU checks of properties the method guarantees at any size: determinism,
masked positions being irrelevant, all-ones masks equal to dense, empty rows,
full overwrite of the outputs, stride handling and empty problems."""
import numpy as np
import pytest
import torch

import io_aware_exact_04_amd as fa
import oracle
import workloads as W
from tests import _parity as P

pytestmark = pytest.mark.gpu


def _inputs(B, H, N, D, dtype="bf16", causal=False, seed=7, **kw):
    w = W.small_case("t", B, H, N, D, dtype, causal, seed, **kw)
    inp = W.make_inputs(w)
    return w, inp, P.to_dev(inp, w)


@pytest.mark.parametrize("D", [64, 128])
def test_forward_is_bitwise_deterministic(D):
    w, inp, (q, k, v, do, _) = _inputs(2, 4, 1000, D, causal=True)
    o1, l1 = fa.fa_fwd(q, k, v, causal=True)
    o2, l2 = fa.fa_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("D", [64, 128])
def test_backward_is_bitwise_deterministic(D):
    # No kernel uses atomics: dQ, dK and dV repeat bit for bit.
    w, inp, (q, k, v, do, _) = _inputs(1, 2, 700, D, causal=True)
    o, l = fa.fa_fwd(q, k, v, causal=True)
    g1 = fa.fa_bwd(q, k, v, o, l, do, causal=True)
    g2 = fa.fa_bwd(q, k, v, o, l, do, causal=True)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("D", [64, 128])
def test_causal_future_keys_do_not_matter(D):
    w, inp, (q, k, v, do, _) = _inputs(1, 2, 512, D, causal=True)
    o1, l1 = fa.fa_fwd(q, k, v, causal=True)
    k2, v2 = k.clone(), v.clone()
    k2[:, :, 300:] = 40.0
    v2[:, :, 300:] = -1000.0
    o2, l2 = fa.fa_fwd(q, k2, v2, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1[:, :, :300], o2[:, :, :300])
    assert torch.equal(l1[:, :, :300], l2[:, :, :300])


@pytest.mark.parametrize("D", [64, 128])
def test_all_ones_block_mask_equals_dense(D):
    w, inp, (q, k, v, do, _) = _inputs(1, 2, 500, D)
    ones = torch.ones((2, 2), dtype=torch.uint8, device="cuda")
    o1, l1 = fa.fa_fwd(q, k, v)
    o2, l2 = fa.fa_fwd(q, k, v, block_mask=ones, mask_block=256)
    g1 = fa.fa_bwd(q, k, v, o1, l1, do)
    g2 = fa.fa_bwd(q, k, v, o2, l2, do, block_mask=ones, mask_block=256)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        torch.testing.assert_close(a.float(), b.float(), rtol=0, atol=2e-2)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_fully_masked_rows(dtype):
    w, inp, (q, k, v, do, _) = _inputs(1, 2, 384, 64, dtype=dtype)
    bm = np.ones((3, 3), np.uint8)
    bm[1] = 0  # queries 128..255 see no key
    m = torch.from_numpy(bm).cuda()
    o, l = fa.fa_fwd(q, k, v, block_mask=m, mask_block=128)
    dq, dk, dv = fa.fa_bwd(q, k, v, o, l, do, block_mask=m, mask_block=128)
    torch.cuda.synchronize()
    assert (o[:, :, 128:256] == 0).all()
    assert torch.isneginf(l[:, :, 128:256]).all()
    assert torch.isfinite(l[:, :, :128]).all()
    assert (dq[:, :, 128:256] == 0).all()
    for t in (o, dq, dk, dv):
        assert torch.isfinite(t).all()
    wm = W.small_case("m", 1, 2, 384, 64, dtype, False, 7, mask_block=128)
    P.check_backward(wm, dict(inp, block_mask=bm), {"dq": dq, "dk": dk,
                                                    "dv": dv}, [(0, 1)])


def test_outputs_fully_overwritten():
    w, inp, (q, k, v, do, _) = _inputs(1, 3, 333, 128, causal=True)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((1, 3, 333), float("nan"), device="cuda")
    fa.fa_fwd(q, k, v, causal=True, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()


@pytest.mark.parametrize("D", [64, 128])
def test_strided_layout_matches_contiguous(D):
    w, inp, (q, k, v, do, _) = _inputs(2, 3, 260, D, causal=True)
    # [B, N, H, d] storage viewed as [B, H, N, d]
    qs, ks, vs, dos = (x.transpose(1, 2).contiguous().transpose(1, 2)
                       for x in (q, k, v, do))
    assert qs.stride() != q.stride()
    o1, l1 = fa.fa_fwd(q, k, v, causal=True)
    o2, l2 = fa.fa_fwd(qs, ks, vs, causal=True)
    g1 = fa.fa_bwd(q, k, v, o1, l1, do, causal=True)
    g2 = fa.fa_bwd(qs, ks, vs, o2, l2, dos, causal=True)
    torch.cuda.synchronize()
    assert o2.stride() == qs.stride()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_empty_problem():
    q = torch.empty((2, 0, 64, 64), dtype=torch.bfloat16, device="cuda")
    o, l = fa.fa_fwd(q, q, q)
    assert o.shape == q.shape and l.shape == (2, 0, 64)
    q = torch.empty((1, 2, 0, 128), dtype=torch.bfloat16, device="cuda")
    o, l = fa.fa_fwd(q, q, q)
    dq, dk, dv = fa.fa_bwd(q, q, q, o, l, q)
    assert dq.shape == q.shape


def test_autograd_function():
    w, inp, (q, k, v, do, _) = _inputs(1, 2, 200, 64, causal=True)
    qq, kk, vv = (x.clone().requires_grad_(True) for x in (q, k, v))
    out = fa.attention(qq, kk, vv, causal=True)
    out.backward(do)
    torch.cuda.synchronize()
    O, _ = oracle.forward_head(inp["q"][0, 1], inp["k"][0, 1], inp["v"][0, 1],
                               w.scale, True)
    assert np.abs(P.head(out.detach(), 0, 1) - O).max() <= P.TOL_O_BF16
    P.check_backward(w, inp, {"dq": qq.grad, "dk": kk.grad, "dv": vv.grad},
                     [(0, 0), (0, 1)])


def _bshd(x):
    """The same values stored as [B, N, H, d] and viewed as [B, H, N, d]."""
    return x.transpose(1, 2).contiguous().transpose(1, 2)


@pytest.mark.parametrize("D", [64, 128])
def test_strided_layout_next_rows(D):
    """Split-KV, dropout with key padding, and the FP8 forward read and write
    [B, N, H, d]-strided tensors exactly as contiguous ones."""
    w, inp, (q, k, v, do, _) = _inputs(2, 3, 300, D, causal=True, seed=11)
    qs, ks, vs, dos = (_bshd(x) for x in (q, k, v, do))
    assert qs.stride() != q.stride()
    # split-KV: the last 40 queries against all 300 keys
    o1, l1 = fa.fa_fwd_splitkv(q[:, :, -40:], k, v, causal=True, num_splits=3)
    o2, l2 = fa.fa_fwd_splitkv(qs[:, :, -40:], ks, vs, causal=True,
                               num_splits=3)
    # and the last query alone (the one-row decode pass)
    d1, m1 = fa.fa_fwd_splitkv(q[:, :, -1:], k, v, causal=True, num_splits=3)
    d2, m2 = fa.fa_fwd_splitkv(qs[:, :, -1:], ks, vs, causal=True,
                               num_splits=3)
    # dropout and key padding
    kl = torch.tensor([300, 123], dtype=torch.int32, device="cuda")
    e1 = fa.fa_fwd_ex(q, k, v, causal=True, dropout_p=0.2, seed=9, kv_lens=kl)
    e2 = fa.fa_fwd_ex(qs, ks, vs, causal=True, dropout_p=0.2, seed=9,
                      kv_lens=kl)
    g1 = fa.fa_bwd_ex(q, k, v, e1[0], e1[1], do, causal=True, dropout_p=0.2,
                      seed=9, kv_lens=kl)
    g2 = fa.fa_bwd_ex(qs, ks, vs, e2[0], e2[1], dos, causal=True,
                      dropout_p=0.2, seed=9, kv_lens=kl)
    # FP8 forward with rotation
    signs = W.hadamard_signs(D, 5)
    f1 = fa.fa_fwd_fp8(q, k, v, causal=True, signs=signs)
    f2 = fa.fa_fwd_fp8(qs, ks, vs, causal=True, signs=signs)
    torch.cuda.synchronize()
    assert o2.stride() == qs[:, :, -40:].stride() and e2[0].stride() == qs.stride()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert d2.stride() == qs[:, :, -1:].stride()
    assert torch.equal(d1, d2) and torch.equal(m1, m2)
    assert torch.equal(e1[0], e2[0]) and torch.equal(e1[1], e2[1])
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
    assert torch.equal(f1[0], f2[0]) and torch.equal(f1[1], f2[1])
