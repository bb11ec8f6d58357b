"""Pins for the dropout generator and the key-padding / dropout extensions of
the oracle, independent of the oracle's own code: the generator's published
known-answer vectors, the byte layout of one generator call written out by
hand, keep-rate statistics, the unbiasedness of the scaled dropout, finite
differences of the gradient with a fixed mask, the row-term identity, and
key padding against the definition on truncated keys.
"""
import math

import numpy as np
import pytest

from oracle import attention as A
from oracle import dropout as Dr


# Known-answer vectors of Philox4x32-10 distributed with the Random123
# library of "Parallel random numbers: as easy as 1, 2, 3" (counter words,
# key words -> output words).
KAT = [
    ((0, 0, 0, 0), (0, 0),
     (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF, 0xFFFFFFFF),
     (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344),
     (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


@pytest.mark.parametrize("ctr,key,want", KAT)
def test_philox_known_answers(ctr, key, want):
    out = Dr.philox4x32_10(*ctr, *key)
    assert tuple(int(x) for x in out) == want


def test_philox_vectorised_equals_scalar():
    rng = np.random.default_rng(1)
    c = rng.integers(0, 2 ** 32, size=(4, 50), dtype=np.uint64)
    out = Dr.philox4x32_10(c[0], c[1], c[2], c[3], 123, 456)
    for j in range(50):
        one = Dr.philox4x32_10(int(c[0, j]), int(c[1, j]), int(c[2, j]),
                               int(c[3, j]), 123, 456)
        assert [int(x) for x in one] == [int(o[j]) for o in out]


def test_keep_bytes_layout_of_one_call():
    # Query 4*qq + r, key 4*kq + c of head (b, h) is byte 4r + c of the call
    # with counter (kq, qq, h, b), bytes little-endian within each word.
    seed = 0x0123456789ABCDEF
    b, h = 1, 3
    kb = Dr.keep_bytes(b, h, 12, 20, seed)
    for qq in range(3):
        for kq in range(5):
            words = [int(x) for x in Dr.philox4x32_10(
                kq, qq, h, b, seed & 0xFFFFFFFF, seed >> 32)]
            raw = b"".join(w.to_bytes(4, "little") for w in words)
            block = kb[4 * qq: 4 * qq + 4, 4 * kq: 4 * kq + 4]
            assert block.reshape(-1).tobytes() == raw


def test_keep_rate_and_quantised_probability():
    assert Dr.quantize_p(0.0) == 0 and Dr.quantize_p(0.1) == 26
    assert Dr.quantize_p(0.5) == 128 and Dr.drop_scale(128) == 2.0
    with pytest.raises(ValueError):
        Dr.quantize_p(0.999)
    with pytest.raises(ValueError):
        Dr.quantize_p(1.0)
    keep = Dr.keep_mask(0, 0, 512, 512, 77, 99)
    n, want = keep.size, (256 - 77) / 256
    sigma = math.sqrt(want * (1 - want) / n)
    assert abs(keep.mean() - want) < 5 * sigma
    assert Dr.keep_mask(0, 0, 64, 64, 0, 5).all()
    # Different heads and seeds give different masks.
    a = Dr.keep_mask(0, 0, 64, 64, 128, 5)
    assert (a != Dr.keep_mask(0, 1, 64, 64, 128, 5)).mean() > 0.4
    assert (a != Dr.keep_mask(0, 0, 64, 64, 128, 6)).mean() > 0.4


def _qkv(rng, n, d):
    return (rng.standard_normal((n, d)) for _ in range(3))


def test_no_dropout_equals_plain():
    rng = np.random.default_rng(2)
    q, k, v = _qkv(rng, 40, 8)
    o0, l0 = A.forward_head(q, k, v, 0.3, True)
    keep = Dr.keep_mask(0, 0, 40, 40, 0, 17)
    o1, l1 = A.forward_head(q, k, v, 0.3, True, drop_keep=keep, drop_scale=1.0)
    np.testing.assert_array_equal(o0, o1)
    np.testing.assert_array_equal(l0, l1)


def test_scaled_dropout_is_unbiased():
    rng = np.random.default_rng(3)
    q, k, v = _qkv(rng, 8, 4)
    o = A.forward_head(q, k, v, 0.5, False)[0]
    p8 = Dr.quantize_p(0.3)
    acc = np.zeros_like(o)
    n = 4000
    sq = np.zeros_like(o)
    for seed in range(n):
        od = A.forward_head(q, k, v, 0.5, False,
                            drop_keep=Dr.keep_mask(0, 0, 8, 8, p8, seed),
                            drop_scale=Dr.drop_scale(p8))[0]
        acc += od
        sq += od ** 2
    mean = acc / n
    se = np.sqrt((sq / n - mean ** 2) / n)
    assert np.all(np.abs(mean - o) < 5 * se + 1e-12)


def _loss(q, k, v, do, scale, causal, kv_len, keep, s):
    return float((A.forward_head(q, k, v, scale, causal, kv_len=kv_len,
                                 drop_keep=keep, drop_scale=s)[0] * do).sum())


@pytest.mark.parametrize("causal,kv_len", [(False, None), (True, None),
                                           (False, 5), (True, 6)])
def test_dropout_gradient_finite_differences(causal, kv_len):
    rng = np.random.default_rng(4)
    n, d, scale = 8, 4, 0.7
    q, k, v = _qkv(rng, n, d)
    do = rng.standard_normal((n, d))
    p8 = Dr.quantize_p(0.25)
    keep, s = Dr.keep_mask(0, 1, n, n, p8, 1234), Dr.drop_scale(p8)
    assert 0 < keep.mean() < 1
    dq, dk, dv, _ = A.backward_head(q, k, v, do, scale, causal, kv_len=kv_len,
                                    drop_keep=keep, drop_scale=s)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            fp = _loss(args["q"], args["k"], args["v"], do, scale, causal,
                       kv_len, keep, s)
            args[name] = xm
            fm = _loss(args["q"], args["k"], args["v"], do, scale, causal,
                       kv_len, keep, s)
            num[idx] = (fp - fm) / (2 * eps)
        rel = np.abs(num - g).max() / max(np.abs(num).max(), 1e-12)
        assert rel < 1e-6, (name, rel)
    if kv_len is not None:      # padded keys get no gradient
        assert not dk[kv_len:].any() and not dv[kv_len:].any()


def test_row_term_identity_with_dropout():
    rng = np.random.default_rng(5)
    n, d = 30, 16
    q, k, v = _qkv(rng, n, d)
    do = rng.standard_normal((n, d))
    p8 = Dr.quantize_p(0.4)
    keep, s = Dr.keep_mask(2, 3, n, n, p8, 77), Dr.drop_scale(p8)
    o = A.forward_head(q, k, v, 0.25, True, drop_keep=keep, drop_scale=s)[0]
    D = A.backward_head(q, k, v, do, 0.25, True, drop_keep=keep,
                        drop_scale=s)[3]
    np.testing.assert_allclose(A.delta_closed_form(o, do), D, rtol=1e-12,
                               atol=1e-12)


def test_key_padding_is_truncation():
    rng = np.random.default_rng(6)
    n, d = 50, 8
    q, k, v = _qkv(rng, n, d)
    for kv_len in (1, 17, 50):
        o, l = A.forward_head(q, k, v, 0.4, False, kv_len=kv_len)
        o2, l2 = A.forward_head(q, k[:kv_len], v[:kv_len], 0.4, False)
        np.testing.assert_allclose(o, o2, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(l, l2, rtol=1e-13, atol=1e-14)
    o, l = A.forward_head(q, k, v, 0.4, False, kv_len=0)
    assert not o.any() and np.all(l == -np.inf)
    # causal and padding intersect: row 3 with kv_len 2 sees keys 0, 1
    o, _ = A.forward_head(q, k, v, 0.4, True, kv_len=2)
    o2, _ = A.forward_head(q[3:4], k[:2], v[:2], 0.4, False)
    np.testing.assert_allclose(o[3], o2[0], rtol=1e-13)
