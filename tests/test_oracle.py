"""Pins for the fp64 oracle, independent of the oracle's own code.

Each test fixes a value the mathematics (or an independent library routine,
or finite differences, or a hand-derived worked example) determines, so that a
dropped term, a wrong sign or index, or a transposed operand in the oracle
fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import attention as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _masked_scores(q, k, scale, keep):
    return np.where(keep, scale * (q @ k.T), -np.inf)


# ------------------------------------------------------------ worked example

@pytest.fixture(scope="module")
def worked():
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        return json.load(f)


def test_worked_example_two_pass(worked):
    q, k, v = (np.array(worked[x]) for x in ("q", "k", "v"))
    O, L = oracle.forward_head(q, k, v, worked["scale"])
    tp = worked["two_pass"]
    assert abs(O[0, 0] - tp["O"]) < 1e-12
    assert abs(L[0] - tp["L"]) < 1e-12
    P, m, l = oracle.softmax_rows(worked["scale"] * (q @ k.T))
    assert m[0] == tp["m"]
    assert abs(l[0] - tp["l"]) < 1e-12
    np.testing.assert_allclose(P[0], tp["P"], rtol=0, atol=1e-12)


def test_worked_example_online(worked):
    q, k, v = (np.array(worked[x]) for x in ("q", "k", "v"))
    trace = []
    O, L = oracle.online_forward_head(q, k, v, worked["scale"], Br=worked["Br"],
                                      Bc=worked["Bc"], trace=trace)
    assert len(trace) == len(worked["online"])
    for (_, _, m, l, acc), want in zip(trace, worked["online"]):
        assert m[0] == want["m"]
        assert abs(l[0] - want["l"]) < 1e-12
        assert abs(acc[0, 0] - want["acc"]) < 1e-12
    assert abs(O[0, 0] - worked["two_pass"]["O"]) < 1e-12
    assert abs(L[0] - worked["two_pass"]["L"]) < 1e-12


def test_worked_example_state_merge_in_any_order(worked):
    # The two tiles' states merged in either order, with the empty state
    # on either side, give the two-pass m, l and sum of exp(s - m) v.
    from oracle import online as on
    q, k, v = (np.array(worked[x]) for x in ("q", "k", "v"))
    s = worked["scale"] * (q @ k.T)
    t1 = on.tile_state(s[:, :2], v[:2])
    t2 = on.tile_state(s[:, 2:], v[2:])
    e = on.empty_state(1, 1)
    tp = worked["two_pass"]
    want_a = sum(p * x for p, x in zip(tp["P"], v[:, 0])) * tp["l"]
    for state in (on.merge(on.merge(e, t1), t2), on.merge(t2, on.merge(t1, e)),
                  on.merge(on.merge(t2, e), t1)):
        m, l, a = state
        assert m[0] == tp["m"]
        assert abs(l[0] - tp["l"]) < 1e-12
        assert abs(a[0, 0] - want_a) < 1e-12
    m, l, a = on.merge(e, e)
    assert m[0] == -np.inf and l[0] == 0.0 and a[0, 0] == 0.0


def test_worked_example_delta(worked):
    q, k, v = (np.array(worked[x]) for x in ("q", "k", "v"))
    dO = np.full((1, 1), worked["backward"]["dO"])
    O, _ = oracle.forward_head(q, k, v, worked["scale"])
    _, _, _, D = oracle.backward_head(q, k, v, dO, worked["scale"])
    assert abs(D[0] - worked["backward"]["D"]) < 1e-12
    assert abs(oracle.delta_closed_form(O, dO)[0] - worked["backward"]["D"]) < 1e-12


# --------------------------------------------------- online == definition

@pytest.mark.parametrize("Br", [1, 2, 3, 64])
@pytest.mark.parametrize("Bc", [1, 2, 3, 64])
@pytest.mark.parametrize("case", ["dense", "causal", "mask"])
def test_online_recurrence_equals_definition(Br, Bc, case):
    rng = np.random.default_rng(100 + Br * 7 + Bc)
    N, d = 67, 5
    q, k, v = _rand(rng, N, d), 2.0 * _rand(rng, N, d), _rand(rng, N, d)
    causal = case == "causal"
    bm = None
    if case == "mask":
        bm = (rng.random((9, 9)) < 0.5).astype(np.uint8)
        np.fill_diagonal(bm, 1)
    O1, L1 = oracle.forward_head(q, k, v, 0.3, causal, bm, 8)
    O2, L2 = oracle.online_forward_head(q, k, v, 0.3, Br, Bc, causal, bm, 8)
    np.testing.assert_allclose(O2, O1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(L2, L1, rtol=0, atol=1e-13)


# ---------------------------------------------- independent library routines

@pytest.mark.parametrize("case", ["dense", "causal", "mask"])
def test_softmax_and_lse_match_scipy(case):
    rng = np.random.default_rng(7)
    N, d = 40, 6
    q, k, v = _rand(rng, N, d), _rand(rng, N, d), _rand(rng, N, d)
    bm = (rng.random((5, 5)) < 0.6).astype(np.uint8) if case == "mask" else None
    if bm is not None:
        np.fill_diagonal(bm, 1)
    keep = A.keep_matrix(N, N, case == "causal", bm, 8)
    S = _masked_scores(q, k, 0.4, keep)
    P, _, _ = oracle.softmax_rows(S)
    np.testing.assert_allclose(P, scipy.special.softmax(S, axis=1), atol=1e-15)
    np.testing.assert_allclose(P.sum(1), 1.0, rtol=0, atol=1e-14)
    O, L = oracle.forward_head(q, k, v, 0.4, case == "causal", bm, 8)
    np.testing.assert_allclose(L, scipy.special.logsumexp(S, axis=1),
                               rtol=0, atol=1e-13)
    np.testing.assert_allclose(O, scipy.special.softmax(S, axis=1) @ v,
                               rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_forward_matches_torch_sdpa_fp64(causal):
    rng = np.random.default_rng(11)
    N, d = 33, 8
    q, k, v = _rand(rng, N, d), _rand(rng, N, d), _rand(rng, N, d)
    scale = 1.0 / math.sqrt(d)
    O, _ = oracle.forward_head(q, k, v, scale, causal)
    t = [torch.from_numpy(x)[None, None] for x in (q, k, v)]
    ref = torch.nn.functional.scaled_dot_product_attention(
        *t, is_causal=causal, scale=scale)[0, 0].numpy()
    np.testing.assert_allclose(O, ref, rtol=0, atol=1e-13)


def test_block_mask_matches_torch_sdpa_bool_mask():
    rng = np.random.default_rng(12)
    N, d, mb = 24, 4, 4
    q, k, v = _rand(rng, N, d), _rand(rng, N, d), _rand(rng, N, d)
    bm = (rng.random((6, 6)) < 0.4).astype(np.uint8)
    np.fill_diagonal(bm, 1)
    bm[0, 3] = 1
    bm[3, 0] = 0  # deliberately asymmetric: rows are query blocks
    O, _ = oracle.forward_head(q, k, v, 0.5, False, bm, mb)
    allowed = np.kron(bm, np.ones((mb, mb))).astype(bool)
    t = [torch.from_numpy(x)[None, None] for x in (q, k, v)]
    ref = torch.nn.functional.scaled_dot_product_attention(
        *t, attn_mask=torch.from_numpy(allowed)[None, None], scale=0.5)
    np.testing.assert_allclose(O, ref[0, 0].numpy(), rtol=0, atol=1e-13)


@pytest.mark.parametrize("case", ["dense", "causal", "mask"])
def test_backward_matches_torch_autograd_fp64(case):
    rng = np.random.default_rng(21)
    N, d = 20, 6
    q, k, v, do = (_rand(rng, N, d) for _ in range(4))
    bm = None
    if case == "mask":
        bm = (rng.random((5, 5)) < 0.5).astype(np.uint8)
        np.fill_diagonal(bm, 1)
    scale = 0.37
    dQ, dK, dV, _ = oracle.backward_head(q, k, v, do, scale, case == "causal",
                                         bm, 4)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    kwargs = {"scale": scale}
    if case == "causal":
        kwargs["is_causal"] = True
    if bm is not None:
        allowed = np.kron(bm, np.ones((4, 4))).astype(bool)
        kwargs["attn_mask"] = torch.from_numpy(allowed)[None, None]
    out = torch.nn.functional.scaled_dot_product_attention(
        tq[None, None], tk[None, None], tv[None, None], **kwargs)[0, 0]
    out.backward(torch.from_numpy(do))
    np.testing.assert_allclose(dQ, tq.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dK, tk.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dV, tv.grad.numpy(), rtol=0, atol=1e-12)


# ------------------------------------------------------------- closed forms

@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_give_the_mean_of_values(causal):
    rng = np.random.default_rng(3)
    N, d = 17, 5
    q, v = _rand(rng, N, d), _rand(rng, N, d)
    k = np.tile(_rand(rng, 1, d), (N, 1))
    O, L = oracle.forward_head(q, k, v, 0.7, causal)
    for i in range(N):
        n = i + 1 if causal else N
        np.testing.assert_allclose(O[i], v[:n].mean(0), rtol=0, atol=1e-13)
        s = 0.7 * float(q[i] @ k[0])
        assert abs(L[i] - (s + math.log(n))) < 1e-12


def test_causal_first_row_sees_only_first_key():
    rng = np.random.default_rng(4)
    q, k, v = (_rand(rng, 9, 3) for _ in range(3))
    O, L = oracle.forward_head(q, k, v, 1.3, causal=True)
    np.testing.assert_allclose(O[0], v[0], rtol=0, atol=0)
    assert abs(L[0] - 1.3 * float(q[0] @ k[0])) < 1e-14
    # the last row sees everything: equals the dense result there
    Od, Ld = oracle.forward_head(q, k, v, 1.3, causal=False)
    np.testing.assert_allclose(O[-1], Od[-1], atol=1e-14)
    assert abs(L[-1] - Ld[-1]) < 1e-14


def test_dominant_score_selects_its_value():
    rng = np.random.default_rng(5)
    N, d = 12, 4
    v = _rand(rng, N, d)
    q = np.zeros((N, d))
    q[:, 0] = 1.0
    k = np.zeros((N, d))
    target = (np.arange(N) * 5 + 3) % N
    k[target[0], 0] = 60.0  # margin 60 over every other key in that row
    O, L = oracle.forward_head(q[:1], k, v, 1.0)
    np.testing.assert_allclose(O[0], v[target[0]], rtol=0, atol=1e-20 + 1e-24)
    assert abs(L[0] - 60.0) < 1e-12


def test_constant_values_pass_through():
    rng = np.random.default_rng(6)
    q, k = _rand(rng, 10, 4), _rand(rng, 10, 4)
    c = np.array([1.5, -2.0, 0.25, 3.0])
    O, _ = oracle.forward_head(q, k, np.tile(c, (10, 1)), 0.5, causal=True)
    np.testing.assert_allclose(O, np.tile(c, (10, 1)), rtol=0, atol=1e-14)


def test_output_is_linear_in_values():
    rng = np.random.default_rng(8)
    q, k, v1, v2 = (_rand(rng, 11, 3) for _ in range(4))
    O1, _ = oracle.forward_head(q, k, v1, 0.9)
    O2, _ = oracle.forward_head(q, k, v2, 0.9)
    O3, _ = oracle.forward_head(q, k, 2.0 * v1 - 3.0 * v2, 0.9)
    np.testing.assert_allclose(O3, 2.0 * O1 - 3.0 * O2, atol=1e-13)


def test_shift_of_every_key_shifts_only_lse():
    """Adding u to every key adds scale*q.u to every score of row q: the
    softmax is unchanged and L moves by exactly that amount."""
    rng = np.random.default_rng(9)
    q, k, v = (_rand(rng, 13, 4) for _ in range(3))
    u = _rand(rng, 4)
    O1, L1 = oracle.forward_head(q, k, v, 0.6, causal=True)
    O2, L2 = oracle.forward_head(q, k + u, v, 0.6, causal=True)
    np.testing.assert_allclose(O2, O1, atol=1e-13)
    np.testing.assert_allclose(L2 - L1, 0.6 * (q @ u), atol=1e-13)


def test_lse_direct_sum_for_small_scores():
    rng = np.random.default_rng(10)
    q, k, v = (_rand(rng, 7, 3) * 0.3 for _ in range(3))
    _, L = oracle.forward_head(q, k, v, 1.0)
    direct = np.array([math.log(math.fsum(math.exp(float(q[i] @ k[j]))
                                           for j in range(7)))
                       for i in range(7)])
    np.testing.assert_allclose(L, direct, atol=1e-14)


def test_zero_queries_give_uniform_attention():
    rng = np.random.default_rng(13)
    k, v = _rand(rng, 9, 4), _rand(rng, 9, 4)
    O, L = oracle.forward_head(np.zeros((9, 4)), k, v, 0.5, causal=True)
    for i in range(9):
        np.testing.assert_allclose(O[i], v[: i + 1].mean(0), atol=1e-14)
        assert abs(L[i] - math.log(i + 1)) < 1e-14


# --------------------------------------------------------------- masks

def test_block_mask_rows_are_query_blocks():
    """Query block 0 keeps only key block 2: its rows average V[4:6] when all
    keys are identical (a transposed mask would give a different set)."""
    rng = np.random.default_rng(14)
    N, d, mb = 8, 3, 2
    q, v = _rand(rng, N, d), _rand(rng, N, d)
    k = np.tile(_rand(rng, 1, d), (N, 1))
    bm = np.eye(4, dtype=np.uint8)
    bm[0] = [0, 0, 1, 0]
    O, _ = oracle.forward_head(q, k, v, 1.0, False, bm, mb)
    np.testing.assert_allclose(O[0], v[4:6].mean(0), atol=1e-14)
    np.testing.assert_allclose(O[1], v[4:6].mean(0), atol=1e-14)
    np.testing.assert_allclose(O[4], v[4:6].mean(0), atol=1e-14)
    np.testing.assert_allclose(O[2], v[2:4].mean(0), atol=1e-14)


def test_all_ones_block_mask_equals_dense():
    rng = np.random.default_rng(15)
    q, k, v = (_rand(rng, 20, 4) for _ in range(3))
    O1, L1 = oracle.forward_head(q, k, v, 0.5)
    O2, L2 = oracle.forward_head(q, k, v, 0.5, False,
                                 np.ones((3, 3), np.uint8), 8)
    np.testing.assert_array_equal(O1, O2)
    np.testing.assert_array_equal(L1, L2)


@pytest.mark.parametrize("case", ["causal", "mask"])
def test_masked_positions_do_not_matter(case):
    rng = np.random.default_rng(16)
    N, d, mb = 16, 4, 4
    q, k, v, do = (_rand(rng, N, d) for _ in range(4))
    if case == "causal":
        bm, causal = None, True
    else:
        bm, causal = np.array([[1, 0, 0, 1], [0, 1, 0, 0], [1, 1, 1, 0],
                               [0, 0, 0, 1]], np.uint8), False
    # rows 0..3 under causal never see keys 4.., under the mask never key block 1,2
    O1, L1 = oracle.forward_head(q, k, v, 0.5, causal, bm, mb)
    k2, v2 = k.copy(), v.copy()
    k2[4:8] += 100.0
    v2[4:8] -= 50.0
    O2, L2 = oracle.forward_head(q, k2, v2, 0.5, causal, bm, mb)
    np.testing.assert_array_equal(O1[:4], O2[:4])
    np.testing.assert_array_equal(L1[:4], L2[:4])
    dQ1, _, _, _ = oracle.backward_head(q, k, v, do, 0.5, causal, bm, mb)
    dQ2, _, _, _ = oracle.backward_head(q, k2, v2, do, 0.5, causal, bm, mb)
    np.testing.assert_allclose(dQ1[:4], dQ2[:4], atol=1e-13)


def test_fully_masked_row_reading():
    rng = np.random.default_rng(17)
    N, d, mb = 8, 3, 2
    q, k, v, do = (_rand(rng, N, d) for _ in range(4))
    bm = np.ones((4, 4), np.uint8)
    bm[1] = 0  # query rows 2 and 3 see no key
    O, L = oracle.forward_head(q, k, v, 1.0, False, bm, mb)
    np.testing.assert_array_equal(O[2:4], 0.0)
    assert np.all(L[2:4] == -np.inf)
    dQ, dK, dV, _ = oracle.backward_head(q, k, v, do, 1.0, False, bm, mb)
    np.testing.assert_array_equal(dQ[2:4], 0.0)
    # dK / dV must not depend on dO of the empty rows
    do2 = do.copy()
    do2[2:4] += 7.0
    _, dK2, dV2, _ = oracle.backward_head(q, k, v, do2, 1.0, False, bm, mb)
    np.testing.assert_allclose(dK2, dK, atol=1e-13)
    np.testing.assert_allclose(dV2, dV, atol=1e-13)


# ------------------------------------------------------------- gradients

def _loss(q, k, v, do, scale, causal, bm, mb):
    O, _ = oracle.forward_head(q, k, v, scale, causal, bm, mb)
    return float((O * do).sum())


@pytest.mark.parametrize("case", ["dense", "causal", "mask"])
def test_gradients_by_central_differences(case):
    rng = np.random.default_rng(30)
    N, d, mb = 8, 4, 2
    q, k, v, do = (_rand(rng, N, d) for _ in range(4))
    causal = case == "causal"
    bm = None
    if case == "mask":
        bm = np.array([[1, 0, 1, 0], [1, 1, 0, 0], [0, 1, 1, 1],
                       [1, 0, 0, 1]], np.uint8)
    scale = 0.5
    dQ, dK, dV, _ = oracle.backward_head(q, k, v, do, scale, causal, bm, mb)
    h = 1e-6
    for name, X, G in (("q", q, dQ), ("k", k, dK), ("v", v, dV)):
        num = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += h
            Xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = Xp
            fp = _loss(args["q"], args["k"], args["v"], do, scale, causal, bm, mb)
            args[name] = Xm
            fm = _loss(args["q"], args["k"], args["v"], do, scale, causal, bm, mb)
            num[idx] = (fp - fm) / (2 * h)
        rel = np.abs(num - G).max() / np.abs(G).max()
        assert rel <= 1e-6, (name, rel)


def test_delta_identity():
    """rowsum(dO * O) = rowsum(P * dP): the closed form equals the
    definition's row term."""
    rng = np.random.default_rng(31)
    N, d = 50, 7
    q, k, v, do = (_rand(rng, N, d) for _ in range(4))
    for causal in (False, True):
        O, _ = oracle.forward_head(q, k, v, 0.4, causal)
        _, _, _, D = oracle.backward_head(q, k, v, do, 0.4, causal)
        Dc = oracle.delta_closed_form(O, do)
        np.testing.assert_allclose(Dc, D, rtol=1e-12, atol=1e-13)


# ------------------------------------------------------ batched wrappers

def test_batched_wrappers_cover_every_head_and_chunking_is_neutral():
    rng = np.random.default_rng(32)
    B, H, N, d = 2, 3, 20, 4
    q, k, v, do = (_rand(rng, B, H, N, d) for _ in range(4))
    O, L = oracle.forward(q, k, v, 0.5, causal=True)
    Oc, Lc = oracle.forward(q, k, v, 0.5, causal=True, row_chunk=7)
    np.testing.assert_array_equal(O, Oc)
    np.testing.assert_array_equal(L, Lc)
    dQ, dK, dV = oracle.backward(q, k, v, do, 0.5, causal=True)
    for b in range(B):
        for h in range(H):
            o1, l1 = oracle.forward_head(q[b, h], k[b, h], v[b, h], 0.5, True)
            np.testing.assert_array_equal(O[b, h], o1)
            g = oracle.backward_head(q[b, h], k[b, h], v[b, h], do[b, h], 0.5,
                                     True)
            np.testing.assert_array_equal(dQ[b, h], g[0])
            np.testing.assert_array_equal(dK[b, h], g[1])
            np.testing.assert_array_equal(dV[b, h], g[2])
    # heads= computes only the listed heads
    Os, _ = oracle.forward(q, k, v, 0.5, causal=True, heads=[(1, 2)])
    np.testing.assert_array_equal(Os[1, 2], O[1, 2])
    assert np.isnan(Os[0, 0]).all()


# ------------------------------------------- decoding shape and split-KV merge

def test_causal_offset_keeps_the_last_positions():
    # Fewer queries than keys: query i is key position i + (Nk - Nq), so it
    # sees exactly the first i + Nk - Nq + 1 keys, and the last query sees all.
    rng = np.random.default_rng(41)
    nq, nk, d = 4, 11, 3
    q, k, v = _rand(rng, nq, d), _rand(rng, nk, d), _rand(rng, nk, d)
    off = nk - nq
    keep = A.keep_matrix(nq, nk, causal=True, causal_offset=off)
    assert [int(r.sum()) for r in keep] == [off + 1 + i for i in range(nq)]
    O, L = oracle.forward_head(q, k, v, 0.9, causal=True, causal_offset=off)
    for i in range(nq):
        n = i + off + 1
        Oi, Li = oracle.forward_head(q[i:i + 1], k[:n], v[:n], 0.9)
        np.testing.assert_allclose(O[i], Oi[0], rtol=0, atol=1e-14)
        assert abs(L[i] - Li[0]) < 1e-14
    # offset 0 with equal lengths is the ordinary causal rule
    O0, L0 = oracle.forward_head(k, k, v, 0.9, causal=True, causal_offset=0)
    O1, L1 = oracle.forward_head(k, k, v, 0.9, causal=True)
    np.testing.assert_array_equal(O0, O1)
    np.testing.assert_array_equal(L0, L1)


def test_worked_example_split_merge(worked):
    # The worked example's four keys in two runs: each run's logsumexp and
    # normalised output in closed form, and their merge is the two-pass
    # result of the whole row.
    q, k, v = (np.array(worked[x]) for x in ("q", "k", "v"))
    O, L, parts = oracle.split_forward_head(q, k, v, worked["scale"],
                                            [0, 2, 4])
    s = [float(q[0, 0] * k[j, 0]) for j in range(4)]
    vv = [float(v[j, 0]) for j in range(4)]
    for (O_s, L_s), (a, b) in zip(parts, [(0, 2), (2, 4)]):
        den = sum(math.exp(s[j]) for j in range(a, b))
        assert abs(L_s[0] - math.log(den)) < 1e-12
        num = sum(vv[j] * math.exp(s[j]) for j in range(a, b))
        assert abs(O_s[0, 0] - num / den) < 1e-12
    assert abs(O[0, 0] - worked["two_pass"]["O"]) < 1e-12
    assert abs(L[0] - worked["two_pass"]["L"]) < 1e-12


@pytest.mark.parametrize("bounds_kind", ["halves", "ones", "ragged", "single"])
@pytest.mark.parametrize("causal", [False, True])
def test_split_merge_equals_definition(bounds_kind, causal):
    rng = np.random.default_rng(57)
    nq, nk, d = 6, 37, 4
    q, k, v = _rand(rng, nq, d), 2.0 * _rand(rng, nk, d), _rand(rng, nk, d)
    off = nk - nq
    bounds = {"halves": [0, 19, 37], "ones": list(range(nk + 1)),
              "ragged": [0, 5, 6, 20, 33, 37], "single": [0, 37]}[bounds_kind]
    O, L, parts = oracle.split_forward_head(q, k, v, 0.6, bounds, causal,
                                            causal_offset=off)
    Od, Ld = oracle.forward_head(q, k, v, 0.6, causal, causal_offset=off)
    np.testing.assert_allclose(O, Od, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, Ld, rtol=0, atol=1e-12)
    if causal and bounds_kind == "ones":
        # runs past a row's last key are empty for it and weigh zero
        assert np.isneginf(parts[-1][1][0]) and not np.any(parts[-1][0][0])
