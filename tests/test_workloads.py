"""Input generator, rounding and counting checks (CPU only)."""
import math
import os

import numpy as np
import pytest
import torch

import workloads as W
from workloads import cost


def test_block_mask_counts_for_the_block_sparse_workload():
    w = W.get("c5")
    inp = W.make_inputs(W.small_case("c5mask", 1, 1, w.N, 1, "bf16", False,
                                     w.seed, mask_block=128, mask_band=1,
                                     mask_frac=0.25))
    bm = inp["block_mask"]
    assert bm.shape == (64, 64) and bm.dtype == np.uint8
    i, j = np.indices(bm.shape)
    band = np.abs(i - j) <= 1
    assert band.sum() == 190
    assert np.all(bm[band] == 1)
    off = (~band).sum()
    assert off == 3906
    assert bm[~band].sum() == math.floor(0.25 * 3906) == 976
    assert bm.sum() == 1166
    again = W.make_inputs(W.small_case("c5mask", 1, 1, w.N, 1, "bf16", False,
                                       w.seed, mask_block=128, mask_band=1,
                                       mask_frac=0.25))["block_mask"]
    np.testing.assert_array_equal(bm, again)


def test_mask_is_drawn_after_the_tensors():
    """The mask depends only on the seed and on the tensors drawn before it."""
    a = W.band_random_block_mask(16, 1, 0.25, np.random.default_rng(1))
    b = W.band_random_block_mask(16, 1, 0.25, np.random.default_rng(2))
    assert a.sum() == b.sum() == 46 + math.floor(0.25 * (256 - 46))
    assert not np.array_equal(a, b)


def test_bf16_rounding_ties_to_even():
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8),
                  1.0 + 2 ** -8 + 2 ** -20, 3.0, 0.0])
    r = W.round_bf16(x)
    np.testing.assert_array_equal(
        r, [1.0, 1.0 + 2 ** -6, -1.0, 1.0 + 2 ** -7, 3.0, 0.0])


def test_bf16_rounding_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * 10).astype(np.float32)
    ours = W.round_bf16(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(ours, ref)
    t = W.to_torch(ours, "bf16")
    assert t.dtype == torch.bfloat16
    np.testing.assert_array_equal(t.to(torch.float64).numpy(), ours)


def test_inputs_are_on_the_grid_and_seeded():
    w = W.small_case("t", 2, 3, 40, 16, "bf16", True, 3, k_scale=3.0)
    a = W.make_inputs(w)
    b = W.make_inputs(w)
    for key in ("q", "k", "v", "do"):
        assert a[key].shape == (2, 3, 40, 16)
        np.testing.assert_array_equal(a[key], b[key])
        np.testing.assert_array_equal(W.round_bf16(a[key]), a[key])
    assert 2.0 < a["k"].std() < 4.0 and 0.6 < a["q"].std() < 1.4
    f = W.make_inputs(W.small_case("f", 1, 1, 30, 8, "fp32", False, 1))
    np.testing.assert_array_equal(f["q"].astype(np.float32).astype(np.float64),
                                  f["q"])


def test_workload_table():
    assert W.get("c3").shape == (2, 32, 4096, 128) and W.get("c3").causal
    assert W.get("c1").dtype == "fp32"
    assert W.get("c4f").N == 16384 and not W.get("c4f").backward
    assert W.get("c4b").N == 8192 and W.get("c4b").k_scale == 3.0
    assert W.get("c5").mask_block == 128


def test_counted_work_of_the_headline_workload():
    w = W.get("c3")
    f = cost.fwd_flops(w.B, w.H, w.N, w.D, causal=True)
    b = cost.bwd_flops(w.B, w.H, w.N, w.D, causal=True)
    assert f == 2 * 32 * 2 * 4096 ** 2 * 128
    assert round(f / 1e9, 2) == 274.88
    assert round(b / 1e9, 2) == 687.19
    assert round((f + b) / 1e9, 2) == 962.07
    assert round(cost.fwd_bytes(w.B, w.H, w.N, w.D, "bf16") / 1e6, 1) == 269.5


def test_block_sparse_work_counts_kept_blocks():
    bm = np.zeros((4, 4), np.uint8)
    bm[0, 0] = bm[1, 2] = bm[3, 3] = 1
    assert cost.fwd_flops(1, 1, 512, 64, block_mask=bm) == 4 * 512 ** 2 * 64 * 3 / 16


def test_four_k_token_traffic_arithmetic():
    """N = 4096, d = 128, bf16: each of Q, K, V is 1 MiB; S and P are 32 MiB
    each; writing and re-reading both is at least 128 MiB per head and 4 GiB
    for 32 heads ("Why is FlashAttention faster?", "The 4K-token traffic
    FlashAttention avoids")."""
    N, d = 4096, 128
    assert N * d * cost.ELT["bf16"] == 2 ** 20
    assert N * N * cost.ELT["bf16"] == 32 * 2 ** 20
    assert cost.naive_intermediate_bytes(N, "bf16") == 128 * 2 ** 20
    assert 32 * cost.naive_intermediate_bytes(N, "bf16") == 4 * 2 ** 30


def test_padding_workload_recipe():
    """The key-padding workload has the shape of the pages' experiment
    (batch 64, 16 heads, N = 1024, d = 64) and seeded valid-key counts on
    [N/4, N], the same on every call."""
    w = W.padding_workload()
    assert (w.B, w.H, w.N, w.D, w.dtype, w.causal) == (64, 16, 1024, 64,
                                                        "bf16", False)
    a, b = W.padding_lengths(w.B, w.N), W.padding_lengths(w.B, w.N)
    assert a == b and len(a) == w.B
    assert min(a) >= w.N // 4 and max(a) <= w.N
    assert len(set(a)) > w.B // 2          # a mix, not a constant


@pytest.mark.parametrize("name,enters", [("probe_mfma.hip", False),
                                         ("fa_api.hip", True)])
def test_traffic_digest_covers_the_library_only(monkeypatch, name, enters):
    """The HBM-traffic record is keyed by a digest of the attention
    library's sources: a change to one of them changes the digest, a change
    to the probe library's does not."""
    import io
    import bench
    from io_aware_exact_04_amd import build as B
    d0 = bench.source_digest()
    target = os.path.abspath(os.path.join(os.path.dirname(B.__file__),
                                          "csrc", name))
    real_open = open

    def fake_open(path, *args, **kw):
        if os.path.abspath(str(path)) == target:
            return io.BytesIO(b"changed")
        return real_open(path, *args, **kw)
    monkeypatch.setattr("builtins.open", fake_open)
    assert (bench.source_digest() != d0) == enters
