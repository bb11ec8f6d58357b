"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs, element by element.

Every case is checked on every head and every row, forward and backward:
small cases span several tiles and a ragged tail; the five full-size
workloads run exactly as the benchmark launches them.  Outputs start as NaN,
so an element the library leaves unwritten fails the comparison.
"""
import numpy as np
import pytest
import torch

import workloads as W
from tests import _parity as P

pytestmark = pytest.mark.gpu


def all_heads(w):
    return [(b, h) for b in range(w.B) for h in range(w.H)]


SMALL = [
    # name, B, H, N, D, dtype, causal, mask_block, band, frac, k_scale
    ("bf16_d64_dense_ragged", 1, 3, 300, 64, "bf16", False, 0, 0, 0.0, 1.0),
    ("bf16_d64_causal_ragged", 2, 2, 333, 64, "bf16", True, 0, 0, 0.0, 1.0),
    ("bf16_d128_dense_ragged", 1, 3, 200, 128, "bf16", False, 0, 0, 0.0, 1.0),
    ("bf16_d128_causal_ragged", 2, 2, 333, 128, "bf16", True, 0, 0, 0.0, 3.0),
    ("bf16_d64_mask", 1, 2, 640, 64, "bf16", False, 128, 0, 0.4, 1.0),
    ("bf16_d128_mask_ragged", 1, 2, 700, 128, "bf16", False, 256, 0, 0.5, 1.0),
    ("bf16_d128_mask_causal", 2, 1, 512, 128, "bf16", True, 128, 1, 0.3, 1.0),
    ("bf16_d128_mask_causal_ragged", 1, 3, 333, 128, "bf16", True, 128, 1, 0.5, 1.0),
    ("bf16_d64_mask256_causal_ragged", 2, 2, 700, 64, "bf16", True, 256, 0, 0.5, 1.0),
    # (Non-causal masks deal row and column blocks heaviest first; mask
    # blocks of two and three 128-row blocks with a short last one.)
    ("bf16_d64_mask256_short_last", 2, 4, 600, 64, "bf16", False, 256, 0, 0.5, 1.0),
    ("bf16_d128_mask384_short_last", 1, 8, 1000, 128, "bf16", False, 384, 1, 0.3, 1.0),
    ("bf16_d64_tiny", 1, 1, 17, 64, "bf16", True, 0, 0, 0.0, 1.0),
    ("bf16_d128_one_row", 1, 2, 1, 128, "bf16", False, 0, 0, 0.0, 1.0),
    ("fp32_d64_dense_ragged", 1, 2, 100, 64, "fp32", False, 0, 0, 0.0, 1.0),
    ("fp32_d128_causal_ragged", 1, 2, 150, 128, "fp32", True, 0, 0, 0.0, 1.0),
    ("fp32_d64_mask", 1, 1, 384, 64, "fp32", False, 128, 0, 0.5, 1.0),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_case_every_head(case):
    name, B, H, N, D, dtype, causal, mb, band, frac, ks = case
    w = W.small_case(name, B, H, N, D, dtype, causal, seed=1000 + len(name),
                     k_scale=ks, mask_block=mb, mask_band=band, mask_frac=frac)
    inp = W.make_inputs(w)
    out = P.run_gpu(w, inp)
    P.check_forward(w, inp, out, all_heads(w))
    P.check_backward(w, inp, out, all_heads(w))


def _window_mask(nmb: int, seed: int) -> np.ndarray:
    """A block mask whose kept blocks sit on both sides of the 64-block
    windows the kernels scan the mask in: rows (and columns) whose only
    kept block is past block 64, runs of dropped blocks across the window
    edge, an empty row and an empty column, a full row, and the rest random
    at 20%."""
    rng = np.random.default_rng(seed)
    m = (rng.random((nmb, nmb)) < 0.2).astype(np.uint8)
    m[0] = 0
    m[0, nmb - 1] = 1             # only the last block
    m[1] = 0
    m[1, [0, 64]] = 1             # first block of each window
    m[2] = 0                      # nothing kept: O = 0, L = -inf
    m[3] = 1                      # everything kept
    m[4] = 0
    m[4, [63, 65]] = 1            # around the window edge
    m[:, 5] = 0                   # a key block no query sees: dK = dV = 0
    m[:, nmb - 2] = 0
    m[nmb - 1, nmb - 2] = 1       # a key block only the last rows see
    return m


@pytest.mark.parametrize("D,causal,H", [(64, False, 2), (128, True, 1)])
def test_block_mask_past_64_blocks(D, causal, H):
    """More mask blocks per row than one 64-block scan window (N = 70 blocks
    of 128), with kept blocks placed to force window refills in the forward
    and dQ row scans and the dK/dV column scans; every head against the
    oracle."""
    nmb = 70
    w = W.small_case(f"mask_windows_d{D}", 1, H, 128 * nmb, D, "bf16", causal,
                     seed=77 + D, mask_block=128, mask_band=0, mask_frac=0.2)
    inp = W.make_inputs(w)
    inp["block_mask"] = _window_mask(nmb, seed=5 + D)
    out = P.run_gpu(w, inp)
    P.check_forward(w, inp, out, all_heads(w))
    P.check_backward(w, inp, out, all_heads(w))


def test_c1_fp32_full():
    w = W.get("c1")
    inp = W.make_inputs(w)
    out = P.run_gpu(w, inp)
    P.check_forward(w, inp, out, all_heads(w))
    P.check_backward(w, inp, out, all_heads(w))


def test_c2_bf16_dense_every_head():
    w = W.get("c2")
    inp = W.make_inputs(w)
    out = P.run_gpu(w, inp)
    P.check_forward(w, inp, out, all_heads(w))
    P.check_backward(w, inp, out, all_heads(w))


def test_c3_headline_every_head():
    w = W.get("c3")
    inp = W.make_inputs(w)
    out = P.run_gpu(w, inp)
    P.check_forward(w, inp, out, all_heads(w))
    P.check_backward(w, inp, out, all_heads(w))


def test_c4_long_forward_every_row():
    w = W.get("c4f")
    inp = W.make_inputs(w)
    out = P.run_gpu(w, inp, backward=False)
    P.check_forward(w, inp, out, all_heads(w))


def test_c4_backward_n8192_every_head():
    w = W.get("c4b")
    inp = W.make_inputs(w)
    out = P.run_gpu(w, inp)
    P.check_forward(w, inp, out, all_heads(w))
    P.check_backward(w, inp, out, all_heads(w))


def test_c5_block_sparse_every_head():
    w = W.get("c5")
    inp = W.make_inputs(w)
    assert int(inp["block_mask"].sum()) == 1166
    out = P.run_gpu(w, inp)
    P.check_forward(w, inp, out, all_heads(w))
    P.check_backward(w, inp, out, all_heads(w))


# The softmax scale is an argument of the boundary: cases at scales other
# than 1/sqrt(d), so that a kernel using 1/sqrt(d) in place of the argument
# (in the scores, the exponentials, L, or dQ and dK) fails.  Scale 1 makes
# the rows sharp (logits of standard deviation sqrt(d), nearly one-hot
# softmax rows), so the row maximum jumps by far more than the lazily moved
# reference allows and the rescale path runs on most tiles.
SCALES = [0.3, 0.05, 1.0]
SCALE_CASES = [
    # name, B, H, N, D, dtype, causal, mask_block, band, frac
    ("d64_dense", 1, 2, 300, 64, "bf16", False, 0, 0, 0.0),
    ("d64_causal", 1, 2, 333, 64, "bf16", True, 0, 0, 0.0),
    ("d64_mask", 1, 2, 640, 64, "bf16", False, 128, 0, 0.4),
    ("d128_dense", 2, 1, 200, 128, "bf16", False, 0, 0, 0.0),
    ("d128_causal", 1, 2, 333, 128, "bf16", True, 0, 0, 0.0),
    ("d128_mask_causal", 1, 2, 700, 128, "bf16", True, 256, 0, 0.5),
    ("f32_d64_dense", 1, 2, 130, 64, "fp32", False, 0, 0, 0.0),
    ("f32_d64_mask", 1, 1, 384, 64, "fp32", False, 128, 0, 0.5),
    ("f32_d128_causal", 1, 2, 150, 128, "fp32", True, 0, 0, 0.0),
]


@pytest.mark.parametrize("scale", SCALES, ids=[f"s{s}" for s in SCALES])
@pytest.mark.parametrize("case", SCALE_CASES, ids=[c[0] for c in SCALE_CASES])
def test_non_default_scale(case, scale):
    name, B, H, N, D, dtype, causal, mb, band, frac = case
    w = W.small_case(f"scale_{name}_{scale}", B, H, N, D, dtype, causal,
                     seed=7000 + len(name) + int(1000 * scale), mask_block=mb,
                     mask_band=band, mask_frac=frac, scale=scale)
    assert abs(w.scale - 1.0 / np.sqrt(D)) > 1e-3
    inp = W.make_inputs(w)
    out = P.run_gpu(w, inp)
    P.check_forward(w, inp, out, all_heads(w))
    # At scale 1 the gradients are about scale * sqrt(d) times larger than
    # at the workloads' unit scale; fp32 keeps the bound relative to them.
    P.check_backward(w, inp, out, all_heads(w),
                     f32_relative=scale * np.sqrt(D) > 2.0)


# Sequence lengths on both sides of every tile boundary the kernels use
# (32-row MFMA blocks, 64/128-key tiles, 128-query forward blocks, 128-key
# backward blocks, 256-row mask blocks), for both head sizes, dense and
# causal; one head of each against the oracle, forward and backward.
SWEEP_N = [1, 2, 31, 33, 63, 65, 127, 129, 191, 255, 257, 383, 513]


@pytest.mark.parametrize("causal", [False, True], ids=["dense", "causal"])
@pytest.mark.parametrize("D", [64, 128])
def test_tile_boundary_sweep(D, causal):
    for i, n in enumerate(SWEEP_N):
        w = W.small_case(f"sweep_{D}_{int(causal)}_{n}", 1, 2, n, D, "bf16",
                         causal, seed=5000 + 7 * i + D + int(causal))
        inp = W.make_inputs(w)
        out = P.run_gpu(w, inp)
        P.check_forward(w, inp, out, [(0, 1)])
        P.check_backward(w, inp, out, [(0, 1)])
