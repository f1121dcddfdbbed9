"""Helpers shared by the GPU tests: device inputs from the seeded generators
and comparisons against the oracle (which the tests feed the same values)."""

import numpy as np
import pytest
import torch

from workloads import as_dtype, host_normal


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def make_matrix_inputs(shape, seed, dtype, gstd=1.0, wstd=1.0, mstd=1.0):
    """(W, G, M) as device tensors; W and G in `dtype`, M float32."""
    w = as_dtype(host_normal(shape, seed, wstd), dtype).cuda()
    g = as_dtype(host_normal(shape, seed + 1, gstd), dtype).cuda()
    m = as_dtype(host_normal(shape, seed + 2, mstd), torch.float32).cuda()
    return w, g, m


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 values at |x| (2^(e-7) for |x| in [2^e, 2^(e+1)))."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def tile_rel_fro(o: np.ndarray, ref: np.ndarray, tile: int = 256) -> float:
    """Largest relative Frobenius error over the tile x tile blocks of a matrix
    (ragged edge blocks included), so that one wrong GEMM tile cannot hide
    under a whole-matrix figure."""
    r, c = ref.shape
    worst = 0.0
    for i in range(0, r, tile):
        for j in range(0, c, tile):
            d = np.linalg.norm(o[i:i + tile, j:j + tile] - ref[i:i + tile, j:j + tile])
            n = np.linalg.norm(ref[i:i + tile, j:j + tile])
            worst = max(worst, d / n if n > 0 else d)
    return worst


def check_w_against_oracle(w1: np.ndarray, w0: np.ndarray, o: np.ndarray, ref_w: np.ndarray, ref_o: np.ndarray,
                           lr: float, scale: float = 1.0, min_one_ulp: float = 0.98) -> float:
    """bf16 parameter after the step against the oracle's float64 W.

    w1 = RNE(W0 - lr wd W0 - lr scale O_gpu) in float32 arithmetic, while the
    oracle's W uses its own O, so elementwise
        |w1 - RNE(W_ref)| <= ulp(w1)/2 + ulp(W_ref)/2 + lr |scale| |O_gpu - O_ref|
                             + float32 rounding,
    which every element must meet (the two roundings, each half an ulp of its
    own result, and the difference of the two directions). Most elements are also within one bf16 ulp
    of RNE(W_ref) outright (all but weights so close to zero that lr |dO|
    exceeds their ulp); at least `min_one_ulp` of them must be. Returns that
    fraction."""
    from oracle import muon_oracle as O
    want = O.bf16_round(ref_w)
    ulp = bf16_ulp(ref_w)
    slack = 8 * 2.0 ** -24 * (np.abs(w0) + lr * abs(scale) * np.abs(o))
    d = np.abs(w1 - want)
    assert np.all(d <= 0.5 * (bf16_ulp(w1) + ulp) + lr * abs(scale) * np.abs(o - ref_o) + slack)
    frac = float(np.mean(d <= ulp))
    assert frac >= min_one_ulp, frac
    return frac
