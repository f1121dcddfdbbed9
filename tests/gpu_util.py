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
