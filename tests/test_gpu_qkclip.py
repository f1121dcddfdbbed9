"""GPU parity of QK-Clip (MuonClip Optimizer page, "QK-Clip") against the CPU oracle.

The oracle and the kernel follow the same arithmetic (gamma = tau / max_logit in
float32, float32 products, round to nearest even to the weight dtype), so the
comparison is bit for bit: bf16 weights against the bf16 rounding of the oracle's
float32 result, float32 weights against it directly.
"""

import numpy as np
import pytest
import torch

from gpu_util import need_gpu, to_np
from oracle import muon_oracle as O
from workloads import as_dtype, host_normal

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    yield


def _expect(w_ref32, dtype):
    return O.bf16_round(w_ref32).astype(np.float32) if dtype == torch.bfloat16 else w_ref32


def _run(specs, dtype, tau, seed, with_gamma=True):
    """specs: list of (q_rows, k_rows, cols, q_heads, k_heads, max_logit list)."""
    import newton_schulz_orthogonalized_amd as nso
    wqs, wks, mls, gos, ref = [], [], [], [], []
    for i, (qr, kr, cols, qh, kh, ml) in enumerate(specs):
        wq = as_dtype(host_normal((qr, cols), seed + 10 * i, 0.02), dtype).cuda()
        wk = as_dtype(host_normal((kr, cols), seed + 10 * i + 1, 0.02), dtype).cuda()
        wq0, wk0 = to_np(wq), to_np(wk)
        m = torch.tensor(np.asarray(ml, dtype=np.float32), device="cuda")
        wqs.append(wq)
        wks.append(wk)
        mls.append(m)
        gos.append(torch.full((qh,), -1.0, dtype=torch.float32, device="cuda"))
        ref.append((wq0, wk0) + O.qk_clip_ref(wq0, wk0, ml, q_heads=qh, k_heads=kh, tau=tau))
    nso.qk_clip(wqs, wks, mls, q_heads=[s[3] for s in specs], k_heads=[s[4] for s in specs], tau=tau,
                gamma_outs=gos if with_gamma else None)
    torch.cuda.synchronize()
    for i, (wq0, wk0, q, k, g) in enumerate(ref):
        np.testing.assert_array_equal(to_np(wqs[i]), _expect(q, dtype), err_msg=f"wq of pair {i}")
        np.testing.assert_array_equal(to_np(wks[i]), _expect(k, dtype), err_msg=f"wk of pair {i}")
        if with_gamma:
            np.testing.assert_array_equal(to_np(gos[i]), g, err_msg=f"gamma of pair {i}")
    return ref


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_mha_and_gqa_in_one_call(dtype):
    print(f"[qk_clip] mha+gqa dtype={dtype}", flush=True)
    rng = np.random.default_rng(3)
    specs = [
        (256, 256, 512, 4, 4, [50.0, 150.0, 100.0, 400.0]),            # MHA; one head exactly at tau
        (512, 128, 512, 8, 2, list(rng.uniform(20.0, 300.0, 8))),       # GQA, 4 query heads per key head
        (96, 96, 100, 3, 3, [250.0, 10.0, 1e6]),                         # ragged: 32 x 100 per head
        (24, 8, 37, 6, 2, [np.nan, np.inf, 90.0, 120.0, 101.0, 99.0]),  # NaN keeps, inf zeroes; odd sizes
    ]
    _run(specs, dtype, 100.0, 5000)


def test_nothing_clipped_writes_nothing():
    """All heads at or below tau: weights bitwise unchanged, gamma 1 everywhere."""
    ref = _run([(128, 32, 64, 8, 2, [10.0] * 7 + [100.0])], torch.bfloat16, 100.0, 5100)
    wq0, wk0, q, k, g = ref[0]
    assert np.all(g == 1.0)


def test_without_gamma_output():
    _run([(64, 64, 48, 2, 2, [300.0, 30.0])], torch.bfloat16, 100.0, 5200, with_gamma=False)


def test_llama_8b_attention_layers():
    """Four layers of the 8B-shaped attention weights (Wq 4096x4096 with 32
    heads, Wk 1024x4096 with 8 heads), half the query heads above tau."""
    print("[qk_clip] 8B attention layers", flush=True)
    rng = np.random.default_rng(11)
    specs = []
    for _ in range(4):
        ml = np.where(rng.random(32) < 0.5, rng.uniform(101.0, 500.0, 32), rng.uniform(1.0, 100.0, 32))
        specs.append((4096, 1024, 4096, 32, 8, list(ml)))
    _run(specs, torch.bfloat16, 100.0, 5300)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_band_tiles_tails_and_unaligned_heads(dtype):
    """Head blocks longer than one band of the tiled layout (131072 elements):
    33 x 4099 per head, so a band plus a ragged tail, and the second head of
    each matrix starts off 16-byte alignment (contiguous path); 36 x 4096 per
    head, a band plus two whole chunks, aligned."""
    print(f"[qk_clip] band tiles dtype={dtype}", flush=True)
    specs = [(66, 33, 4099, 2, 1, [150.0, 300.0]),
             (72, 36, 4096, 2, 1, [120.0, 90.0])]
    _run(specs, dtype, 100.0, 5400)
