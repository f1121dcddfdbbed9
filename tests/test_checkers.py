"""The comparison helpers the GPU parity tests use, checked on the CPU: they
pass a result that meets the bound and catch a planted mistake."""

import numpy as np
import pytest

from gpu_util import check_w_against_oracle, tile_rel_fro
from oracle import muon_oracle as O


def test_tile_rel_fro_finds_one_bad_tile():
    rng = np.random.default_rng(1)
    ref = rng.standard_normal((700, 900))
    o = ref * (1 + 1e-3)
    assert abs(tile_rel_fro(o, ref) - 1e-3) < 1e-12
    bad = o.copy()
    bad[256:512, 512:768] *= 1.05          # one tile off by 5 %
    assert tile_rel_fro(bad, ref) > 4.9e-2
    assert O.rel_fro(bad, ref) < 2e-2       # which the whole-matrix figure hides
    edge = o.copy()
    edge[512:, 768:] = 0.0                  # the ragged corner block
    assert tile_rel_fro(edge, ref) == pytest.approx(1.0)


def _emulated_step(w0, o, lr, wd):
    """bf16 parameter as the kernel forms it: float32 arithmetic, one RNE."""
    w32 = w0.astype(np.float32)
    x = (w32 - np.float32(lr * wd) * w32) - np.float32(lr) * o.astype(np.float32)
    return O.bf16_round(x.astype(np.float64))


def test_w_check_accepts_the_kernel_form_and_catches_an_ulp_slip():
    rng = np.random.default_rng(2)
    w0 = O.bf16_round(0.02 * rng.standard_normal((300, 400)))
    ref_o = rng.standard_normal((300, 400)) / 20
    o = ref_o * (1 + 5e-3 * rng.standard_normal((300, 400)))   # a bf16-path-sized error in O
    ref_w = w0 - 0.02 * 0.01 * w0 - 0.02 * ref_o
    w1 = _emulated_step(w0, o, 0.02, 0.01)
    frac = check_w_against_oracle(w1, w0, o, ref_w, ref_o, 0.02)
    assert frac > 0.95
    # a parameter moved by two ulps somewhere is caught
    w_bad = w1.copy()
    big = np.argmax(np.abs(w0))
    w_bad.flat[big] += 2 * 2.0 ** (np.floor(np.log2(abs(w_bad.flat[big]))) - 7)
    with pytest.raises(AssertionError):
        check_w_against_oracle(w_bad, w0, o, ref_w, ref_o, 0.02)
    # a dropped weight-decay term is caught
    w_nowd = _emulated_step(w0, o, 0.02, 0.0)
    with pytest.raises(AssertionError):
        check_w_against_oracle(w_nowd, w0, o, ref_w, ref_o, 0.02)
