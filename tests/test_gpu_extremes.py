"""GPU parity of the Frobenius normalisation at the ends of the float32 range.

The library sums ||U||_F in float64 and, when the norm lies outside the band
where the unscaled Gram is exact in float32, stores X0 = U * 2^e (exact) and
folds 2^-e / (||U||_F + eps) into the first step. These cases compare it with
the float64 oracle, which is scale-invariant by construction:

* U scaled by 1e-25 with eps = 0: O equals the unscaled result;
* U scaled by 1e-25 with the default eps = 1e-7: ||U||_F << eps, so X0 is tiny
  and O stays in the linear regime (the product of the a_k times X0);
* U scaled by 1e18: sums of squares beyond the float32 range;
* U = 0 with eps = 0 (reading: the zero input gives O = 0).

Tolerances: float32 path 1e-4, bf16 path 2e-2 (relative Frobenius error), the
reported norm 1e-5.
"""

import numpy as np
import pytest
import torch

from gpu_util import make_matrix_inputs, need_gpu, to_np
from oracle import muon_oracle as O
from workloads import as_dtype, host_normal

pytestmark = pytest.mark.gpu

F32_TOL = 1e-4
BF16_TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    import newton_schulz_orthogonalized_amd as nso  # noqa: F401  (fails loudly without the library)
    yield


def nso():
    import newton_schulz_orthogonalized_amd as m
    return m


CASES = [(1e-25, 0.0), (1e-25, 1e-7), (1e18, 1e-7), (1e18, 0.0), (1e-33, 0.0)]
SHAPES = [(300, 520), (520, 300), (768, 2304), (1024, 2048)]   # the last takes Gram-side steps in bf16


@pytest.mark.parametrize("scale,eps", CASES)
@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("prec", ["f32", "bf16"])
def test_orthogonalize_at_extreme_magnitudes(scale, eps, shape, prec):
    print(f"[extremes orthogonalize] scale={scale:g} eps={eps:g} shape={shape} prec={prec}", flush=True)
    dtype = torch.float32 if prec == "f32" else torch.bfloat16
    x = as_dtype(host_normal(shape, 31000) * scale, dtype)
    norm = torch.zeros(1, device="cuda")
    out, = nso().orthogonalize([x.cuda()], precision=prec, norm_eps=eps, norm_outs=[norm])
    torch.cuda.synchronize()
    ref, nref = O.orthogonalize_ref(to_np(x), eps=float(np.float32(eps)))
    o = to_np(out)
    assert np.all(np.isfinite(o))
    assert O.rel_fro(o, ref) <= (F32_TOL if prec == "f32" else BF16_TOL)
    assert abs(norm.item() - nref[0]) <= 1e-5 * nref[0]


@pytest.mark.parametrize("scale,eps", CASES)
@pytest.mark.parametrize("prec", ["f32", "bf16"])
def test_muon_step_at_extreme_magnitudes(scale, eps, prec):
    """The full step, with grad and momentum both scaled: the momentum, O and
    the update against the oracle, a tall and a wide matrix in one call."""
    print(f"[extremes step] scale={scale:g} eps={eps:g} prec={prec}", flush=True)
    dtype = torch.float32 if prec == "f32" else torch.bfloat16
    shapes = [(384, 1000), (1000, 384)]
    ws, gs, ms, host, oo = [], [], [], [], []
    for i, sh in enumerate(shapes):
        w = as_dtype(host_normal(sh, 31100 + 3 * i, 0.02), dtype).cuda()
        g = as_dtype(host_normal(sh, 31101 + 3 * i) * scale, dtype).cuda()
        m = as_dtype(host_normal(sh, 31102 + 3 * i) * scale, torch.float32).cuda()
        host.append((to_np(w), to_np(g), to_np(m)))
        ws.append(w); gs.append(g); ms.append(m)
        oo.append(torch.zeros(sh, dtype=torch.float32, device="cuda"))
    nso().muon_step(ws, gs, ms, lr=0.02, weight_decay=0.01, precision=prec, norm_eps=eps, ortho_outs=oo)
    torch.cuda.synchronize()
    tol = F32_TOL if prec == "f32" else BF16_TOL
    for i, sh in enumerate(shapes):
        w0, g0, m0 = host[i]
        ref = O.muon_step_ref(w0, g0, m0, lr=float(np.float32(0.02)), weight_decay=float(np.float32(0.01)),
                              eps=float(np.float32(eps)))
        assert O.rel_fro(to_np(ms[i]), ref["m"]) <= 1e-6, sh
        assert O.rel_fro(to_np(oo[i]), ref["o"]) <= tol, sh
        # W against the oracle's W: float32 rounding of the stored weight plus
        # lr times the difference of the two directions (a relative check of
        # W - W0 would be meaningless here: with O near 1e-18 the step is pure
        # decay, 2e-4 W, of the size of W's own float32 rounding)
        # (float32 arithmetic: two roundings of values as large as |W0| and
        # lr |O|; bf16: one more rounding, half an ulp of the result)
        w1, o = to_np(ws[i]), to_np(oo[i])
        dir_diff = 0.02 * np.abs(o - ref["o"])
        bound = dir_diff + 2.0 ** -21 * (np.abs(w0) + 0.02 * np.abs(o))
        if prec == "bf16":
            bound += 2.0 ** -8 * (np.abs(ref["w"]) + dir_diff)
        assert np.all(np.abs(w1 - ref["w"]) <= bound + 1e-30), sh


@pytest.mark.parametrize("prec", ["f32", "bf16"])
def test_zero_input_with_zero_eps(prec):
    dtype = torch.float32 if prec == "f32" else torch.bfloat16
    x = torch.zeros((200, 330), dtype=dtype, device="cuda")
    norm = torch.full((1,), 7.0, device="cuda")
    out, = nso().orthogonalize([x], precision=prec, norm_eps=0.0, norm_outs=[norm])
    torch.cuda.synchronize()
    assert torch.all(out == 0) and norm.item() == 0.0
    # the step: pure decay of the weight, for zero steps too
    for steps in (5, 0):
        w, g, m = make_matrix_inputs((256, 384), 31200, dtype, 0.0, 0.02, 0.0)
        w0 = to_np(w)
        oo = torch.full(w.shape, 3.0, dtype=torch.float32, device="cuda")
        nso().muon_step([w], [g], [m], lr=0.1, weight_decay=0.5, precision=prec, norm_eps=0.0, ns_steps=steps,
                        coeffs=None if steps else [], ortho_outs=[oo])
        torch.cuda.synchronize()
        assert torch.all(oo == 0), steps
        want = w0 - np.float32(0.1) * np.float32(0.5) * w0
        assert np.allclose(to_np(w), want, rtol=2.0 ** -7 if prec == "bf16" else 1e-6, atol=0), steps


@pytest.mark.parametrize("prec", ["f32", "bf16"])
def test_zero_steps_at_extreme_magnitudes(prec):
    """ns_steps = 0 applies O = X0 itself, read from the transposed copy for a
    tall block on the float32 path: both copies carry the rescale."""
    dtype = torch.float32 if prec == "f32" else torch.bfloat16
    for shape in [(64, 200), (200, 64)]:
        for scale in (1e-30, 1e20):
            x = as_dtype(host_normal(shape, 31300) * scale, dtype)
            out, = nso().orthogonalize([x.cuda()], precision=prec, norm_eps=0.0, ns_steps=0, coeffs=[])
            torch.cuda.synchronize()
            ref, _ = O.orthogonalize_ref(to_np(x), coeffs=[], eps=0.0)
            assert O.rel_fro(to_np(out), ref) <= (F32_TOL if prec == "f32" else 4e-3), (shape, scale)


def test_rescale_touches_only_its_problems():
    """A list mixing a tiny matrix, a huge one, a per-head matrix with one
    tiny head and ordinary matrices: every block against the oracle, and the
    ordinary ones bit for bit the same as in a call without the others."""
    specs = [((512, 768), 1e-28, 1), ((768, 512), 1.0, 1), ((256, 1024), 1e20, 1), ((640, 384), 1.0, 1)]
    xs = [as_dtype(host_normal(sh, 31400 + i) * sc, torch.bfloat16) for i, (sh, sc, _) in enumerate(specs)]
    # a per-head matrix whose second head is tiny
    ph = host_normal((512, 640), 31410)
    ph[128:256] *= 1e-27
    xs.append(as_dtype(ph, torch.bfloat16))
    heads = [1, 1, 1, 1, 4]
    outs = nso().orthogonalize([x.cuda() for x in xs], heads=heads, precision="bf16", norm_eps=0.0)
    torch.cuda.synchronize()
    for i, x in enumerate(xs):
        ref, _ = O.orthogonalize_ref(to_np(x), heads=heads[i], eps=0.0)
        for sl in O.head_blocks(x.shape[0], heads[i]):
            assert O.rel_fro(to_np(outs[i])[sl], ref[sl]) <= BF16_TOL, (i, sl)
    alone = nso().orthogonalize([xs[1].cuda(), xs[3].cuda()], precision="bf16", norm_eps=0.0)
    torch.cuda.synchronize()
    assert torch.equal(alone[0], outs[1]) and torch.equal(alone[1], outs[3])


def test_fused_short_blocks_at_extreme_magnitudes():
    """256 heads of 128 rows (the fused short-block path), some scaled to the
    ends of the range, with eps = 0."""
    x = host_normal((256 * 128, 512), 31500)
    for h in range(0, 256, 7):
        x[128 * h:128 * (h + 1)] *= 1e-26 if h % 2 else 1e19
    xb = as_dtype(x, torch.bfloat16)
    out, = nso().orthogonalize([xb.cuda()], heads=[256], precision="bf16", norm_eps=0.0)
    torch.cuda.synchronize()
    ref, _ = O.orthogonalize_ref(to_np(xb), heads=256, eps=0.0)
    o = to_np(out)
    for h in range(0, 256, 7):
        sl = slice(128 * h, 128 * (h + 1))
        assert O.rel_fro(o[sl], ref[sl]) <= BF16_TOL, h
    assert O.rel_fro(o, ref) <= BF16_TOL
