"""Cautious weight decay on the GPU (a reading of the nanochat optimizer page,
"Muon Step Implementation", which names it without a formula): the decoupled
decay acts only where the update u = lr*scale*O has the sign of W or is zero.

The mask is a decision taken in floating point, so the update is checked with
the GPU's own O, where both sides decide W*u >= 0 on the same values, and O
itself against the oracle as everywhere else. The oracle's W (with the
oracle's O) must agree wherever the two masks agree.
"""

import numpy as np
import pytest
import torch

from gpu_util import bf16_ulp, make_matrix_inputs, need_gpu, to_np
from oracle import muon_oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    import newton_schulz_orthogonalized_amd  # noqa: F401  (fails loudly without the library)
    yield


def _run(shapes, dtype, prec, seed, lr, wd, scale, ns_steps=5, workspace=None, tensors=None):
    import newton_schulz_orthogonalized_amd as nso
    ins = tensors or [make_matrix_inputs(sh, seed + 10 * i, dtype, 1e-3, 0.02, 1e-3) for i, sh in enumerate(shapes)]
    host = [tuple(to_np(t) for t in x) for x in ins]
    oo = [torch.zeros(sh, dtype=torch.float32, device="cuda") for sh in shapes]
    nso.muon_step([x[0] for x in ins], [x[1] for x in ins], [x[2] for x in ins], lr=lr, weight_decay=wd,
                  scales=[scale] * len(shapes), precision=prec, ns_steps=ns_steps,
                  coeffs=None if ns_steps else [], ortho_outs=oo, cautious_wd=True, workspace=workspace)
    torch.cuda.synchronize()
    return ins, host, oo


def _check(w1, w0, o, ref, lr, wd, scale, bf16):
    # the update with the GPU's O, mask decided on the same values
    u = np.float32(lr) * np.float32(scale) * o
    mask = w0 * u >= 0
    want = w0 - np.float32(lr) * np.float32(wd) * w0 * mask - u
    slack = 2.0 ** -21 * (np.abs(w0) + np.abs(u))
    tol = (0.5 * bf16_ulp(want) + slack) if bf16 else slack
    assert np.all(np.abs(w1 - want) <= tol)
    # both cases occur
    assert 0.2 < mask.mean() < 0.8
    # the oracle's W wherever its mask agrees
    ref_mask = w0 * (lr * scale * ref["o"]) >= 0
    agree = ref_mask == mask
    assert agree.mean() > 0.99
    bound = abs(lr * scale) * np.abs(o - ref["o"]) + tol + 2.0 ** -22 * np.abs(w0)
    assert np.all(np.abs(w1 - ref["w"])[agree] <= bound[agree])
    # and the decay really is masked: where the update opposes W, W moved by u alone
    off = ~mask
    assert np.all(np.abs(w1[off] - (w0[off] - u[off])) <= tol[off])


@pytest.mark.parametrize("scale", [1.5, -1.0])
def test_cautious_f32(scale):
    shapes = [(128, 256), (300, 77)]
    ins, host, oo = _run(shapes, torch.float32, "f32", 42000, 0.05, 0.3, scale)
    for i, sh in enumerate(shapes):
        w0, g0, m0 = host[i]
        ref = O.muon_step_ref(w0, g0, m0, lr=0.05, weight_decay=0.3, scale=scale, cautious=True)
        o = to_np(oo[i])
        assert O.rel_fro(o, ref["o"]) <= 1e-4
        assert O.rel_fro(to_np(ins[i][2]), ref["m"]) <= 1e-6
        _check(to_np(ins[i][0]), w0, o, ref, 0.05, 0.3, scale, False)


def test_cautious_bf16_prefetched_and_edge_epilogues():
    """Wide and tall blocks whose 128 x 128 wave blocks are fully in bounds
    (the update with the parameter values loaded ahead) and ragged ones (the
    element-wise path)."""
    shapes = [(768, 2304), (2304, 768), (300, 77)]
    ins, host, oo = _run(shapes, torch.bfloat16, "bf16", 42100, 0.02, 0.5, 1.0)
    for i, sh in enumerate(shapes):
        w0, g0, m0 = host[i]
        ref = O.muon_step_ref(w0, g0, m0, lr=0.02, weight_decay=0.5, cautious=True)
        o = to_np(oo[i])
        assert O.rel_fro(o, ref["o"]) <= 2e-2, sh
        _check(to_np(ins[i][0]), w0, o, ref, 0.02, 0.5, 1.0, True)


@pytest.mark.parametrize("prec", ["f32", "bf16"])
def test_cautious_zero_steps(prec):
    dtype = torch.float32 if prec == "f32" else torch.bfloat16
    shapes = [(64, 200), (200, 64)]
    ins, host, oo = _run(shapes, dtype, prec, 42200, 0.05, 0.3, 1.0, ns_steps=0)
    for i, sh in enumerate(shapes):
        w0, g0, m0 = host[i]
        ref = O.muon_step_ref(w0, g0, m0, lr=0.05, weight_decay=0.3, coeffs=[], cautious=True)
        o = to_np(oo[i])
        assert O.rel_fro(o, ref["o"]) <= (1e-4 if prec == "f32" else 4e-3), sh
        _check(to_np(ins[i][0]), w0, o, ref, 0.05, 0.3, 1.0, prec == "bf16")


def test_cautious_flag_toggles_on_a_replayed_structure():
    """The flag travels with the call's scalars: one structure called with it
    off, on, off gives the plain update, the cautious one, the plain one."""
    import newton_schulz_orthogonalized_amd as nso
    from newton_schulz_orthogonalized_amd import _lib
    shape = (512, 1024)
    w, g, m = make_matrix_inputs(shape, 42300, torch.bfloat16, 1e-3, 0.02, 1e-3)
    w0, m0 = w.clone(), m.clone()
    oo = torch.zeros(shape, dtype=torch.float32, device="cuda")
    ws = _lib.workspace(nso.muon_workspace_bytes([w], [g], [m]), "cuda")
    outs = []
    for cautious in (False, True, False, True):
        w.copy_(w0)
        m.copy_(m0)
        nso.muon_step([w], [g], [m], lr=0.02, weight_decay=0.5, ortho_outs=[oo], workspace=ws, cautious_wd=cautious)
        torch.cuda.synchronize()
        outs.append((w.clone(), to_np(oo)))
    assert torch.equal(outs[0][0], outs[2][0]) and torch.equal(outs[1][0], outs[3][0])
    assert not torch.equal(outs[0][0], outs[1][0])
    wd0, o = to_np(w0), outs[1][1]
    u = np.float32(0.02) * o
    mask = wd0 * u >= 0
    want = wd0 - np.float32(0.02 * 0.5) * wd0 * mask - u
    assert np.all(np.abs(to_np(outs[1][0]) - want) <= 0.5 * bf16_ulp(want) + 2.0 ** -21 * (np.abs(wd0) + np.abs(u)))
