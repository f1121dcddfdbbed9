"""Gram-side Newton-Schulz steps on the GPU against the CPU oracle.

Wide blocks (n > m, m >= 1024, bf16, cubic steps) run their first steps on
the m x m side: A_{k+1} = (B_k B_k) A_k, Q_{k+1} = B_k Q_k (symmetric products
of commuting matrices, computed on their upper tiles), then X_R = Q_R X_0 and
the remaining steps as usual. In exact arithmetic that is the iteration
of the MuonClip Optimizer page ("Newton-Schulz Orthogonalization"), so the
oracle is the plain iteration and the bar is the bf16 tolerance. The same
inputs with MU_GRAMSIDE=0 (every step on X) meet the same bar.
"""

import os

import numpy as np
import pytest
import torch

from gpu_util import check_w_against_oracle, make_matrix_inputs, need_gpu, tile_rel_fro, to_np
from oracle import muon_oracle as O
from workloads import as_dtype, host_normal

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
MOM_TOL = 1e-6


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    yield
    os.environ.pop("MU_GRAMSIDE", None)


def nso():
    import newton_schulz_orthogonalized_amd as m
    return m


def _ortho_check(x, steps=5, coeffs=None, heads=1, label=""):
    out, = nso().orthogonalize([x.cuda()], heads=[heads], ns_steps=steps, coeffs=coeffs, precision="bf16")
    torch.cuda.synchronize()
    ref, _ = O.orthogonalize_ref(to_np(x), heads=heads, coeffs=coeffs if coeffs is not None else
                                 O.default_coeffs(steps))
    o = to_np(out)
    err, terr = O.rel_fro(o, ref), tile_rel_fro(o, ref)
    print(f"[gram-side] {label} shape={tuple(x.shape)} steps={steps} heads={heads} "
          f"relF={err:.3e} worst tile={terr:.3e}", flush=True)
    assert np.isfinite(o).all()
    assert err <= BF16_TOL
    assert terr <= BF16_TOL
    return err


@pytest.mark.parametrize("shape", [(1024, 4096), (4096, 1024), (1000, 2600), (2600, 1000), (1024, 1300)])
def test_five_steps(shape):
    x = as_dtype(host_normal(shape, 31000 + shape[0]), torch.bfloat16)
    _ortho_check(x, 5, label="gaussian")


@pytest.mark.parametrize("steps", [3, 4, 7])
def test_restart_positions(steps):
    """Restart after 2, 3 and 3 Gram-side steps (3, 4 and 7 steps in all: the
    restart comes at step min(S - 1, 3))."""
    x = as_dtype(host_normal((1000, 2600), 31100 + steps), torch.bfloat16)
    _ortho_check(x, steps, label="ragged")


def test_per_step_coefficients():
    """Each step's own (a, b): B_{k+1} is formed with step k+1's pair in the
    epilogue of the product that forms A_{k+1}, so an off-by-one there fails
    against the oracle."""
    co = [(1.5 + 0.06 * k, -0.5 - 0.03 * k, 0.0) for k in range(6)]
    x = as_dtype(host_normal((1024, 3000), 31200), torch.bfloat16)
    _ortho_check(x, 6, coeffs=co, label="per-step coefficients")


def test_heads():
    x = as_dtype(host_normal((2048, 4096), 31300), torch.bfloat16)
    _ortho_check(x, 5, heads=2, label="two heads")


def test_rank_one_dominated():
    m, n = 1024, 4096
    u, v = host_normal(m, 31400), host_normal(n, 31401)
    x = as_dtype(np.outer(u, v) + 0.01 * host_normal((m, n), 31402), torch.bfloat16)
    _ortho_check(x, 5, label="rank-1 + 1 % noise")


# rank one plus 0.1 % noise: blocks on which a restart at step 4 went past the
# bf16 bound (worst 256 x 256 tile 2.0e-2 to 3.1e-2); with the restart at step
# 3 they stay at the plain steps' error (1.2-1.6e-2)
@pytest.mark.parametrize("shape,seed", [((4096, 1024), 3), ((1024, 1536), 2), ((2048, 4096), 2),
                                        ((1024, 4096), 0), ((1024, 2048), 0)])
def test_rank_one_with_small_noise(shape, seed):
    m, n = shape
    base = 50000 + 100 * seed + m + 7 * n + 23
    x = np.outer(host_normal(m, base), host_normal(n, base + 1)) + 0.001 * host_normal((m, n), base + 2)
    _ortho_check(as_dtype(x, torch.bfloat16), 5, label="rank-1 + 0.1 % noise")


def test_rank_one_with_small_noise_8b_mlp_shape():
    """The 8B set's MLP shape: with a restart at step 4 this block reached a
    worst 256 x 256 tile error of 2.8e-2; at step 3 it measures 1.2e-2 (worst
    tile 1.4e-2), within the bf16 bound."""
    m, n, seed, eps = 4096, 14336, 2, 1e-3
    base = 70000 + 100 * seed + m + 3 * n + int(1 / eps)
    x = np.outer(host_normal(m, base), host_normal(n, base + 1)) + eps * host_normal((m, n), base + 2)
    _ortho_check(as_dtype(x, torch.bfloat16), 5, label="8B MLP shape, rank-1 + 0.1 % noise")


def test_muon_step_mixed_list_on_and_off():
    """One Muon call over Gram-side blocks and plain ones (square, short, tall),
    with and without Gram-side steps: both against the oracle's O, M and W."""
    shapes = [(1024, 4096), (1024, 1024), (4096, 1024), (256, 1024), (1000, 2600), (2048, 1400)]
    results = {}
    for mode in ("on", "off"):
        if mode == "off":
            os.environ["MU_GRAMSIDE"] = "0"
        ws, gs, ms, oo, keep = [], [], [], [], []
        for i, sh in enumerate(shapes):
            w, g, m = make_matrix_inputs(sh, 31500 + 10 * i, torch.bfloat16, 1e-3, 0.02, 1e-3)
            keep.append((to_np(w), to_np(g), to_np(m)))
            ws.append(w); gs.append(g); ms.append(m)
            oo.append(torch.zeros(sh, dtype=torch.float32, device="cuda"))
        nso().muon_step(ws, gs, ms, lr=0.02, weight_decay=0.01, ortho_outs=oo)
        torch.cuda.synchronize()
        results[mode] = [to_np(o) for o in oo]
        for i, sh in enumerate(shapes):
            w0, g0, m0 = keep[i]
            ref = O.muon_step_ref(w0, g0, m0, lr=0.02, weight_decay=0.01)
            o = results[mode][i]
            err = O.rel_fro(o, ref["o"])
            print(f"[gram-side step {mode}] {sh}: O relF {err:.3e}", flush=True)
            assert err <= BF16_TOL
            assert tile_rel_fro(o, ref["o"]) <= BF16_TOL
            assert O.rel_fro(to_np(ms[i]), ref["m"]) <= MOM_TOL
            check_w_against_oracle(to_np(ws[i]), w0, o, ref["w"], ref["o"], 0.02)
    # blocks that never take Gram-side steps run the same kernels either way
    for i in (1, 3):
        assert np.array_equal(results["on"][i], results["off"][i]), shapes[i]


def test_repeated_calls_replay_bit_for_bit():
    """The second call of a structure replays the captured launch sequence
    (all Gram-side launches included): bit for bit the first call's result."""
    x = as_dtype(host_normal((1024, 4096), 31600), torch.bfloat16).cuda()
    outs = []
    for _ in range(3):
        out, = nso().orthogonalize([x], precision="bf16")
        torch.cuda.synchronize()
        outs.append(out.clone())
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[1], outs[2])


@pytest.mark.parametrize("cautious", [False, True])
def test_float32_parameters_scale_and_cautious_decay(cautious):
    """Gram-side blocks with float32 parameters (bf16 Newton-Schulz), a
    per-matrix scale of 2 and, optionally, cautious weight decay: the last
    apply's float32 update instance after the restart. O, M and the float32
    update W1 - W0 against the oracle."""
    shapes = [(1024, 2048), (2048, 1024)]
    ws, gs, ms, oo, keep = [], [], [], [], []
    for i, sh in enumerate(shapes):
        w, g, m = make_matrix_inputs(sh, 31700 + 10 * i, torch.float32, 1.0, 1.0, 1.0)
        keep.append((to_np(w), to_np(g), to_np(m)))
        ws.append(w); gs.append(g); ms.append(m)
        oo.append(torch.zeros(sh, dtype=torch.float32, device="cuda"))
    nso().muon_step(ws, gs, ms, lr=0.05, weight_decay=0.3, scales=[2.0, 2.0], ortho_outs=oo, precision="bf16",
                    cautious_wd=cautious)
    torch.cuda.synchronize()
    for i, sh in enumerate(shapes):
        w0, g0, m0 = keep[i]
        ref = O.muon_step_ref(w0, g0, m0, lr=0.05, weight_decay=0.3, scale=2.0, cautious=cautious)
        o = to_np(oo[i])
        err = O.rel_fro(o, ref["o"])
        print(f"[gram-side f32 params] {sh} cautious={cautious}: O relF {err:.3e}", flush=True)
        assert err <= BF16_TOL
        assert O.rel_fro(to_np(ms[i]), ref["m"]) <= MOM_TOL
        # the update with the GPU's own O, element by element (cautious: the same sign rule)
        u = 0.05 * 2.0 * o
        decay = 0.05 * 0.3 * np.where(cautious & (w0 * u < 0), 0.0, 1.0)
        want = w0 - decay * w0 - u
        assert np.allclose(to_np(ws[i]), want, rtol=1e-5, atol=1e-6)
        # and against the oracle's W: the difference is lr scale (O - O_ref) away from the decay
        dw, dref = to_np(ws[i]) - w0, ref["w"] - w0
        assert O.rel_fro(dw, dref) <= BF16_TOL


# seeds whose draws give 3, 4, 5, 6 and 7 steps (restart after 2, 3, 3, 3 and 3
# Gram-side steps), two to four Gram-side blocks each, and heads in two of them
@pytest.mark.parametrize("seed", [26, 1, 25, 20, 11])
def test_random_lists_with_gram_side_blocks(seed):
    """Seeded random lists in which most blocks take Gram-side steps (wide or
    tall, with or without heads, ragged sides), with 3 to 7 cubic steps and
    per-step coefficients drawn per call, so the restart falls at every
    position it can take; plain blocks ride along. O (whole matrix and every
    256 x 256 tile) and M against the oracle."""
    rng = np.random.default_rng(32000 + seed)
    sides = [256, 777, 1000, 1024, 1100, 1280, 1536, 2048, 2300, 3000]
    specs = []
    while len(specs) < int(rng.integers(3, 6)):
        r, c = (int(x) for x in rng.choice(sides, 2))
        if r * c > 2_400_000:
            continue
        specs.append(((r, c), 2 if r % 2 == 0 and r >= 2048 and rng.random() < 0.5 else 1))
    steps = int(rng.integers(3, 8))
    co = [(1.5 + 0.02 * int(rng.integers(0, 5)), -0.5 + 0.01 * int(rng.integers(0, 3)), 0.0) for _ in range(steps)]
    nest = bool(seed % 2 == 0)
    print(f"[gram-side random] seed={seed} steps={steps} nesterov={nest} specs={specs}", flush=True)
    ws, gs, ms, oo, keep = [], [], [], [], []
    for i, (sh, _) in enumerate(specs):
        w, g, m = make_matrix_inputs(sh, 32100 + 100 * seed + 10 * i, torch.bfloat16, 1e-3, 0.02, 1e-3)
        keep.append((to_np(w), to_np(g), to_np(m)))
        ws.append(w); gs.append(g); ms.append(m)
        oo.append(torch.zeros(sh, dtype=torch.float32, device="cuda"))
    nso().muon_step(ws, gs, ms, lr=0.02, weight_decay=0.01, nesterov=nest, heads=[h for _, h in specs],
                    ns_steps=steps, coeffs=co, ortho_outs=oo)
    torch.cuda.synchronize()
    for i, (sh, heads) in enumerate(specs):
        w0, g0, m0 = keep[i]
        ref = O.muon_step_ref(w0, g0, m0, lr=0.02, weight_decay=0.01, nesterov=nest, heads=heads, coeffs=co)
        o = to_np(oo[i])
        err, terr = O.rel_fro(o, ref["o"]), tile_rel_fro(o, ref["o"])
        print(f"[gram-side random]   {sh} heads={heads}: O relF {err:.3e}, worst tile {terr:.3e}", flush=True)
        assert np.isfinite(o).all()
        assert err <= BF16_TOL and terr <= BF16_TOL, (sh, heads)
        assert O.rel_fro(to_np(ms[i]), ref["m"]) <= MOM_TOL, (sh, heads)
