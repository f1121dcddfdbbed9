"""GPU parity of the fused path for short problems: a call with at least 256
(matrix, head) blocks whose short side is at most 128 (bf16, cubic steps) runs
every Newton-Schulz step but the last apply in one launch, one workgroup per
block, with B kept in LDS. Compared with the float64 oracle head by head, at
the bf16 tolerance; each test also checks that the fused kernel ran.
"""

import numpy as np
import pytest
import torch

from gpu_util import bf16_ulp, make_matrix_inputs, need_gpu, to_np
from oracle import muon_oracle as O

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
MOM_TOL = 1e-6


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    import newton_schulz_orthogonalized_amd as nso  # noqa: F401  (fails loudly without the library)
    yield


def _lib():
    from newton_schulz_orthogonalized_amd import _lib as L
    return L


def _run(shape, heads, seed, coeffs=None, ns_steps=5):
    import newton_schulz_orthogonalized_amd as nso
    L = _lib()
    w, g, m = make_matrix_inputs(shape, seed, torch.bfloat16, 1e-3, 0.02, 1e-3)
    w0, g0, m0 = to_np(w), to_np(g), to_np(m)
    oout = torch.zeros(shape, dtype=torch.float32, device="cuda")
    L.mu_profile_enable(True)
    nso.muon_step([w], [g], [m], lr=0.02, weight_decay=0.01, heads=[heads], ns_steps=ns_steps, coeffs=coeffs,
                  precision="bf16", ortho_outs=[oout])
    torch.cuda.synchronize()
    L.mu_profile_enable(False)
    fused = L.mu_profile_read(L.MU_K_FUSED)["launches"]
    ref = O.muon_step_ref(w0, g0, m0, lr=0.02, weight_decay=0.01, heads=heads,
                          coeffs=coeffs if coeffs is not None else None)
    return w0, to_np(w), to_np(m), to_np(oout), ref, fused


def _check(shape, heads, w0, w1, m1, o, ref):
    assert O.rel_fro(m1, ref["m"]) <= MOM_TOL
    assert O.rel_fro(o, ref["o"]) <= BF16_TOL
    for h, sl in enumerate(O.head_blocks(shape[0], heads)):
        assert O.rel_fro(o[sl], ref["o"][sl]) <= BF16_TOL, h
    want = w0 - 0.02 * 0.01 * w0 - 0.02 * o
    assert np.all(np.abs(w1 - want) <= bf16_ulp(want) * 0.5 + 8 * 2.0 ** -24 * (np.abs(w0) + 0.02 * np.abs(o)))


@pytest.mark.parametrize("shape,heads", [((32768, 512), 256),     # 256 wide 128 x 512 heads, 4 column blocks
                                         ((131072, 128), 256),    # 256 tall 512 x 128 heads
                                         ((25600, 300), 256),     # 100 x 300 heads: padded to 128 x 384, 3 blocks
                                         ((49152, 256), 384)])    # 384 heads of 128 x 256 (more blocks than CUs)
def test_fused_heads_match_oracle(shape, heads):
    print(f"[fused] shape={shape} heads={heads}", flush=True)
    w0, w1, m1, o, ref, fused = _run(shape, heads, 21000 + heads)
    assert fused == 1
    _check(shape, heads, w0, w1, m1, o, ref)


@pytest.mark.parametrize("coeffs", [[(1.5, -0.5, 0.0)], [(2.0, -1.2, 0.0), (1.6, -0.6, 0.0)]])
def test_fused_short_schedules(coeffs):
    shape, heads = (32768, 512), 256
    print(f"[fused] {len(coeffs)} step(s)", flush=True)
    w0, w1, m1, o, ref, fused = _run(shape, heads, 22000 + len(coeffs), coeffs=coeffs, ns_steps=len(coeffs))
    assert fused == 1
    _check(shape, heads, w0, w1, m1, o, ref)


def test_fused_not_used_below_threshold_or_for_quintic():
    shape, heads = (16384, 512), 128   # 128 short problems: the tiled path
    _, _, _, _, _, fused = _run(shape, heads, 23000)
    assert fused == 0
    coeffs = [(3.4445, -4.775, 2.0315)] * 5   # quintic steps take the A^2 pass
    w0, w1, m1, o, ref, fused = _run((32768, 512), 256, 23001, coeffs=coeffs)
    assert fused == 0
    _check((32768, 512), 256, w0, w1, m1, o, ref)


def test_fused_orthogonalize_call():
    import newton_schulz_orthogonalized_amd as nso
    L = _lib()
    from workloads import as_dtype, host_normal
    x = as_dtype(host_normal((32768, 512), 24000, 1e-3), torch.bfloat16)
    L.mu_profile_enable(True)
    out, = nso.orthogonalize([x.cuda()], heads=[256], precision="bf16")
    torch.cuda.synchronize()
    L.mu_profile_enable(False)
    assert L.mu_profile_read(L.MU_K_FUSED)["launches"] == 1
    ref, _ = O.orthogonalize_ref(to_np(x), heads=256)
    assert O.rel_fro(to_np(out), ref) <= BF16_TOL


def test_fused_matches_tiled_path_closely():
    """The same 256 heads, once through the fused path and once split into two
    calls of 128 (tiled path): both are bf16 runs of the same iteration, so
    they agree far inside the oracle tolerance."""
    import newton_schulz_orthogonalized_amd as nso
    shape, heads = (32768, 512), 256
    w, g, m = make_matrix_inputs(shape, 25000, torch.bfloat16, 1e-3, 0.02, 1e-3)
    o1 = torch.zeros(shape, dtype=torch.float32, device="cuda")
    nso.muon_step([w.clone()], [g], [m.clone()], lr=0.02, weight_decay=0.01, heads=[heads], precision="bf16",
                  ortho_outs=[o1])
    half = shape[0] // 2
    o2 = torch.zeros(shape, dtype=torch.float32, device="cuda")
    for part in (slice(0, half), slice(half, shape[0])):
        wp, gp, mp = w[part].clone(), g[part].clone(), m[part].clone()
        op = torch.zeros(wp.shape, dtype=torch.float32, device="cuda")
        nso.muon_step([wp], [gp], [mp], lr=0.02, weight_decay=0.01, heads=[heads // 2], precision="bf16",
                      ortho_outs=[op])
        o2[part] = op
    torch.cuda.synchronize()
    assert O.rel_fro(to_np(o1), to_np(o2)) <= 5e-3


def test_fused_and_tiled_problems_in_one_call():
    """A call holding a fused group (256 short heads) next to tiled problems
    (a 256-tile block, a ragged 128-tile block, a tall one): the fused launch,
    the tiled steps and the shared last-apply launches must not disturb each
    other."""
    import newton_schulz_orthogonalized_amd as nso
    specs = [((32768, 512), 256), ((1024, 2048), 1), ((300, 77), 1), ((1536, 640), 2)]
    print(f"[fused + tiled] {specs}", flush=True)
    ws, gs, ms, oo, host = [], [], [], [], []
    for i, (shape, heads) in enumerate(specs):
        w, g, m = make_matrix_inputs(shape, 26000 + 10 * i, torch.bfloat16, 1e-3, 0.02, 1e-3)
        host.append((to_np(w), to_np(g), to_np(m)))
        ws.append(w); gs.append(g); ms.append(m)
        oo.append(torch.zeros(shape, dtype=torch.float32, device="cuda"))
    L = _lib()
    L.mu_profile_enable(True)
    nso.muon_step(ws, gs, ms, lr=0.02, weight_decay=0.01, heads=[h for _, h in specs], precision="bf16",
                  ortho_outs=oo)
    torch.cuda.synchronize()
    L.mu_profile_enable(False)
    assert L.mu_profile_read(L.MU_K_FUSED)["launches"] == 1
    for i, (shape, heads) in enumerate(specs):
        w0, g0, m0 = host[i]
        ref = O.muon_step_ref(w0, g0, m0, lr=0.02, weight_decay=0.01, heads=heads)
        _check(shape, heads, w0, to_np(ws[i]), to_np(ms[i]), to_np(oo[i]), ref)
