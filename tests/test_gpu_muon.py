"""GPU parity of the Muon step and the orthogonalise-only call against the CPU
oracle, at sizes the oracle finishes in seconds (several GEMM tiles, ragged
tails, tall and wide blocks, heads, mixed lists) and on the degenerate cases.

Tolerances (relative Frobenius error against the float64 oracle): float32 path
1e-4, bf16-MFMA path 2e-2, momentum 1e-6.
"""

import numpy as np
import pytest
import torch

from gpu_util import bf16_ulp, check_w_against_oracle, make_matrix_inputs, need_gpu, tile_rel_fro, to_np
from oracle import muon_oracle as O
from workloads import as_dtype, host_normal

pytestmark = pytest.mark.gpu

F32_TOL = 1e-4
BF16_TOL = 2e-2
MOM_TOL = 1e-6


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    import newton_schulz_orthogonalized_amd as nso  # noqa: F401  (fails loudly without the library)
    yield


def nso():
    import newton_schulz_orthogonalized_amd as m
    return m


SHAPES = [(128, 256), (256, 128), (77, 300), (300, 77), (5, 3), (1, 9), (9, 1), (129, 1000), (520, 520),
          (640, 384), (768, 2304)]


@pytest.mark.parametrize("shape", SHAPES)
def test_orthogonalize_f32(shape):
    print(f"[orthogonalize f32] shape={shape}", flush=True)
    x = as_dtype(host_normal(shape, 101), torch.float32)
    out, = nso().orthogonalize([x.cuda()], precision="f32")
    ref, _ = O.orthogonalize_ref(to_np(x))
    assert O.rel_fro(to_np(out), ref) <= F32_TOL


@pytest.mark.parametrize("shape", SHAPES)
def test_orthogonalize_bf16(shape):
    print(f"[orthogonalize bf16] shape={shape}", flush=True)
    x = as_dtype(host_normal(shape, 202, 1e-3), torch.bfloat16)
    norm = torch.zeros(1, device="cuda")
    out, = nso().orthogonalize([x.cuda()], precision="bf16", norm_outs=[norm])
    ref, nref = O.orthogonalize_ref(to_np(x))
    # the bf16 output itself is rounded, which costs at most 2^-9 relative
    assert O.rel_fro(to_np(out), ref) <= BF16_TOL
    assert abs(norm.item() - nref[0]) <= 1e-5 * nref[0]


@pytest.mark.parametrize("prec,tol", [("f32", F32_TOL), ("bf16", BF16_TOL)])
def test_orthogonalize_f32_input_any_precision(prec, tol):
    x = as_dtype(host_normal((200, 330), 303), torch.float32)
    out, = nso().orthogonalize([x.cuda()], precision=prec)
    ref, _ = O.orthogonalize_ref(to_np(x))
    assert O.rel_fro(to_np(out), ref) <= tol


def _step_case(shape, dtype, prec, seed, heads=1, scale=1.0, lr=0.02, wd=0.01, nesterov=True, coeffs=None,
               ns_steps=5, gstd=1.0, wstd=1.0, mstd=1.0):
    w, g, m = make_matrix_inputs(shape, seed, dtype, gstd, wstd, mstd)
    w0, g0, m0 = to_np(w), to_np(g), to_np(m)
    oout = torch.zeros(shape, dtype=torch.float32, device="cuda")
    norms = torch.zeros(heads, dtype=torch.float32, device="cuda")
    nso().muon_step([w], [g], [m], lr=lr, weight_decay=wd, mu=0.95, nesterov=nesterov, heads=[heads],
                    scales=[scale], ns_steps=ns_steps, coeffs=coeffs, precision=prec, norm_outs=[norms],
                    ortho_outs=[oout])
    torch.cuda.synchronize()
    ref = O.muon_step_ref(w0, g0, m0, lr=lr, weight_decay=wd, mu=0.95, nesterov=nesterov, heads=heads,
                          coeffs=None if coeffs is None else coeffs if ns_steps else [], scale=scale)
    return w0, to_np(w), to_np(m), to_np(oout), to_np(norms), ref


def test_fp32_config_step_128x256():
    """The small float32 case: 128x256, N(0,1) inputs, 5 cubic steps, lr 0.02, wd 0.01."""
    w0, w1, m1, o, norms, ref = _step_case((128, 256), torch.float32, "f32", 7000)
    assert O.rel_fro(m1, ref["m"]) <= MOM_TOL
    assert O.rel_fro(o, ref["o"]) <= F32_TOL
    assert O.rel_fro(w1 - w0, ref["w"] - w0) <= F32_TOL
    assert abs(norms[0] - ref["norms"][0]) <= 1e-5 * ref["norms"][0]


@pytest.mark.parametrize("shape", [(1024, 1536), (1536, 1024), (1100, 1300), (1300, 1100)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32-param", "bf16-param"])
def test_f32_step_large_tiles(shape, dtype):
    """Float32 Newton-Schulz on blocks whose short side takes the 128 x 128
    float32 tiles (exact and ragged, wide and tall; the last apply's staged
    update for float32 and bf16 parameters): M, O, the update and the norm
    against the oracle."""
    print(f"[f32 step, 128 tiles] shape={shape} dtype={dtype}", flush=True)
    w0, w1, m1, o, norms, ref = _step_case(shape, dtype, "f32", 7100, gstd=1e-3, wstd=0.02, mstd=1e-3)
    assert O.rel_fro(m1, ref["m"]) <= MOM_TOL
    assert O.rel_fro(o, ref["o"]) <= F32_TOL
    assert tile_rel_fro(o, ref["o"], 128) <= F32_TOL
    assert abs(norms[0] - ref["norms"][0]) <= 1e-5 * ref["norms"][0]
    if dtype == torch.float32:
        assert O.rel_fro(w1 - w0, ref["w"] - w0) <= F32_TOL
    else:   # the update with the GPU's O, rounded once to bf16
        want = w0 - 0.02 * 0.01 * w0 - 0.02 * o
        assert np.all(np.abs(w1 - want) <= bf16_ulp(want) * 0.5 + 8 * 2.0 ** -24 * (np.abs(w0) + 0.02 * np.abs(o)))


@pytest.mark.parametrize("shape", [(768, 2304), (2304, 768), (768, 768), (300, 77), (129, 1000)])
def test_bf16_step(shape):
    print(f"[bf16 step] shape={shape}", flush=True)
    w0, w1, m1, o, _, ref = _step_case(shape, torch.bfloat16, "bf16", 8000, gstd=1e-3, wstd=0.02, mstd=1e-3)
    assert O.rel_fro(m1, ref["m"]) <= MOM_TOL
    assert O.rel_fro(o, ref["o"]) <= BF16_TOL
    assert tile_rel_fro(o, ref["o"]) <= BF16_TOL
    # the update arithmetic: W1 is the bf16 rounding of W0 - lr wd W0 - lr O (with the GPU's O)
    want = w0 - 0.02 * 0.01 * w0 - 0.02 * o
    assert np.all(np.abs(w1 - want) <= bf16_ulp(want) * 0.5 + 8 * 2.0 ** -24 * (np.abs(w0) + 0.02 * np.abs(o)))
    # and against the oracle's W
    frac = check_w_against_oracle(w1, w0, o, ref["w"], ref["o"], 0.02)
    print(f"[bf16 step] {shape}: W within 1 ulp of RNE(oracle W) for {100 * frac:.2f} %", flush=True)
    # without the O copy (the usual call) the parameter comes out bit for bit the same
    w, g, m = make_matrix_inputs(shape, 8000, torch.bfloat16, 1e-3, 0.02, 1e-3)
    nso().muon_step([w], [g], [m], lr=0.02, weight_decay=0.01, mu=0.95, nesterov=True, heads=[1], scales=[1.0],
                    precision="bf16")
    torch.cuda.synchronize()
    assert np.array_equal(to_np(w), w1)
    assert np.array_equal(to_np(m), m1)


@pytest.mark.parametrize("shape,heads", [((512, 256), 4), ((256, 64), 8), ((1024, 128), 2), ((4096, 4096), 32)])
@pytest.mark.parametrize("prec", ["f32", "bf16"])
def test_per_head(shape, heads, prec):
    print(f"[per-head] shape={shape} heads={heads} prec={prec}", flush=True)
    dtype = torch.float32 if prec == "f32" else torch.bfloat16
    w0, w1, m1, o, norms, ref = _step_case(shape, dtype, prec, 9000 + heads, heads=heads, gstd=1e-3, wstd=0.02,
                                           mstd=1e-3)
    tol = F32_TOL if prec == "f32" else BF16_TOL
    for h, sl in enumerate(O.head_blocks(shape[0], heads)):
        assert O.rel_fro(o[sl], ref["o"][sl]) <= tol, h
        assert tile_rel_fro(o[sl], ref["o"][sl], 128) <= tol, h
    assert np.allclose(norms, ref["norms"], rtol=1e-5, atol=0)


COEFF_SETS = [
    [(1.875, -1.25, 0.375)] * 5,                                   # quintic every step
    [(1.5, -0.5, 0.0), (1.875, -1.25, 0.375), (2.0, -1.5, 0.5), (1.5, -0.5, 0.0)],   # mixed, 4 steps
    [(1.5, -0.5, 0.0)] * 8,                                          # more cubic steps
    [(1.5, -0.5, 0.0)],                                              # one step
]


@pytest.mark.parametrize("ci", range(len(COEFF_SETS)))
@pytest.mark.parametrize("prec", ["f32", "bf16"])
def test_configurable_coefficients(ci, prec):
    coeffs = COEFF_SETS[ci]
    dtype = torch.float32 if prec == "f32" else torch.bfloat16
    w0, w1, m1, o, _, ref = _step_case((300, 520), dtype, prec, 9500 + ci, coeffs=coeffs, ns_steps=len(coeffs))
    assert O.rel_fro(o, ref["o"]) <= (F32_TOL if prec == "f32" else BF16_TOL)


@pytest.mark.parametrize("shape", [(768, 1000), (1000, 768)])
def test_quintic_on_256_tiles(shape):
    """Quintic steps where the bf16 path picks 256x256 tiles (several tiles per
    side): the A^2 pass, its mirrored and diagonal tiles, and an apply that reads
    B, in both orientations, mixed with cubic steps."""
    print(f"[quintic 256 tiles] shape={shape}", flush=True)
    coeffs = [(1.875, -1.25, 0.375)] * 3 + [(1.5, -0.5, 0.0)] * 2
    w0, w1, m1, o, _, ref = _step_case(shape, torch.bfloat16, "bf16", 9600, coeffs=coeffs, ns_steps=len(coeffs),
                                       gstd=1e-3, wstd=0.02, mstd=1e-3)
    assert O.rel_fro(o, ref["o"]) <= BF16_TOL


@pytest.mark.parametrize("prec", ["f32", "bf16"])
def test_zero_steps_applies_normalised_u(prec):
    dtype = torch.float32 if prec == "f32" else torch.bfloat16
    for shape in [(64, 200), (200, 64)]:
        w0, w1, m1, o, _, ref = _step_case(shape, dtype, prec, 9700, ns_steps=0, coeffs=[])
        assert O.rel_fro(o, ref["o"]) <= (F32_TOL if prec == "f32" else 4e-3)


def test_nesterov_off_and_scale():
    w0, w1, m1, o, _, ref = _step_case((256, 384), torch.float32, "f32", 9800, nesterov=False, scale=2.5,
                                       lr=0.05, wd=0.1)
    assert O.rel_fro(o, ref["o"]) <= F32_TOL
    assert O.rel_fro(w1 - w0, ref["w"] - w0) <= F32_TOL
    assert O.rel_fro(m1, ref["m"]) <= MOM_TOL


def test_mixed_list_one_call():
    """Shapes that land in different tile groups, tall and wide, with heads, in one call."""
    specs = [((768, 2304), 1), ((2304, 768), 1), ((128, 4096), 1), ((512, 256), 4), ((77, 300), 1),
             ((1024, 1024), 8), ((5, 3), 1)]
    ws, gs, ms, oo, w0s, g0s, m0s = [], [], [], [], [], [], []
    for i, (shape, heads) in enumerate(specs):
        w, g, m = make_matrix_inputs(shape, 12000 + 10 * i, torch.bfloat16, 1e-3, 0.02, 1e-3)
        ws.append(w); gs.append(g); ms.append(m)
        w0s.append(to_np(w)); g0s.append(to_np(g)); m0s.append(to_np(m))
        oo.append(torch.zeros(shape, dtype=torch.float32, device="cuda"))
    nso().muon_step(ws, gs, ms, lr=0.02, weight_decay=0.01, heads=[h for _, h in specs], ortho_outs=oo)
    torch.cuda.synchronize()
    for i, (shape, heads) in enumerate(specs):
        ref = O.muon_step_ref(w0s[i], g0s[i], m0s[i], lr=0.02, weight_decay=0.01, heads=heads)
        assert O.rel_fro(to_np(oo[i]), ref["o"]) <= BF16_TOL, shape
        assert O.rel_fro(to_np(ms[i]), ref["m"]) <= MOM_TOL, shape


def test_grouped_call_matches_separate_calls():
    """One call over several matrices (grouped launches: one grid covers every
    matrix, tiles found by search over the tile prefix) gives bitwise the same
    parameters, momenta and O as one call per matrix."""
    shapes = [(2048, 4608), (2048, 4608), (4608, 2048), (2048, 4608)]
    print(f"[grouped vs separate] shapes={shapes}", flush=True)
    ins = [make_matrix_inputs(sh, 13000 + i, torch.bfloat16, 1e-3, 0.02, 1e-3) for i, sh in enumerate(shapes)]
    kw = dict(lr=0.02, weight_decay=0.01, mu=0.95, nesterov=True, ns_steps=5, precision="bf16")
    w1 = [w.clone() for w, _, _ in ins]
    m1 = [m.clone() for _, _, m in ins]
    o1 = [torch.zeros(sh, dtype=torch.float32, device="cuda") for sh in shapes]
    nso().muon_step(w1, [g for _, g, _ in ins], m1, ortho_outs=o1, **kw)
    torch.cuda.synchronize()
    for i, (w, g, m) in enumerate(ins):
        w2, m2 = w.clone(), m.clone()
        o2 = torch.zeros(shapes[i], dtype=torch.float32, device="cuda")
        nso().muon_step([w2], [g], [m2], ortho_outs=[o2], **kw)
        torch.cuda.synchronize()
        assert torch.equal(w1[i], w2), i
        assert torch.equal(m1[i], m2), i
        assert torch.equal(o1[i], o2), i


def test_long_k_gram_windows():
    """A call dominated by long-K problems (K >= 12288), whose Gram tiles are
    dealt to the XCDs in windows: parity with the oracle, ragged shapes and a
    tall block included, and bitwise the same result as one call per matrix
    (a tile's arithmetic does not depend on the order tiles run in)."""
    shapes = [(1024, 12288), (12800, 512), (256, 16384), (300, 13000)]
    print(f"[long-K Gram windows] shapes={shapes}", flush=True)
    ins = [make_matrix_inputs(sh, 13500 + i, torch.bfloat16, 1e-3, 0.02, 1e-3) for i, sh in enumerate(shapes)]
    host = [(to_np(w), to_np(g), to_np(m)) for w, g, m in ins]
    kw = dict(lr=0.02, weight_decay=0.01, precision="bf16")
    w1 = [w.clone() for w, _, _ in ins]
    m1 = [m.clone() for _, _, m in ins]
    o1 = [torch.zeros(sh, dtype=torch.float32, device="cuda") for sh in shapes]
    nso().muon_step(w1, [g for _, g, _ in ins], m1, ortho_outs=o1, **kw)
    torch.cuda.synchronize()
    for i, sh in enumerate(shapes):
        ref = O.muon_step_ref(*host[i], lr=0.02, weight_decay=0.01)
        assert O.rel_fro(to_np(o1[i]), ref["o"]) <= BF16_TOL, sh
        assert O.rel_fro(to_np(m1[i]), ref["m"]) <= MOM_TOL, sh
        w, g, m = ins[i]
        w2, m2 = w.clone(), m.clone()
        o2 = torch.zeros(sh, dtype=torch.float32, device="cuda")
        nso().muon_step([w2], [g], [m2], ortho_outs=[o2], **kw)
        torch.cuda.synchronize()
        assert torch.equal(w1[i], w2) and torch.equal(o1[i], o2), sh


def test_long_k_quintic_steps():
    """Quintic steps (the A^2 pass) on a call dominated by long K, so both
    Gram passes run with windowed tile order and mirrored diagonal tiles."""
    shapes = [(512, 12800), (12544, 768)]
    coeffs = [(3.4445, -4.775, 2.0315)] * 5
    print(f"[long-K quintic] shapes={shapes}", flush=True)
    ins = [make_matrix_inputs(sh, 13700 + i, torch.bfloat16, 1e-3, 0.02, 1e-3) for i, sh in enumerate(shapes)]
    host = [(to_np(w), to_np(g), to_np(m)) for w, g, m in ins]
    oo = [torch.zeros(sh, dtype=torch.float32, device="cuda") for sh in shapes]
    nso().muon_step([w for w, _, _ in ins], [g for _, g, _ in ins], [m for _, _, m in ins], lr=0.02,
                    weight_decay=0.01, coeffs=coeffs, precision="bf16", ortho_outs=oo)
    torch.cuda.synchronize()
    for i, sh in enumerate(shapes):
        ref = O.muon_step_ref(*host[i], lr=0.02, weight_decay=0.01, coeffs=coeffs)
        assert O.rel_fro(to_np(oo[i]), ref["o"]) <= BF16_TOL, sh


@pytest.mark.parametrize("shape", [(2560, 2816), (2816, 2560)])
def test_gram_tile_blocks_with_a_partial_block(shape):
    """m = 2560: 10 x 10 Gram tiles of 256, enumerated as one 8 x 8 block, a
    partial 8 x 2 block and a 2 x 2 triangle, with diagonal tiles whose lower
    parts are mirrored; wide and tall."""
    print(f"[gram blocks] shape={shape}", flush=True)
    w, g, m = make_matrix_inputs(shape, 14100, torch.bfloat16, 1e-3, 0.02, 1e-3)
    w0, g0, m0 = to_np(w), to_np(g), to_np(m)
    o = torch.zeros(shape, dtype=torch.float32, device="cuda")
    nso().muon_step([w], [g], [m], lr=0.02, weight_decay=0.01, precision="bf16", ortho_outs=[o])
    torch.cuda.synchronize()
    ref = O.muon_step_ref(w0, g0, m0, lr=0.02, weight_decay=0.01)
    assert O.rel_fro(to_np(o), ref["o"]) <= BF16_TOL
    assert O.rel_fro(to_np(m), ref["m"]) <= MOM_TOL


@pytest.mark.parametrize("shape", [(256, 1 << 21), (1 << 21, 128)])
def test_longest_side_at_the_limit(shape):
    """A long side of 2^21, the largest the C ABI accepts: a wide block on the
    256-row tiles and a tall one on the 128-row tiles, each streaming one K
    of 2^21 through every Gram tile."""
    print(f"[longest side] shape={shape}", flush=True)
    w0, w1, m1, o, norms, ref = _step_case(shape, torch.bfloat16, "bf16", 9900, gstd=1e-3, wstd=0.02, mstd=1e-3)
    assert O.rel_fro(m1, ref["m"]) <= MOM_TOL
    assert O.rel_fro(o, ref["o"]) <= BF16_TOL
    assert abs(norms[0] - ref["norms"][0]) <= 1e-4 * ref["norms"][0]
    want = w0 - 0.02 * 0.01 * w0 - 0.02 * o
    assert np.all(np.abs(w1 - want) <= bf16_ulp(want) * 0.5 + 8 * 2.0 ** -24 * (np.abs(w0) + 0.02 * np.abs(o)))


def test_zero_gradient_and_momentum_decay_only():
    w = as_dtype(host_normal((256, 512), 13000, 0.02), torch.bfloat16).cuda()
    w0 = to_np(w)
    g = torch.zeros_like(w)
    m = torch.zeros(w.shape, dtype=torch.float32, device="cuda")
    oo = torch.full(w.shape, 7.0, dtype=torch.float32, device="cuda")
    nso().muon_step([w], [g], [m], lr=0.1, weight_decay=0.5, ortho_outs=[oo])
    torch.cuda.synchronize()
    assert torch.all(oo == 0)
    want = w0 - 0.1 * 0.5 * w0
    assert np.all(np.abs(to_np(w) - want) <= bf16_ulp(want) * 0.5 + 1e-6 * np.abs(want) + 1e-30)


def test_nan_stays_in_its_matrix():
    a = as_dtype(host_normal((64, 128), 13100), torch.float32).cuda()
    b = as_dtype(host_normal((64, 128), 13101), torch.float32).cuda()
    a_cpu = a.clone()
    a_cpu[3, 5] = float("nan")
    outs = nso().orthogonalize([a_cpu, b], precision="f32")
    torch.cuda.synchronize()
    assert torch.all(torch.isnan(outs[0]))
    ref, _ = O.orthogonalize_ref(to_np(b))
    assert O.rel_fro(to_np(outs[1]), ref) <= F32_TOL


def test_rank_one_inputs_keep_their_direction():
    """A rank-1 gradient maps to its unit dyad, not to zero (rank-1 hazard claim of the MuonClip page)."""
    u = host_normal(200, 13200)
    v = host_normal(70, 13201)
    x = as_dtype(np.outer(u, v), torch.float32).cuda()
    col = as_dtype(u[:, None], torch.float32).cuda()
    o1, o2 = nso().orthogonalize([x, col], precision="f32")
    want = np.outer(u / np.linalg.norm(u), v / np.linalg.norm(v))
    assert O.rel_fro(to_np(o1), want) <= F32_TOL
    assert O.rel_fro(to_np(o2)[:, 0], u / np.linalg.norm(u)) <= F32_TOL


@pytest.mark.parametrize("shape", [(256, 1024), (1024, 256)])
def test_bf16_rank_one_dominated_input(shape):
    """A rank-1 input plus 1 % noise in bf16: after normalisation its one large
    singular value is converged while the rest stay in the linear regime, the
    case where bf16 rounding costs the most accuracy."""
    m, n = shape
    u = host_normal(m, 13300)
    v = host_normal(n, 13301)
    x0 = np.outer(u, v) + 0.01 * host_normal(shape, 13302)
    x = as_dtype(x0, torch.bfloat16)
    out, = nso().orthogonalize([x.cuda()], precision="bf16")
    ref, _ = O.orthogonalize_ref(to_np(x))
    err = O.rel_fro(to_np(out), ref)
    print(f"[rank-1 dominated bf16] shape={shape} relF={err:.3e}", flush=True)
    assert err <= BF16_TOL


def test_determinism_bitwise():
    def run():
        w, g, m = make_matrix_inputs((768, 2304), 14000, torch.bfloat16, 1e-3, 0.02, 1e-3)
        oo = torch.zeros(w.shape, dtype=torch.float32, device="cuda")
        nso().muon_step([w], [g], [m], lr=0.02, weight_decay=0.01, ortho_outs=[oo])
        torch.cuda.synchronize()
        return w.cpu(), m.cpu(), oo.cpu()
    a, b = run(), run()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32),
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32))


def test_empty_list_is_noop():
    nso().muon_step([], [], [], lr=0.02, weight_decay=0.01)
    assert nso().orthogonalize([]) == []


def test_errors_leave_buffers_untouched():
    from newton_schulz_orthogonalized_amd import _lib
    w, g, m = make_matrix_inputs((30, 40), 15000, torch.float32)
    w0, m0 = w.clone(), m.clone()
    with pytest.raises(_lib.MuonError) as e:
        nso().muon_step([w], [g], [m], lr=0.02, weight_decay=0.01, heads=[7])
    assert e.value.status == _lib.MU_ERR_INVALID_ARG
    with pytest.raises(_lib.MuonError) as e:
        nso().muon_step([w], [g], [m], lr=0.02, weight_decay=0.01, workspace=torch.empty(256, dtype=torch.uint8,
                                                                                          device="cuda"))
    assert e.value.status == _lib.MU_ERR_WORKSPACE
    with pytest.raises(_lib.MuonError) as e:
        nso().muon_step([w], [w], [m], lr=0.02, weight_decay=0.01)   # grad aliases param
    assert e.value.status == _lib.MU_ERR_LAYOUT
    torch.cuda.synchronize()
    assert torch.equal(w, w0) and torch.equal(m, m0)


def test_side_stream_with_internal_workspace():
    """A step queued on a side stream with the workspace allocated inside the
    call: the buffer is recorded on the side stream, so memory allocated and
    overwritten on the current stream right after the call cannot be the
    workspace while the kernels still run. The result equals the same step on
    the current stream."""
    shape = (2048, 4608)
    w, g, m = make_matrix_inputs(shape, 16000, torch.bfloat16, 1e-3, 0.02, 1e-3)
    w2, m2 = w.clone(), m.clone()
    nso().muon_step([w2], [g], [m2], lr=0.02, weight_decay=0.01)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    need = nso().muon_workspace_bytes([w], [g], [m])
    nso().muon_step([w], [g], [m], lr=0.02, weight_decay=0.01, stream=side)
    junk = [torch.full((need // 4 + 1024,), float("nan"), device="cuda") for _ in range(3)]
    torch.cuda.synchronize()
    del junk
    assert torch.equal(w, w2) and torch.equal(m, m2)


def test_stream_capture_is_rejected():
    """Calls on a stream that is capturing a graph return MU_ERR_INVALID_ARG
    before enqueuing anything (the tables are staged through reused host
    memory, so a replay would read another call's table)."""
    from newton_schulz_orthogonalized_amd import _lib
    w, g, m = make_matrix_inputs((256, 384), 16100, torch.bfloat16, 1e-3, 0.02, 1e-3)
    w0, m0 = w.clone(), m.clone()
    ws = _lib.workspace(nso().muon_workspace_bytes([w], [g], [m]), "cuda")
    p = torch.zeros(1000, device="cuda")
    ea, eq, pg = torch.zeros_like(p), torch.zeros_like(p), torch.ones_like(p)
    aws = _lib.workspace(_lib.mu_adamw_workspace_size(1), "cuda")
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    for call in (lambda: nso().muon_step([w], [g], [m], lr=0.02, weight_decay=0.01, workspace=ws),
                 lambda: nso().muon_step([w], [g], [m], lr=0.02, weight_decay=0.01, noalloc=True),
                 lambda: nso().adamw_step([p], [pg], [ea], [eq], lr=0.1, weight_decay=0.0, workspace=aws)):
        graph = torch.cuda.CUDAGraph()
        with pytest.raises(_lib.MuonError) as e:
            with torch.cuda.graph(graph, stream=s):
                call()
        assert e.value.status == _lib.MU_ERR_INVALID_ARG and "captur" in str(e.value)
        del graph
    torch.cuda.synchronize()
    assert torch.equal(w, w0) and torch.equal(m, m0)
    assert torch.all(p == 0) and torch.all(ea == 0)


@pytest.mark.parametrize("shape", [(256, 1024), (1024, 256)])
def test_quintic_rank_one_dominated_f32(shape):
    """Quintic steps (15/8, -5/4, 3/8) grow the small singular values 23-fold
    over five steps, so on a rank-1 input with 1 % noise bf16 storage of X
    leaves about 2.5e-2 in those directions; the float32 path is the one for
    such schedules and meets its 1e-4 bound."""
    m, n = shape
    u = host_normal(m, 13400)
    v = host_normal(n, 13401)
    x0 = np.outer(u, v) + 0.01 * host_normal(shape, 13402)
    x = as_dtype(x0, torch.float32)
    q = [(1.875, -1.25, 0.375)] * 5
    out, = nso().orthogonalize([x.cuda()], coeffs=q, precision="f32")
    ref, _ = O.orthogonalize_ref(to_np(x), coeffs=q)
    err = O.rel_fro(to_np(out), ref)
    print(f"[quintic rank-1 dominated f32] shape={shape} relF={err:.3e}", flush=True)
    assert err <= F32_TOL
