"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every check here is independent of the oracle's own code path: closed forms,
scalar recursions in plain Python floats, LAPACK's SVD, torch's bfloat16 cast,
brute-force loops, algebraic identities, and the constants the pages print.
"""

import json
import math
import os

import numpy as np
import pytest

from oracle import muon_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _semi_orthogonal(r, c, seed):
    """A random r x c matrix with orthonormal rows (r <= c) or columns."""
    g = _rng(seed).standard_normal((max(r, c), min(r, c)))
    q, _ = np.linalg.qr(g)
    return q.T if r <= c else q


def _phi_chain(s, coeffs):
    """The scalar map every singular value goes through, in plain floats."""
    for a, b, c in coeffs:
        s = a * s + b * s ** 3 + c * s ** 5
    return s


# --------------------------------------------------------------------------
# constants printed by the pages
# --------------------------------------------------------------------------

def test_page_constants_match_oracle_defaults():
    with open(os.path.join(GOLDEN, "page_constants.json")) as f:
        k = json.load(f)
    assert O.DEFAULT_MU == k["momentum_decay"]["value"]
    assert O.DEFAULT_NS_STEPS == k["newton_schulz_steps"]["value"]
    assert list(O.CUBIC[:2]) == k["newton_schulz_cubic_coefficients"]["value"]
    assert O.CUBIC[2] == 0.0
    assert O.default_coeffs() == [O.CUBIC] * 5
    assert O.route_ref(k["routing_min_ndim_for_muon"]["value"]) == "muon"
    assert O.route_ref(1) == "adamw" and O.route_ref(0) == "adamw"
    assert O.route_ref(2, is_embedding_or_head=True) == k["embedding_and_head_rule"]["value"]


# --------------------------------------------------------------------------
# Newton-Schulz: spectral closed form (SVD from LAPACK)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(7, 19), (19, 7), (12, 12), (1, 9), (9, 1), (32, 48)])
@pytest.mark.parametrize("coeffs", [
    O.default_coeffs(5),
    O.default_coeffs(1),
    [(1.5, -0.5, 0.0), (2.0, -1.25, 0.25), (1.7, -0.9, 0.2)],
    [(3.4445, -4.7750, 2.0315)] * 3,
])
def test_ns_matches_spectral_map(shape, coeffs):
    x = _rng(sum(shape))
    x = x.standard_normal(shape)
    x /= np.linalg.norm(x)  # singular values in (0, 1]
    got = O.newton_schulz_ref(x, coeffs)
    want = O.ns_spectral_ref(x, coeffs)
    assert O.rel_fro(got, want) < 1e-11
    # and the spectral form itself against the scalar chain on the singular values
    s = np.linalg.svd(x, compute_uv=False)
    s_out = np.linalg.svd(got, compute_uv=False)
    chained = np.sort(np.abs([_phi_chain(float(v), coeffs) for v in s]))[::-1]
    assert np.allclose(s_out, chained, rtol=1e-10, atol=1e-13)


def test_ns_zero_steps_is_identity():
    x = _rng(3).standard_normal((5, 8))
    assert np.array_equal(O.newton_schulz_ref(x, []), x)


def test_ns_two_coefficient_form_equals_cubic():
    x = _rng(4).standard_normal((6, 10)) / 10
    assert np.allclose(O.newton_schulz_ref(x, [(1.5, -0.5)] * 5), O.newton_schulz_ref(x), rtol=0, atol=0)


# --------------------------------------------------------------------------
# Special cases with closed forms
# --------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(16, 64), (64, 16), (20, 20)])
def test_semi_orthogonal_is_fixed_point_of_cubic_step(shape):
    q = _semi_orthogonal(*shape, seed=11)
    out = O.newton_schulz_ref(q)
    assert np.max(np.abs(out - q)) < 1e-13


@pytest.mark.parametrize("r,c", [(128, 256), (256, 128), (64, 64), (8, 1024)])
def test_pipeline_on_semi_orthogonal_input(r, c):
    """||Q||_F = sqrt(min(r,c)), so every singular value after normalisation is
    1/(sqrt(k) + eps) with k = min(r, c), and the output is phi^5 of that times Q."""
    q = _semi_orthogonal(r, c, seed=r + c)
    k = min(r, c)
    assert abs(np.linalg.norm(q) - math.sqrt(k)) < 1e-10  # Frobenius, not another norm
    out, norms = O.orthogonalize_ref(q)
    assert abs(norms[0] - math.sqrt(k)) < 1e-10
    s0 = 1.0 / (math.sqrt(k) + O.DEFAULT_NORM_EPS)
    factor = _phi_chain(s0, O.default_coeffs())
    assert np.max(np.abs(out - factor * q)) < 1e-12


def test_rank_one_input_maps_to_its_unit_dyad():
    """Contradicts the MuonClip page's rank-1 hazard claim: after Frobenius
    normalisation the single singular value is 1 (up to eps), a fixed point, so
    the result is (u/|u|)(v/|v|)^T, not zero."""
    rng = _rng(21)
    u = rng.standard_normal(40)
    v = rng.standard_normal(90)
    out, _ = O.orthogonalize_ref(np.outer(u, v))
    want = np.outer(u / np.linalg.norm(u), v / np.linalg.norm(v))
    assert np.max(np.abs(out - want)) < 1e-12
    # the [d, 1] head of the page: a column vector maps to its unit vector
    col, _ = O.orthogonalize_ref(u[:, None])
    assert np.max(np.abs(col[:, 0] - u / np.linalg.norm(u))) < 1e-12


def test_well_conditioned_input_reaches_polar_factor():
    """Singular values 0.8 and 0.6 after normalisation: five cubic steps bring
    both within 3e-9 of 1, so the result is the polar factor U V^T (LAPACK)."""
    rng = _rng(5)
    u, _ = np.linalg.qr(rng.standard_normal((2, 2)))
    v, _ = np.linalg.qr(rng.standard_normal((9, 2)))
    x = u @ np.diag([0.8, 0.6]) @ v.T  # ||x||_F = 1 exactly
    out, _ = O.orthogonalize_ref(x, eps=0.0)
    uu, _, vt = np.linalg.svd(x, full_matrices=False)
    polar = uu @ vt
    assert np.max(np.abs(out - polar)) < 3e-9
    assert np.max(np.abs(out - polar)) > 1e-12  # five steps do not fully converge


def test_zero_input_gives_zero_direction_and_pure_decay():
    w = _rng(6).standard_normal((4, 6))
    r = O.muon_step_ref(w, np.zeros((4, 6)), np.zeros((4, 6)), lr=0.1, weight_decay=0.5)
    assert np.all(r["o"] == 0.0)
    assert np.allclose(r["w"], w * (1 - 0.05), rtol=0, atol=1e-15)


def test_nan_propagates():
    g = np.ones((3, 5))
    g[1, 2] = np.nan
    r = O.muon_step_ref(np.zeros((3, 5)), g, np.zeros((3, 5)), lr=0.1, weight_decay=0.0)
    assert np.all(np.isnan(r["o"]))


# --------------------------------------------------------------------------
# Symmetries of the whole normalise + iterate pipeline
# --------------------------------------------------------------------------

def test_transpose_equivariance():
    x = _rng(7).standard_normal((12, 30))
    a, _ = O.orthogonalize_ref(x)
    b, _ = O.orthogonalize_ref(x.T)
    assert O.rel_fro(b, a.T) < 1e-13


def test_orthogonal_equivariance_oddness_and_scale_invariance():
    rng = _rng(8)
    x = rng.standard_normal((10, 25))
    p, _ = np.linalg.qr(rng.standard_normal((10, 10)))
    q, _ = np.linalg.qr(rng.standard_normal((25, 25)))
    base, _ = O.orthogonalize_ref(x)
    rot, _ = O.orthogonalize_ref(p @ x @ q)
    assert O.rel_fro(rot, p @ base @ q) < 1e-12
    neg, _ = O.orthogonalize_ref(-x)
    assert O.rel_fro(neg, -base) < 1e-15
    scaled, _ = O.orthogonalize_ref(37.5 * x, eps=0.0)
    unscaled, _ = O.orthogonalize_ref(x, eps=0.0)
    assert O.rel_fro(scaled, unscaled) < 1e-13


def test_output_times_input_transpose_is_symmetric_psd():
    x = _rng(9).standard_normal((14, 40))
    out, _ = O.orthogonalize_ref(x)
    x0, _ = O.frobenius_normalize_ref(x)
    s = out @ x0.T
    assert np.max(np.abs(s - s.T)) < 1e-13
    assert np.min(np.linalg.eigvalsh((s + s.T) / 2)) > -1e-13


def test_per_head_equals_pipeline_on_each_row_block():
    x = _rng(10).standard_normal((24, 16))
    out, norms = O.orthogonalize_ref(x, heads=4)
    for h in range(4):
        blk, s = O.orthogonalize_ref(x[6 * h:6 * h + 6])
        assert np.array_equal(out[6 * h:6 * h + 6], blk)
        assert norms[h] == s[0]
    # and differs from orthogonalising the whole matrix at once
    whole, _ = O.orthogonalize_ref(x)
    assert O.rel_fro(out, whole) > 1e-2


def test_heads_must_divide_rows():
    with pytest.raises(ValueError):
        O.orthogonalize_ref(np.ones((10, 4)), heads=3)


# --------------------------------------------------------------------------
# Cautious weight decay (a reading: decay only where it agrees with the update)
# --------------------------------------------------------------------------

def test_cautious_decay_hand_values():
    # lr 0.1, wd 0.5 (decay factor 0.05), scale 2: u = 0.2 * O
    w = np.array([1.0, 1.0, -2.0, -2.0, 0.0, 3.0])
    o = np.array([0.5, -0.5, -1.0, 1.0, 4.0, 0.0])
    got = O.muon_update_ref(w, o, lr=0.1, weight_decay=0.5, scale=2.0, cautious=True)
    # same sign: decayed (1 - 0.05 - 0.1 = 0.85; -2 + 0.1 + 0.2 = -1.7); opposite sign: not
    # (1 + 0.1 = 1.1; -2 - 0.2 = -2.2); W = 0: only the update (-0.8); O = 0: plain decay (2.85)
    want = np.array([0.85, 1.1, -1.7, -2.2, -0.8, 2.85])
    assert np.allclose(got, want, rtol=0, atol=1e-15)


def test_cautious_decay_reduces_to_the_two_plain_updates():
    rng = _rng(50)
    w = np.abs(rng.standard_normal((5, 9))) + 0.1
    o = np.abs(rng.standard_normal((5, 9))) + 0.1
    # every W u > 0: the plain decoupled update
    assert np.array_equal(O.muon_update_ref(w, o, 0.02, 0.1, 1.5, cautious=True),
                          O.muon_update_ref(w, o, 0.02, 0.1, 1.5))
    # every W u < 0: the update without decay
    assert np.array_equal(O.muon_update_ref(w, -o, 0.02, 0.1, 1.5, cautious=True),
                          O.muon_update_ref(w, -o, 0.02, 0.0, 1.5))
    # a negative scale flips which coordinates decay
    assert np.array_equal(O.muon_update_ref(w, o, 0.02, 0.1, -1.5, cautious=True),
                          O.muon_update_ref(w, o, 0.02, 0.0, -1.5))


def test_cautious_step_changes_only_the_update():
    rng = _rng(51)
    w, g, m = (rng.standard_normal((6, 10)) for _ in range(3))
    a = O.muon_step_ref(w, g, m, lr=0.05, weight_decay=0.2)
    b = O.muon_step_ref(w, g, m, lr=0.05, weight_decay=0.2, cautious=True)
    assert np.array_equal(a["o"], b["o"]) and np.array_equal(a["m"], b["m"])
    keep = w * (0.05 * b["o"]) >= 0
    assert np.array_equal(a["w"][keep], b["w"][keep])
    assert np.allclose(b["w"][~keep], (w - 0.05 * b["o"])[~keep], rtol=0, atol=1e-15)


# --------------------------------------------------------------------------
# Exact arithmetic on tiny inputs: the iteration in rational numbers
# --------------------------------------------------------------------------

def _exact_pipeline(x, norm, steps):
    """X / norm, then each step X <- a X + b X X^T X + c X X^T X X^T X with every
    entry written as its scalar sum over the inner indices, in Fractions."""
    from fractions import Fraction as Fr
    r, c = len(x), len(x[0])
    cur = [[Fr(v) / norm for v in row] for row in x]
    for a, b, q in steps:
        a, b, q = Fr(a), Fr(b), Fr(q)
        # G[i][l] = sum_k x_ik x_lk, then (G X)_ij and (G G X)_ij
        g = [[sum(cur[i][k] * cur[l][k] for k in range(c)) for l in range(r)] for i in range(r)]
        gx = [[sum(g[i][l] * cur[l][j] for l in range(r)) for j in range(c)] for i in range(r)]
        ggx = [[sum(g[i][l] * gx[l][j] for l in range(r)) for j in range(c)] for i in range(r)]
        cur = [[a * cur[i][j] + b * gx[i][j] + q * ggx[i][j] for j in range(c)] for i in range(r)]
    return np.array([[float(v) for v in row] for row in cur])


@pytest.mark.parametrize("x,norm", [([[1, 2, 2], [0, 4, 0]], 5), ([[2, 0], [1, 2], [0, 4]], 5),
                                    ([[1, 1, 1, 1]], 2)])
def test_exact_rational_cubic_iteration(x, norm):
    """Inputs whose Frobenius norm is an integer, with eps = 0, so X0 is
    rational and five cubic steps can be done exactly; the float64 pipeline
    (tall inputs included) must agree to rounding."""
    from fractions import Fraction as Fr
    want = _exact_pipeline(x, norm, [(Fr(3, 2), Fr(-1, 2), 0)] * 5)
    out, norms = O.orthogonalize_ref(np.array(x, dtype=np.float64), eps=0.0)
    assert norms[0] == float(norm)
    assert np.max(np.abs(out - want)) < 1e-15


def test_exact_rational_mixed_coefficients():
    from fractions import Fraction as Fr
    steps = [(Fr(15, 8), Fr(-5, 4), Fr(3, 8)), (Fr(3, 2), Fr(-1, 2), 0), (Fr(2), Fr(-3, 2), Fr(1, 2))]
    x = [[1, 2, 2], [0, 4, 0]]
    want = _exact_pipeline(x, 5, steps)
    out, _ = O.orthogonalize_ref(np.array(x, dtype=np.float64), coeffs=[tuple(map(float, t)) for t in steps],
                                 eps=0.0)
    assert np.max(np.abs(out - want)) < 1e-15


# --------------------------------------------------------------------------
# Extreme magnitudes and the zero input
# --------------------------------------------------------------------------

@pytest.mark.parametrize("c", [1e-25, 1e-35, 1e18, 1e30])
def test_scale_invariance_at_extreme_magnitudes(c):
    """With eps = 0 the iteration sees only U / ||U||_F, so a positive factor
    drops out at either end of the float32 range."""
    x = _rng(40).standard_normal((9, 21))
    base, nb = O.orthogonalize_ref(x, eps=0.0)
    out, ns = O.orthogonalize_ref(c * x, eps=0.0)
    assert O.rel_fro(out, base) < 1e-13
    assert abs(ns[0] / (c * nb[0]) - 1.0) < 1e-14


@pytest.mark.parametrize("coeffs", [None, [(1.875, -1.25, 0.375), (1.5, -0.5, 0.0), (2.0, -1.5, 0.5)]])
def test_input_far_below_eps_stays_linear(coeffs):
    """||U||_F << eps: X0 = U / (||U||_F + eps) has singular values near 1e-18,
    where a step multiplies X by a to within |b| s^2 ~ 1e-36 relative, so the
    output is the product of the a_k times X0."""
    x = _rng(41).standard_normal((9, 21)) * 1e-25
    out, norms = O.orthogonalize_ref(x, coeffs=coeffs)
    ks = O.default_coeffs() if coeffs is None else coeffs
    gain = float(np.prod([k[0] for k in ks]))
    x0 = x / (norms[0] + O.DEFAULT_NORM_EPS)
    assert O.rel_fro(out, gain * x0) < 1e-14


def test_zero_input_with_zero_eps_gives_zero_direction():
    out, norms = O.orthogonalize_ref(np.zeros((3, 7)), eps=0.0)
    assert np.all(out == 0.0) and norms[0] == 0.0
    w = _rng(42).standard_normal((3, 7))
    r = O.muon_step_ref(w, np.zeros((3, 7)), np.zeros((3, 7)), lr=0.1, weight_decay=0.5, eps=0.0)
    assert np.all(r["o"] == 0.0)
    assert np.allclose(r["w"], w * (1 - 0.05), rtol=0, atol=1e-15)


# --------------------------------------------------------------------------
# The parity measure itself
# --------------------------------------------------------------------------

def test_rel_fro_hand_values():
    # ||x - ref||_F / ||ref||_F: a difference of 1 against sqrt(1 + 4 + 9 + 25)
    assert abs(O.rel_fro([[1, 2], [3, 4]], [[1, 2], [3, 5]]) - 1 / math.sqrt(39)) < 1e-16
    # the denominator is the reference's norm, not the candidate's
    assert O.rel_fro([6.0, 8.0], [3.0, 4.0]) == 1.0
    assert O.rel_fro([3.0, 4.0], [6.0, 8.0]) == 0.5
    assert O.rel_fro([0.0, 0.0], [3.0, 4.0]) == 1.0
    # a zero reference: the absolute error
    assert O.rel_fro([3.0, 4.0], [0.0, 0.0]) == 5.0
    assert O.rel_fro([0.0, 0.0], [0.0, 0.0]) == 0.0
    # every element counts, whatever the shape
    assert O.rel_fro(np.ones((2, 3)), np.zeros((2, 3)) + 2.0) == 0.5


# --------------------------------------------------------------------------
# Momentum and Nesterov, element by element in plain floats
# --------------------------------------------------------------------------

def test_momentum_hand_values():
    # G = 1, M = 0, mu = 0.95: M_new = 0.05; Nesterov U = 0.05 + 0.95 * 0.05 = 0.0975
    m, u = O.momentum_ref(np.array([1.0]), np.array([0.0]), 0.95, True)
    assert abs(m[0] - 0.05) < 1e-16 and abs(u[0] - 0.0975) < 1e-16
    m, u = O.momentum_ref(np.array([1.0]), np.array([0.0]), 0.95, False)
    assert u[0] == m[0]
    # G = -2, M = 4, mu = 0.5: M_new = 2 - 1 = 1; U = -1 + 0.5 = -0.5
    m, u = O.momentum_ref(np.array([-2.0]), np.array([4.0]), 0.5, True)
    assert m[0] == 1.0 and u[0] == -0.5


def test_nesterov_reading_equals_sum_form_direction():
    """EMA buffer M and sum-form buffer M/(1-mu) give the same direction."""
    rng = _rng(13)
    g = rng.standard_normal((6, 11))
    m_sum = rng.standard_normal((6, 11))
    mu = 0.95
    _, u_ema = O.momentum_ref(g, (1 - mu) * m_sum, mu, True)
    m_sum_new = mu * m_sum + g
    u_sum = g + mu * m_sum_new
    assert np.allclose(u_ema, (1 - mu) * u_sum, rtol=1e-14, atol=1e-15)
    a, _ = O.orthogonalize_ref(u_ema, eps=0.0)
    b, _ = O.orthogonalize_ref(u_sum, eps=0.0)
    assert O.rel_fro(a, b) < 1e-13


def test_update_hand_values_and_scale():
    w = np.array([[1.0, -2.0]])
    o = np.array([[0.5, 0.25]])
    got = O.muon_update_ref(w, o, lr=0.1, weight_decay=0.2, scale=2.0)
    # 1 - 0.02 - 0.1 * 2 * 0.5 = 0.88 ; -2 + 0.04 - 0.05 = -2.01
    assert np.allclose(got, [[0.88, -2.01]], rtol=0, atol=1e-15)


# --------------------------------------------------------------------------
# AdamW closed forms
# --------------------------------------------------------------------------

def test_adamw_first_step_from_zero_state_is_sign_like():
    p = np.array([1.0, -3.0, 0.5])
    g = np.array([0.5, -0.25, 2.0])
    z = np.zeros(3)
    lr, wd, eps = 0.02, 0.01, 1e-8
    pn, m, v = O.adamw_ref(p, g, z, z, lr=lr, weight_decay=wd, beta1=0.9, beta2=0.95, eps=eps, step=1)
    want = [pi - lr * wd * pi - lr * gi / (abs(gi) + eps) for pi, gi in zip(p, g)]
    assert np.allclose(pn, want, rtol=0, atol=1e-15)
    # first entry by hand: 1 - 0.0002 - 0.02 * 0.5 / 0.50000001
    assert abs(pn[0] - (1 - 0.0002 - 0.01 / 0.50000001)) < 1e-15
    assert np.allclose(m, 0.1 * g) and np.allclose(v, 0.05 * g * g)


@pytest.mark.parametrize("t", [1, 2, 10, 100])
def test_adamw_constant_gradient_bias_correction_is_exact(t):
    """With a constant gradient from zero state, m_t = (1-b1^t) g and
    v_t = (1-b2^t) g^2, so the bias-corrected step is g/(|g|+eps) at every t."""
    g = np.array([0.3, -1.7])
    p = np.array([2.0, -1.0])
    m = np.zeros(2)
    v = np.zeros(2)
    for k in range(1, t + 1):
        pn, m, v = O.adamw_ref(p, g, m, v, lr=0.01, weight_decay=0.0, beta1=0.9, beta2=0.95, eps=1e-8, step=k)
        step = pn - p
        assert np.allclose(step, -0.01 * g / (np.abs(g) + 1e-8), rtol=1e-12, atol=0)
        p = pn


def test_adamw_eps_sits_outside_the_square_root():
    g = np.array([1e-9])
    z = np.zeros(1)
    pn, _, _ = O.adamw_ref(np.zeros(1), g, z, z, lr=1.0, weight_decay=0.0, beta1=0.9, beta2=0.95, eps=1e-8, step=1)
    assert abs(pn[0] - (-1e-9 / (1e-9 + 1e-8))) < 1e-15


def test_adamw_zero_gradient_is_pure_decay_and_bad_step_rejected():
    p = np.array([3.0])
    z = np.zeros(1)
    pn, _, _ = O.adamw_ref(p, z, z, z, lr=0.5, weight_decay=0.1, beta1=0.9, beta2=0.95, eps=1e-8, step=3)
    assert abs(pn[0] - 2.85) < 1e-15
    with pytest.raises(ValueError):
        O.adamw_ref(p, z, z, z, lr=0.5, weight_decay=0.1, beta1=0.9, beta2=0.95, eps=1e-8, step=0)


def test_adamw_tenth_step_hand_value():
    # m0 = 0.2, v0 = 0.04, g = -0.1, b1 = 0.9, b2 = 0.95, t = 10, lr = 1, wd = 0
    # m = 0.18 - 0.01 = 0.17 ; v = 0.038 + 0.0005 = 0.0385
    pn, m, v = O.adamw_ref(np.zeros(1), np.array([-0.1]), np.array([0.2]), np.array([0.04]),
                           lr=1.0, weight_decay=0.0, beta1=0.9, beta2=0.95, eps=0.0, step=10)
    assert abs(m[0] - 0.17) < 1e-15 and abs(v[0] - 0.0385) < 1e-15
    bc1 = 1 - 0.9 ** 10
    bc2 = 1 - 0.95 ** 10
    assert abs(pn[0] + (0.17 / bc1) / math.sqrt(0.0385 / bc2)) < 1e-14


# --------------------------------------------------------------------------
# bfloat16 rounding against torch's cast (a library routine)
# --------------------------------------------------------------------------

def test_bf16_round_matches_torch():
    torch = pytest.importorskip("torch")
    rng = _rng(14)
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
        np.array([0.0, -0.0, 1.0, 1.00390625, 1.005859375, 1.0029296875, 3.4e38, -3.4e38, 1e-39, 2e-45]),
    ]).astype(np.float32).astype(np.float64)
    want = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.bf16_round(x)
    assert np.array_equal(got, want)
    assert np.isnan(O.bf16_round(np.array([np.nan]))[0])
    assert O.bf16_round(np.array([1e39]))[0] == np.inf


def test_bf16_round_ties_to_even():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties go to the even mantissa (1.0)
    assert O.bf16_round(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    # 1 + 3 * 2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: goes to 1 + 2^-6
    assert O.bf16_round(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6
    # just above a tie rounds up (a double value that binary32 cannot hold)
    assert O.bf16_round(np.array([1.0 + 2.0 ** -8 + 2.0 ** -40]))[0] == 1.0 + 2.0 ** -7


# --------------------------------------------------------------------------
# Whole step: composition of the stages
# --------------------------------------------------------------------------

def test_muon_step_composes_stages():
    rng = _rng(15)
    w, g, m = (rng.standard_normal((8, 20)) for _ in range(3))
    r = O.muon_step_ref(w, g, m, lr=0.02, weight_decay=0.01, heads=2, scale=1.5)
    m_new, u = O.momentum_ref(g, m)
    o, norms = O.orthogonalize_ref(u, heads=2)
    assert np.array_equal(r["m"], m_new) and np.array_equal(r["o"], o)
    assert np.array_equal(r["norms"], norms)
    assert np.array_equal(r["w"], w - 0.02 * 0.01 * w - 0.02 * 1.5 * o)


def test_golden_regression_fixture():
    """Oracle outputs on a fixed small input, written by tests/golden/make_golden.py."""
    path = os.path.join(GOLDEN, "oracle_small_step.npz")
    data = np.load(path)
    r = O.muon_step_ref(data["w"], data["g"], data["m"], lr=0.02, weight_decay=0.01, heads=2,
                        mu=0.95, nesterov=True, scale=1.0)
    assert np.allclose(r["w"], data["w_new"], rtol=0, atol=1e-15)
    assert np.allclose(r["o"], data["o"], rtol=0, atol=1e-14)
    assert np.allclose(r["m"], data["m_new"], rtol=0, atol=1e-15)


# ---------------------------------------------------------------------------
# QK-Clip (MuonClip Optimizer page, "QK-Clip"): per-head rescale of the query
# and key weights when the head's largest logit magnitude exceeds tau.
# ---------------------------------------------------------------------------

def test_qk_clip_hand_values():
    """Two heads, tau 100: max logits 50 (kept) and 200 (gamma 0.5, exact)."""
    wq = np.arange(1, 9, dtype=np.float32).reshape(4, 2)
    wk = -np.arange(1, 9, dtype=np.float32).reshape(4, 2)
    q, k, g = O.qk_clip_ref(wq, wk, [50.0, 200.0], q_heads=2, k_heads=2, tau=100.0)
    assert g.tolist() == [1.0, 0.5]
    assert q.tolist() == [[1, 2], [3, 4], [2.5, 3], [3.5, 4]]
    assert k.tolist() == [[-1, -2], [-3, -4], [-2.5, -3], [-3.5, -4]]


def test_qk_clip_bounds_the_logits():
    """With equal head counts, scaling Wq and Wk of a head by gamma scales its
    logits (x Wq_h^T)(x Wk_h^T)^T by gamma^2: a clipped head's new largest logit
    is tau^2 / max_logit < tau, recomputed here from synthetic activations."""
    rng = np.random.default_rng(5)
    heads, dh, d, tokens = 4, 8, 32, 16
    x = rng.standard_normal((tokens, d))
    wq = (rng.standard_normal((heads * dh, d)) * 2.0).astype(np.float32)
    wk = (rng.standard_normal((heads * dh, d)) * 2.0).astype(np.float32)

    def max_logits(a, b):
        out = []
        for sl in O.head_blocks(heads * dh, heads):
            lg = (x @ a[sl].astype(np.float64).T) @ (x @ b[sl].astype(np.float64).T).T
            out.append(np.abs(lg).max())
        return np.array(out)

    ml = max_logits(wq, wk)
    tau = float(np.median(ml))            # about half the heads are clipped
    q, k, g = O.qk_clip_ref(wq, wk, ml, q_heads=heads, k_heads=heads, tau=tau)
    after = max_logits(q, k)
    for h in range(heads):
        if ml[h] > np.float32(tau):
            assert after[h] == pytest.approx(float(g[h]) ** 2 * ml[h], rel=2e-6)
            assert after[h] < tau
        else:
            assert after[h] == ml[h]


def test_qk_clip_grouped_query_heads_take_the_group_minimum():
    """Four query heads sharing two key heads: key head g takes the smallest
    gamma of query heads 2g and 2g+1."""
    wq = np.ones((8, 3), dtype=np.float32)
    wk = np.ones((4, 3), dtype=np.float32)
    ml = [125.0, 90.0, 400.0, 200.0]
    q, k, g = O.qk_clip_ref(wq, wk, ml, q_heads=4, k_heads=2, tau=100.0)
    f08 = np.float32(0.8)                 # 100 / 125 in float32
    np.testing.assert_array_equal(g, np.array([f08, 1.0, 0.25, 0.5], dtype=np.float32))
    np.testing.assert_array_equal(q[:, 0], np.array([f08, f08, 1, 1, 0.25, 0.25, 0.5, 0.5], dtype=np.float32))
    np.testing.assert_array_equal(k[:, 0], np.array([f08, f08, 0.25, 0.25], dtype=np.float32))


def test_qk_clip_equal_heads_is_the_page_rule():
    """With one key head per query head every head uses its own gamma."""
    rng = np.random.default_rng(6)
    wq = rng.standard_normal((6, 5)).astype(np.float32)
    wk = rng.standard_normal((6, 5)).astype(np.float32)
    ml = np.array([30.0, 101.0, 1e4], dtype=np.float32)
    q, k, g = O.qk_clip_ref(wq, wk, ml, q_heads=3, k_heads=3, tau=100.0)
    for h in range(3):
        s = slice(2 * h, 2 * h + 2)
        want = np.float32(100.0) / ml[h] if ml[h] > 100 else np.float32(1.0)
        assert g[h] == want
        np.testing.assert_array_equal(q[s], want * wq[s] if want != 1 else wq[s])
        np.testing.assert_array_equal(k[s], want * wk[s] if want != 1 else wk[s])


def test_qk_clip_nan_keeps_and_inf_zeroes():
    wq = np.full((2, 2), 3.0, dtype=np.float32)
    wk = np.full((2, 2), -3.0, dtype=np.float32)
    q, k, g = O.qk_clip_ref(wq, wk, [np.nan, np.inf], q_heads=2, k_heads=2)
    assert g[0] == 1.0 and g[1] == 0.0
    assert q[0].tolist() == [3.0, 3.0] and k[0].tolist() == [-3.0, -3.0]
    assert np.all(q[1] == 0) and np.all(k[1] == 0)
