"""Plain CPU oracle for the Muon optimizer step and the AdamW step.

TEST INFRASTRUCTURE ONLY. Nothing in the library imports or calls this module;
only the test-suite, the smoke check in ``__graft_entry__`` and the CPU-baseline
leg of ``bench.py`` may use it. It shares no code with the HIP path.

Everything is computed in float64 with numpy, step by step, in the order the
pages give, with no blocking, fusion or reordering:

* momentum: an exponential moving average with decay 0.95 (MuonClip Optimizer
  page, sections "Momentum" and "Design Decisions"); a Nesterov blend is named
  on the nanochat optimizer page ("Muon Step Implementation") and as the
  ``nesterov`` flag of ``_prepare`` on the NeMo AutoModel muown_triton page,
  but defined on neither; the reading used here is written at ``momentum_ref``;
* Frobenius normalisation of each (matrix, head) block before the iteration;
* Newton-Schulz: a fixed number of steps of X <- a X + b X (X^T X), default
  five steps with (a, b) = (1.5, -0.5) (MuonClip Optimizer page, section
  "Newton-Schulz Orthogonalization"); per-step coefficients and an optional
  quintic term c X (X^T X)^2 are the configurable extension;
* per-head orthogonalisation: each head's block of rows is handled as its own
  matrix (Qwen training-details page, section "Confirmed");
* the decoupled-weight-decay parameter update;
* AdamW with bias correction for the tensors routed away from Muon (nanochat
  optimizer page, "Parameter Grouping Strategy" and "AdamW Step
  Implementation"; the bias-correction scalars appear as runtime arguments of
  ``_finish_kernel`` on the NeMo AutoModel muown_triton page);
* QK-Clip, the post-update rescale of attention query/key weights (MuonClip
  Optimizer page, "QK-Clip").

Parity of each function is pinned in ``tests/test_oracle.py`` against closed
forms, library routines (LAPACK SVD, torch's bfloat16 cast) and brute force.
"""

from __future__ import annotations

import math
from typing import Iterable, Sequence

import numpy as np

# Momentum decay 0.95: MuonClip Optimizer page, "Momentum" / "Design Decisions".
DEFAULT_MU = 0.95
# Five iterations, "empirically sufficient": MuonClip page, "Design Decisions".
DEFAULT_NS_STEPS = 5
# Cubic iteration coefficients: MuonClip page, "Newton-Schulz Orthogonalization".
CUBIC = (1.5, -0.5, 0.0)
# Guard added to the Frobenius norm before dividing (a reading; the pages do not
# write the normalisation down at all).
DEFAULT_NORM_EPS = 1e-7


def default_coeffs(steps: int = DEFAULT_NS_STEPS) -> list[tuple[float, float, float]]:
    """The pages' cubic step repeated ``steps`` times."""
    return [CUBIC] * steps


def _as_coeffs(coeffs) -> list[tuple[float, float, float]]:
    out = []
    for c in coeffs:
        c = tuple(float(x) for x in c)
        if len(c) == 2:
            c = (c[0], c[1], 0.0)
        if len(c) != 3:
            raise ValueError("each Newton-Schulz step needs (a, b) or (a, b, c)")
        out.append(c)
    return out


# ----------------------------------------------------------------------------
# bfloat16 rounding (round to nearest, ties to even), used to state what a
# bf16 parameter holds after the update. Written from the IEEE-754 layout:
# bfloat16 keeps the sign, the 8 exponent bits and the top 7 mantissa bits of a
# binary32 value.
# ----------------------------------------------------------------------------

def bf16_round(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (ties to even).

    The rounding is done once, from float64, at bit 45 of the float64 mantissa
    (52 - 7). Values whose magnitude lies in the binary32 subnormal range are
    first rounded to binary32; NaN stays NaN and overflow gives +-inf.
    """
    a = np.asarray(x, dtype=np.float64)
    out = np.empty_like(a)
    flat = a.reshape(-1)
    res = out.reshape(-1)
    small = np.abs(flat) < 2.0 ** -126
    big = ~small
    if np.any(big):
        u = flat[big].view(np.uint64).copy()
        nan = np.isnan(flat[big])
        lsb = (u >> np.uint64(45)) & np.uint64(1)
        u = (u + np.uint64((1 << 44) - 1) + lsb) & ~np.uint64((1 << 45) - 1)
        r = u.view(np.float64)
        r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, r), r)
        r[nan] = np.nan
        res[big] = r
    if np.any(small):
        f = flat[small].astype(np.float32)
        u = f.view(np.uint32).astype(np.uint64)
        lsb = (u >> np.uint64(16)) & np.uint64(1)
        u = ((u + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)).astype(np.uint32)
        res[small] = u.view(np.float32).astype(np.float64)
    return out


# ----------------------------------------------------------------------------
# Muon step, one stage at a time.
# ----------------------------------------------------------------------------

def momentum_ref(grad, momentum, mu: float = DEFAULT_MU, nesterov: bool = True):
    """Momentum update and the vector handed to the orthogonaliser.

    EMA form (MuonClip page, "Momentum"): M <- mu*M + (1 - mu)*G.
    Nesterov reading: U = (1 - mu)*G + mu*M_new, the same EMA step taken once
    more from the updated buffer. It equals (1 - mu) times the sum-form
    Nesterov vector G + mu*M_sum when M_sum = M/(1 - mu), so the orthogonalised
    direction is the same under either convention. Without Nesterov, U = M_new.

    Returns (M_new, U) as float64 arrays.
    """
    g = np.asarray(grad, dtype=np.float64)
    m = np.asarray(momentum, dtype=np.float64)
    m_new = mu * m + (1.0 - mu) * g
    u = (1.0 - mu) * g + mu * m_new if nesterov else m_new.copy()
    return m_new, u


def frobenius_normalize_ref(block, eps: float = DEFAULT_NORM_EPS):
    """X0 = B / (||B||_F + eps). Returns (X0, ||B||_F).

    B = 0 gives X0 = 0 for every eps, eps = 0 included (a reading: the zero
    input has the zero direction, so the step only decays the weight; the
    formula alone would give 0/0 there).
    """
    b = np.asarray(block, dtype=np.float64)
    s = math.sqrt(float(np.sum(b * b)))
    if s == 0.0:
        return np.zeros_like(b), s
    return b / (s + eps), s


def newton_schulz_ref(x, coeffs=None):
    """Newton-Schulz iteration (MuonClip page, "Newton-Schulz Orthogonalization").

    Each step computes X <- a X + b X (X^T X) + c X (X^T X)^2. For a wide X the
    same product is evaluated as (X X^T) X, which is the identical matrix by
    associativity and keeps the Gram matrix on the short side.
    """
    coeffs = default_coeffs() if coeffs is None else _as_coeffs(coeffs)
    x = np.array(x, dtype=np.float64, copy=True)
    wide = x.shape[0] <= x.shape[1]
    for a, b, c in coeffs:
        if wide:
            gram = x @ x.T          # X X^T  (rows x rows)
            y = gram @ x            # (X X^T) X  ==  X (X^T X)
            z = gram @ y if c != 0.0 else 0.0
        else:
            gram = x.T @ x          # X^T X  (cols x cols)
            y = x @ gram            # X (X^T X)
            z = y @ gram if c != 0.0 else 0.0
        x = a * x + b * y + c * z
    return x


def ns_spectral_ref(x, coeffs=None):
    """Closed form of the iteration through the SVD (used as a pin).

    If X = U diag(s) V^T then every step maps each singular value through the
    scalar polynomial p(s) = a s + b s^3 + c s^5 and leaves U, V unchanged.
    """
    coeffs = default_coeffs() if coeffs is None else _as_coeffs(coeffs)
    x = np.asarray(x, dtype=np.float64)
    u, s, vt = np.linalg.svd(x, full_matrices=False)
    for a, b, c in coeffs:
        s = a * s + b * s ** 3 + c * s ** 5
    return (u * s) @ vt


def head_blocks(rows: int, heads: int) -> list[slice]:
    """Row blocks of the per-head split: ``heads`` equal contiguous blocks."""
    if heads < 1 or rows % heads != 0:
        raise ValueError("rows must be a positive multiple of heads")
    h = rows // heads
    return [slice(i * h, (i + 1) * h) for i in range(heads)]


def orthogonalize_ref(u, heads: int = 1, coeffs=None, eps: float = DEFAULT_NORM_EPS):
    """Normalise and orthogonalise each head block of ``u`` independently.

    Returns (O, norms) where norms[h] = ||U_h||_F before normalisation.
    """
    u = np.asarray(u, dtype=np.float64)
    out = np.empty_like(u)
    norms = np.empty(heads, dtype=np.float64)
    for h, sl in enumerate(head_blocks(u.shape[0], heads)):
        x0, s = frobenius_normalize_ref(u[sl], eps)
        out[sl] = newton_schulz_ref(x0, coeffs)
        norms[h] = s
    return out, norms


def muon_update_ref(weight, ortho, lr: float, weight_decay: float, scale: float = 1.0, cautious: bool = False):
    """Decoupled-weight-decay update: W <- W - lr*wd*W - lr*scale*O (both from W_old).

    cautious=True: cautious weight decay, which the nanochat optimizer page
    ("Muon Step Implementation") names without a formula. Reading: the decay
    acts only on the coordinates where it moves the weight the same way as the
    update, i.e. where u = lr*scale*O has the sign of W or is zero:
    W <- W - lr*wd*W*[W*u >= 0] - u. With O = 0 this is the plain decay; where
    every W*u < 0 it is the update without decay.
    """
    w = np.asarray(weight, dtype=np.float64)
    o = np.asarray(ortho, dtype=np.float64)
    if cautious:
        u = lr * scale * o
        return w - lr * weight_decay * w * (w * u >= 0.0) - u
    return w - lr * weight_decay * w - lr * scale * o


def muon_step_ref(weight, grad, momentum, *, lr: float, weight_decay: float,
                  mu: float = DEFAULT_MU, nesterov: bool = True, heads: int = 1,
                  coeffs=None, eps: float = DEFAULT_NORM_EPS, scale: float = 1.0, cautious: bool = False):
    """One Muon step for one 2-D weight, all four stages in order.

    Returns a dict with the new weight ``w`` (float64, before any bf16 cast),
    the new momentum ``m``, the orthogonalised direction ``o``, the per-head
    Frobenius norms ``norms`` and the normalised input ``x0`` of the iteration.
    """
    m_new, u = momentum_ref(grad, momentum, mu, nesterov)
    o, norms = orthogonalize_ref(u, heads, coeffs, eps)
    x0 = np.empty_like(u)
    for sl in head_blocks(u.shape[0], heads):
        x0[sl], _ = frobenius_normalize_ref(u[sl], eps)
    w_new = muon_update_ref(weight, o, lr, weight_decay, scale, cautious)
    return {"w": w_new, "m": m_new, "o": o, "norms": norms, "x0": x0, "u": u}


# ----------------------------------------------------------------------------
# AdamW
# ----------------------------------------------------------------------------

def adamw_ref(param, grad, exp_avg, exp_avg_sq, *, lr: float, weight_decay: float,
              beta1: float, beta2: float, eps: float, step: int):
    """Bias-corrected AdamW with decoupled, lr-scaled weight decay.

    m <- b1 m + (1-b1) g;  v <- b2 v + (1-b2) g^2;
    p <- p - lr*wd*p - lr * (m / (1-b1^t)) / (sqrt(v / (1-b2^t)) + eps),
    with t >= 1 the number of this step. Returns (p, m, v) in float64.
    """
    if step < 1:
        raise ValueError("AdamW step count starts at 1")
    p = np.asarray(param, dtype=np.float64)
    g = np.asarray(grad, dtype=np.float64)
    m = beta1 * np.asarray(exp_avg, dtype=np.float64) + (1.0 - beta1) * g
    v = beta2 * np.asarray(exp_avg_sq, dtype=np.float64) + (1.0 - beta2) * g * g
    m_hat = m / (1.0 - beta1 ** step)
    v_hat = v / (1.0 - beta2 ** step)
    p_new = p - lr * weight_decay * p - lr * m_hat / (np.sqrt(v_hat) + eps)
    return p_new, m, v


# ----------------------------------------------------------------------------
# Routing of parameters between the two rules.
# ----------------------------------------------------------------------------

# QK-Clip threshold: MuonClip Optimizer page, "QK-Clip" and "Design Decisions".
DEFAULT_QK_TAU = 100.0


def qk_clip_ref(wq, wk, max_logit, *, q_heads: int, k_heads: int, tau: float = DEFAULT_QK_TAU):
    """QK-Clip after the update (MuonClip Optimizer page, section "QK-Clip"):
    every attention head whose largest logit magnitude exceeds tau has its
    query and key weights multiplied by gamma = tau / max_logit; other heads are
    left alone.

    Readings where the page is silent:
    * ``max_logit`` is given per query head (measured in the forward pass);
    * gamma is formed in float32 and each weight becomes the float32 product
      gamma * w (the caller rounds it to the weight's dtype);
    * with grouped-query attention (``k_heads`` dividing ``q_heads``) a key
      head takes the smallest gamma of the query heads that share it; with
      ``k_heads == q_heads`` this is the page's per-head rule;
    * a NaN max_logit never exceeds tau (no clip); +inf gives gamma = 0.

    Heads are equal contiguous row blocks of ``wq`` [q_rows, cols] and ``wk``
    [k_rows, cols]. Returns (wq_new, wk_new, gamma_q) in float32.
    """
    wq = np.asarray(wq, dtype=np.float32)
    wk = np.asarray(wk, dtype=np.float32)
    ml = np.asarray(max_logit, dtype=np.float32)
    assert ml.shape == (q_heads,) and q_heads % k_heads == 0
    t = np.float32(tau)
    gamma_q = np.ones(q_heads, dtype=np.float32)
    for h in range(q_heads):
        if ml[h] > t:                      # False for NaN
            with np.errstate(divide="ignore"):
                gamma_q[h] = t / ml[h]     # float32 division; 0 for +inf
    group = q_heads // k_heads
    gamma_k = np.array([gamma_q[g * group:(g + 1) * group].min() for g in range(k_heads)], dtype=np.float32)
    out_q, out_k = wq.copy(), wk.copy()
    for h, sl in enumerate(head_blocks(wq.shape[0], q_heads)):
        if gamma_q[h] != np.float32(1):
            out_q[sl] = gamma_q[h] * wq[sl]      # float32 products
    for g, sl in enumerate(head_blocks(wk.shape[0], k_heads)):
        if gamma_k[g] != np.float32(1):
            out_k[sl] = gamma_k[g] * wk[sl]
    return out_q, out_k, gamma_q


def route_ref(ndim: int, is_embedding_or_head: bool = False) -> str:
    """'muon' for hidden weights with two or more dimensions, else 'adamw'.

    nanochat optimizer page, "Parameter Grouping Strategy": fewer than two
    dimensions go to AdamW, matrices to Muon; issue page "Guidelines for whether
    to use muon for parameters": the embedding and the output head are
    non-hidden and stay with AdamW.
    """
    if is_embedding_or_head:
        return "adamw"
    return "muon" if ndim >= 2 else "adamw"


def rel_fro(x, ref) -> float:
    """Relative Frobenius error ||x - ref||_F / ||ref||_F (0 when both vanish)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = float(np.linalg.norm((x - ref).reshape(-1)))
    r = float(np.linalg.norm(ref.reshape(-1)))
    if r == 0.0:
        return d
    return d / r
