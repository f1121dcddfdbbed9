"""Tensor-level calls over the C ABI: one Muon step, orthogonalise-only, AdamW.

Each function marshals torch tensors into the library's descriptor lists,
allocates the workspace the library asks for (unless one is passed in) and
enqueues the work on `stream` (default: the current stream). A workspace
allocated here on the current stream is recorded on `stream` when that is
another stream, so the caching allocator does not reuse it while the library's
kernels still read it. Nothing here computes.
"""

from __future__ import annotations

from typing import Optional, Sequence

import torch

from . import _lib


def muon_step(params: Sequence[torch.Tensor], grads: Sequence[torch.Tensor], moms: Sequence[torch.Tensor], *,
              lr: float, weight_decay: float, mu: float = 0.95, nesterov: bool = True,
              heads: Optional[Sequence[int]] = None, scales: Optional[Sequence[float]] = None,
              ns_steps: int = 5, coeffs=None, precision: str = "bf16", norm_eps: float = 1e-7,
              norm_outs: Optional[Sequence[torch.Tensor]] = None,
              ortho_outs: Optional[Sequence[Optional[torch.Tensor]]] = None,
              workspace: Optional[torch.Tensor] = None, stream=None, noalloc: bool = False,
              cautious_wd: bool = False) -> None:
    """In-place Muon step over 2-D params (momentum fp32, grads in the param dtype).

    noalloc=True runs mu_muon_step_noalloc: no workspace is allocated, the
    library's static per-GPU scratch (MU_NOALLOC_SCRATCH_BYTES) is used, and
    calls on one GPU must not overlap in time. cautious_wd=True applies the
    decay only where it agrees in sign with the update (see the header)."""
    mats, n = _lib.matrices(params, grads, moms, heads, scales, norm_outs, ortho_outs)
    hp, keep = _lib.muon_hparams(lr, weight_decay, mu, nesterov, norm_eps, ns_steps, coeffs, precision, cautious_wd)
    if n == 0:
        return
    if noalloc:
        if workspace is not None:
            raise ValueError("noalloc=True takes no workspace")
        _lib.mu_muon_step_noalloc(mats, n, hp, stream)
        del keep
        return
    if workspace is None:
        workspace = _lib.workspace(_lib.mu_muon_workspace_size(mats, n, hp), params[0].device)
        _lib.tie_to_stream(workspace, stream)
    _lib.mu_muon_step(mats, n, hp, workspace, stream)
    del keep


def muon_workspace_bytes(params, grads, moms, *, heads=None, ns_steps: int = 5, coeffs=None,
                         precision: str = "bf16") -> int:
    mats, n = _lib.matrices(params, grads, moms, heads)
    hp, keep = _lib.muon_hparams(0.0, 0.0, 0.95, True, 1e-7, ns_steps, coeffs, precision)
    return _lib.mu_muon_workspace_size(mats, n, hp)


def orthogonalize(inputs: Sequence[torch.Tensor], *, heads: Optional[Sequence[int]] = None, ns_steps: int = 5,
                  coeffs=None, precision: str = "bf16", norm_eps: float = 1e-7,
                  outputs: Optional[Sequence[torch.Tensor]] = None,
                  norm_outs: Optional[Sequence[torch.Tensor]] = None,
                  workspace: Optional[torch.Tensor] = None, stream=None):
    """Frobenius-normalise and Newton-Schulz-orthogonalise each input (per head)."""
    if outputs is None:
        outputs = [torch.empty_like(x) for x in inputs]
    xs, n = _lib.orthos(inputs, outputs, heads, norm_outs)
    hp, keep = _lib.muon_hparams(0.0, 0.0, 0.95, True, norm_eps, ns_steps, coeffs, precision)
    if n == 0:
        return list(outputs)
    if workspace is None:
        workspace = _lib.workspace(_lib.mu_ortho_workspace_size(xs, n, hp), inputs[0].device)
        _lib.tie_to_stream(workspace, stream)
    _lib.mu_muon_orthogonalize(xs, n, hp, workspace, stream)
    del keep
    return list(outputs)


def adamw_step(params, grads, exp_avgs, exp_avg_sqs, *, lr, weight_decay, beta1: float = 0.9,
               beta2: float = 0.95, eps: float = 1e-8, step: int = 1,
               workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """In-place AdamW step over a flat list; lr and weight_decay may be per-tensor lists."""
    n = len(params)
    lrs = list(lr) if isinstance(lr, (list, tuple)) else [lr] * n
    wds = list(weight_decay) if isinstance(weight_decay, (list, tuple)) else [weight_decay] * n
    ts, n = _lib.tensors(params, grads, exp_avgs, exp_avg_sqs, lrs, wds)
    if n == 0:
        return
    if workspace is None:
        workspace = _lib.workspace(_lib.mu_adamw_workspace_size(n), params[0].device)
        _lib.tie_to_stream(workspace, stream)
    _lib.mu_adamw_step(ts, n, beta1, beta2, eps, step, workspace, stream)


def qk_clip(wqs, wks, max_logits, *, q_heads, k_heads, tau: float = 100.0, gamma_outs=None,
            workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """QK-Clip over attention layers (one (wq, wk, max_logit) per layer): heads
    whose max |logit| exceeds tau get their query and key rows scaled by
    tau / max_logit, in place. q_heads / k_heads are per layer (or one int)."""
    n = len(wqs)
    qh = list(q_heads) if isinstance(q_heads, (list, tuple)) else [q_heads] * n
    kh = list(k_heads) if isinstance(k_heads, (list, tuple)) else [k_heads] * n
    pairs, n = _lib.qk_pairs(wqs, wks, max_logits, qh, kh, gamma_outs)
    if n == 0:
        return
    if workspace is None:
        workspace = _lib.workspace(_lib.mu_qk_clip_workspace_size(pairs, n), wqs[0].device)
        _lib.tie_to_stream(workspace, stream)
    _lib.mu_qk_clip(pairs, n, tau, workspace, stream)
