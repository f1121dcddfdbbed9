"""MI355X-native Muon optimizer step (momentum, Frobenius normalisation,
Newton-Schulz orthogonalisation, decoupled-weight-decay update) and fused
AdamW, on hand-written gfx950 HIP kernels behind a C ABI.

The HIP library is loaded on first use of any compute entry point; a missing
library raises ImportError (there is no CPU fallback).
"""

__all__ = ["muon_step", "orthogonalize", "adamw_step", "qk_clip", "muon_workspace_bytes", "MuonAdamW", "split_params"]


def __getattr__(name):
    if name in ("muon_step", "orthogonalize", "adamw_step", "qk_clip", "muon_workspace_bytes"):
        from . import api
        return getattr(api, name)
    if name in ("MuonAdamW", "split_params"):
        from . import optim
        return getattr(optim, name)
    raise AttributeError(name)
