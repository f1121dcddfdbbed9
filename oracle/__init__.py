"""CPU oracle (test infrastructure only; see muon_oracle.py)."""
from .muon_oracle import *  # noqa: F401,F403
from .muon_oracle import (adamw_ref, bf16_round, default_coeffs, frobenius_normalize_ref,  # noqa: F401
                          head_blocks, momentum_ref, muon_step_ref, muon_update_ref,
                          newton_schulz_ref, ns_spectral_ref, orthogonalize_ref, rel_fro,
                          qk_clip_ref, route_ref, CUBIC, DEFAULT_MU, DEFAULT_NS_STEPS, DEFAULT_NORM_EPS,
                          DEFAULT_QK_TAU)
