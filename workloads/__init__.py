"""Seeded synthetic inputs and the transformer-shaped parameter sets.

This module holds no arithmetic of the method: it only describes shapes and
draws seeded normal numbers. Both the oracle side and the HIP side of every
test receive the values it produces.

Parameter sets (shapes of the weights; values are synthetic normals):
  fp32_128x256   one float32 128x256 matrix under Muon, one 256-element vector under AdamW
  gpt2_small     12 layers of Wqkv 2304x768, Wo 768x768, MLP 3072x768 and 768x3072 (Muon);
                 LayerNorm gains/biases (50 x 768) and the 50304x768 embedding (AdamW)
  per_head_wq    24 x Wq 4096x4096, 32 heads of 128x4096 each (Muon)
  llama_1b       d=2048, 24 layers: Wq/Wk/Wv/Wo 2048x2048, up 8192x2048, down 2048x8192 (Muon);
                 49 RMSNorm gains of 2048, embedding and unembedding 32768x2048 (AdamW)
  llama_8b       d=4096, 32 layers: Wq/Wo 4096x4096, Wk/Wv 1024x4096, gate/up 14336x4096,
                 down 4096x14336 (Muon); 65 RMSNorm gains of 4096, embedding and
                 unembedding 128256x4096 (AdamW)
Gradients are N(0, 1e-3) (standard deviation), weights N(0, 0.02), momentum
N(0, 1e-3); the fp32_128x256 set draws everything from N(0, 1).
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Tuple

import numpy as np


@dataclass
class MuonEntry:
    name: str
    shape: Tuple[int, int]
    heads: int = 1


@dataclass
class AdamWEntry:
    name: str
    shape: Tuple[int, ...]


@dataclass
class ParamSet:
    name: str
    muon: List[MuonEntry] = field(default_factory=list)
    adamw: List[AdamWEntry] = field(default_factory=list)
    dtype: str = "bf16"          # parameter / gradient dtype
    grad_std: float = 1e-3
    weight_std: float = 0.02
    mom_std: float = 1e-3

    def muon_elems(self) -> int:
        return sum(e.shape[0] * e.shape[1] for e in self.muon)

    def adamw_elems(self) -> int:
        return sum(int(np.prod(e.shape)) for e in self.adamw)

    def ns_flops(self, steps: int = 5, quintic_steps: int = 0) -> float:
        """Algorithmic Newton-Schulz flops: per step m(m+1)n (Gram, symmetric half)
        + 2 m^2 n (apply) + 3 m n (axpy), with m <= n the sides of each head block,
        plus m(m+1)m (A A^T, symmetric half) on each of `quintic_steps` steps."""
        tot = 0.0
        for e in self.muon:
            r, c = e.shape[0] // e.heads, e.shape[1]
            m, n = min(r, c), max(r, c)
            tot += e.heads * steps * (m * (m + 1) * n + 2.0 * m * m * n + 3.0 * m * n)
            tot += e.heads * quintic_steps * (m * (m + 1) * m)
        return tot


def fp32_128x256() -> ParamSet:
    return ParamSet("fp32_128x256", [MuonEntry("w", (128, 256))], [AdamWEntry("b", (256,))], dtype="f32",
                    grad_std=1.0, weight_std=1.0, mom_std=1.0)


def gpt2_small() -> ParamSet:
    ps = ParamSet("gpt2_small")
    for l in range(12):
        ps.muon += [MuonEntry(f"h{l}.attn.c_attn", (2304, 768)), MuonEntry(f"h{l}.attn.c_proj", (768, 768)),
                    MuonEntry(f"h{l}.mlp.c_fc", (3072, 768)), MuonEntry(f"h{l}.mlp.c_proj", (768, 3072))]
    for l in range(12):
        ps.adamw += [AdamWEntry(f"h{l}.ln_1.weight", (768,)), AdamWEntry(f"h{l}.ln_1.bias", (768,)),
                     AdamWEntry(f"h{l}.ln_2.weight", (768,)), AdamWEntry(f"h{l}.ln_2.bias", (768,))]
    ps.adamw += [AdamWEntry("ln_f.weight", (768,)), AdamWEntry("ln_f.bias", (768,)), AdamWEntry("wte", (50304, 768))]
    return ps


def per_head_wq() -> ParamSet:
    return ParamSet("per_head_wq", [MuonEntry(f"l{l}.wq", (4096, 4096), heads=32) for l in range(24)])


def llama_1b() -> ParamSet:
    ps = ParamSet("llama_1b")
    for l in range(24):
        ps.muon += [MuonEntry(f"l{l}.wq", (2048, 2048)), MuonEntry(f"l{l}.wk", (2048, 2048)),
                    MuonEntry(f"l{l}.wv", (2048, 2048)), MuonEntry(f"l{l}.wo", (2048, 2048)),
                    MuonEntry(f"l{l}.up", (8192, 2048)), MuonEntry(f"l{l}.down", (2048, 8192))]
    ps.adamw += [AdamWEntry(f"norm{i}", (2048,)) for i in range(49)]
    ps.adamw += [AdamWEntry("embed", (32768, 2048)), AdamWEntry("unembed", (32768, 2048))]
    return ps


def llama_8b() -> ParamSet:
    ps = ParamSet("llama_8b")
    for l in range(32):
        ps.muon += [MuonEntry(f"l{l}.wq", (4096, 4096)), MuonEntry(f"l{l}.wk", (1024, 4096)),
                    MuonEntry(f"l{l}.wv", (1024, 4096)), MuonEntry(f"l{l}.wo", (4096, 4096)),
                    MuonEntry(f"l{l}.gate", (14336, 4096)), MuonEntry(f"l{l}.up", (14336, 4096)),
                    MuonEntry(f"l{l}.down", (4096, 14336))]
    ps.adamw += [AdamWEntry(f"norm{i}", (4096,)) for i in range(65)]
    ps.adamw += [AdamWEntry("embed", (128256, 4096)), AdamWEntry("unembed", (128256, 4096))]
    return ps


PARAM_SETS = {f.__name__: f for f in (fp32_128x256, gpt2_small, per_head_wq, llama_1b, llama_8b)}


def seed_for(set_index: int, tensor_index: int) -> int:
    """Tensor j of parameter set i draws from seed 1000*i + j (and +500000 per role)."""
    return 1000 * set_index + tensor_index


def host_normal(shape, seed: int, std: float = 1.0) -> np.ndarray:
    """float64 N(0, std) values from numpy's PCG64 with the given seed."""
    return np.random.default_rng(seed).standard_normal(shape) * std


def device_normal(shape, seed: int, std: float, dtype, device):
    """torch N(0, std) drawn on `device` in float32 from a seeded generator, then
    cast to `dtype` (torch's round-to-nearest-even for bfloat16)."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    t.mul_(std)
    return t.to(dtype)


def as_dtype(x: np.ndarray, dtype):
    """A torch CPU tensor of `dtype` holding x (bfloat16: torch's RNE cast from float32)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dtype)
