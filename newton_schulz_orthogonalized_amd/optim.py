"""torch.optim wrapper: parameter routing and optimizer state around the C ABI.

Routing (nanochat optimizer page, "Parameter Grouping Strategy"; issue page
"Guidelines for whether to use muon for parameters"): hidden weights with two
or more dimensions take the Muon step; tensors with fewer than two dimensions,
and the embedding and output head, take AdamW. Each parameter group carries a
``kind`` of "muon" or "adamw" and step() sends each kind to one library call
per distinct set of hyper-parameters (nanochat optimizer page, "The MuonAdamW
Class Architecture").

State lives here as torch tensors (momentum_buffer for Muon; exp_avg,
exp_avg_sq and step for AdamW), so state_dict()/load_state_dict() work as for
any torch optimizer. The library holds no state between calls.
"""

from __future__ import annotations

from typing import Dict, Iterable, List, Tuple

import torch

from . import _lib

NON_HIDDEN_NAME_PARTS = ("embed", "wte", "wpe", "lm_head", "unembed", "output_head")


def split_params(model: torch.nn.Module, non_hidden: Iterable[str] = NON_HIDDEN_NAME_PARTS) -> Tuple[list, list]:
    """(muon_params, adamw_params) of a model by the routing rule.

    Parameters of nn.Embedding modules and parameters whose name contains one of
    `non_hidden` are embeddings/heads and go to AdamW, as do all tensors with
    fewer than two dimensions; every other parameter goes to Muon.
    """
    emb = set()
    for mod in model.modules():
        if isinstance(mod, torch.nn.Embedding):
            emb.update(id(p) for p in mod.parameters(recurse=False))
    muon, adamw = [], []
    for name, p in model.named_parameters():
        if not p.requires_grad:
            continue
        is_nh = id(p) in emb or any(part in name.lower() for part in non_hidden)
        (muon if (p.dim() >= 2 and not is_nh) else adamw).append(p)
    return muon, adamw


class MuonAdamW(torch.optim.Optimizer):
    """Muon for groups with kind="muon", AdamW for kind="adamw".

    Muon group options: lr, weight_decay, momentum (mu), nesterov, ns_steps,
    coeffs (per-step (a, b, c) or None for the cubic step), precision
    ("bf16" | "f32"), norm_eps, num_heads (int, or a callable p -> int),
    scale (float, or a callable p -> float; 1.0 is plain Muon) and cautious_wd
    (decay only where it agrees in sign with the update).
    AdamW group options: lr, weight_decay, betas, eps.
    Tensors with more than two dimensions are orthogonalised as
    [shape[0], prod(shape[1:])] matrices.
    """

    def __init__(self, param_groups: List[Dict], *, lr: float = 0.02, weight_decay: float = 0.0,
                 momentum: float = 0.95, nesterov: bool = True, ns_steps: int = 5, coeffs=None,
                 precision: str = "bf16", norm_eps: float = 1e-7, num_heads=1, scale=1.0, cautious_wd: bool = False,
                 adamw_lr: float = 3e-4, betas=(0.9, 0.95), eps: float = 1e-8, adamw_weight_decay: float = 0.0):
        groups = []
        for g in param_groups:
            g = dict(g)
            kind = g.get("kind")
            if kind not in ("muon", "adamw"):
                raise ValueError("every parameter group needs kind='muon' or kind='adamw'")
            if kind == "muon":
                for k, v in (("lr", lr), ("weight_decay", weight_decay), ("momentum", momentum),
                             ("nesterov", nesterov), ("ns_steps", ns_steps), ("coeffs", coeffs),
                             ("precision", precision), ("norm_eps", norm_eps), ("num_heads", num_heads),
                             ("scale", scale), ("cautious_wd", cautious_wd)):
                    g.setdefault(k, v)
            else:
                for k, v in (("lr", adamw_lr), ("weight_decay", adamw_weight_decay), ("betas", betas),
                             ("eps", eps)):
                    g.setdefault(k, v)
            groups.append(g)
        super().__init__(groups, {})
        self._workspaces: Dict[tuple, torch.Tensor] = {}

    # float32 state of both rules (the library reads and writes it as float32)
    _F32_STATE = ("momentum_buffer", "exp_avg", "exp_avg_sq")

    def load_state_dict(self, state_dict):
        """torch's load_state_dict, except that the momentum and moment buffers
        stay float32: torch casts floating-point state to each parameter's dtype
        (bfloat16 for bf16 weights), which would lose their precision."""
        saved = state_dict["state"]
        super().load_state_dict(state_dict)
        params = [p for g in self.param_groups for p in g["params"]]
        for idx, st in saved.items():
            p = params[idx]
            for key in self._F32_STATE:
                v = st.get(key)
                if torch.is_tensor(v):
                    self.state[p][key] = v.to(device=p.device, dtype=torch.float32, copy=True).contiguous()

    def _ws(self, key, nbytes, device):
        if nbytes == 0:
            return None
        ws = self._workspaces.get(key)
        if ws is None or ws.numel() < nbytes or ws.device != device:
            ws = _lib.workspace(nbytes, device)
            self._workspaces[key] = ws
        return ws

    @torch.no_grad()
    def step(self, closure=None):
        loss = None
        if closure is not None:
            with torch.enable_grad():
                loss = closure()
        for g in self.param_groups:
            if g["kind"] == "muon":
                self._step_muon(g)
            else:
                self._step_adamw(g)
        return loss

    def _step_muon(self, g):
        ps, gs, ms, heads, scales = [], [], [], [], []
        for p in g["params"]:
            if p.grad is None:
                continue
            if p.dim() < 2:
                raise ValueError("a Muon group holds a tensor with fewer than two dimensions")
            st = self.state[p]
            if "momentum_buffer" not in st:
                st["momentum_buffer"] = torch.zeros_like(p, dtype=torch.float32, memory_format=torch.contiguous_format)
            w2 = p.view(p.shape[0], -1)
            grad = p.grad if p.grad.is_contiguous() else p.grad.contiguous()
            ps.append(w2)
            gs.append(grad.view(p.shape[0], -1))
            ms.append(st["momentum_buffer"].view(p.shape[0], -1))
            h = g["num_heads"]
            heads.append(int(h(p) if callable(h) else h))
            s = g["scale"]
            scales.append(float(s(p) if callable(s) else s))
        if not ps:
            return
        mats, n = _lib.matrices(ps, gs, ms, heads, scales)
        hp, keep = _lib.muon_hparams(g["lr"], g["weight_decay"], g["momentum"], g["nesterov"], g["norm_eps"],
                                     g["ns_steps"], g["coeffs"], g["precision"], g.get("cautious_wd", False))
        need = _lib.mu_muon_workspace_size(mats, n, hp)
        ws = self._ws(("muon", id(g)), need, ps[0].device)
        _lib.mu_muon_step(mats, n, hp, ws)
        del keep

    def _step_adamw(self, g):
        batches: Dict[int, list] = {}
        for p in g["params"]:
            if p.grad is None:
                continue
            st = self.state[p]
            if "step" not in st:
                st["step"] = 0
                st["exp_avg"] = torch.zeros_like(p, dtype=torch.float32, memory_format=torch.contiguous_format)
                st["exp_avg_sq"] = torch.zeros_like(p, dtype=torch.float32, memory_format=torch.contiguous_format)
            st["step"] += 1
            grad = p.grad if p.grad.is_contiguous() else p.grad.contiguous()
            batches.setdefault(int(st["step"]), []).append((p, grad, st["exp_avg"], st["exp_avg_sq"]))
        b1, b2 = g["betas"]
        for t, items in batches.items():
            ts, n = _lib.tensors([x[0] for x in items], [x[1] for x in items], [x[2] for x in items],
                                 [x[3] for x in items], [g["lr"]] * len(items), [g["weight_decay"]] * len(items))
            ws = self._ws(("adamw", id(g), len(items)), _lib.mu_adamw_workspace_size(n), items[0][0].device)
            _lib.mu_adamw_step(ts, n, b1, b2, g["eps"], t, ws)
