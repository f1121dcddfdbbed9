"""Parameter routing (CPU): hidden matrices to Muon, the rest to AdamW."""

import torch

from oracle import muon_oracle as O


class Tiny(torch.nn.Module):
    def __init__(self):
        super().__init__()
        self.wte = torch.nn.Embedding(50, 16)
        self.attn = torch.nn.Linear(16, 48)
        self.proj = torch.nn.Linear(16, 16, bias=False)
        self.norm = torch.nn.LayerNorm(16)
        self.conv = torch.nn.Conv1d(4, 8, 3)
        self.lm_head = torch.nn.Linear(16, 50, bias=False)
        self.gain = torch.nn.Parameter(torch.ones(()))


def test_split_params_follows_the_routing_rule():
    from newton_schulz_orthogonalized_amd.optim import split_params
    m = Tiny()
    muon, adamw = split_params(m)
    ids_m = {id(p) for p in muon}
    for name, p in m.named_parameters():
        non_hidden = name.startswith("wte") or name.startswith("lm_head")
        want = O.route_ref(p.dim(), non_hidden)
        assert (id(p) in ids_m) == (want == "muon"), name
    assert {id(m.attn.weight), id(m.proj.weight), id(m.conv.weight)} == ids_m
