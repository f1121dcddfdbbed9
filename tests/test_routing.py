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


def test_load_state_dict_keeps_float32_state_for_bf16_weights():
    """torch casts floating-point optimizer state to the parameter dtype on
    load; the momentum and moment buffers must stay float32 (exact values)."""
    import newton_schulz_orthogonalized_amd as nso
    w = torch.nn.Parameter(torch.zeros(8, 16, dtype=torch.bfloat16))
    b = torch.nn.Parameter(torch.zeros(16, dtype=torch.bfloat16))
    opt = nso.MuonAdamW([{"params": [w], "kind": "muon"}, {"params": [b], "kind": "adamw"}])
    mom = torch.linspace(-1, 1, 128, dtype=torch.float32).reshape(8, 16) / 3.0   # not representable in bf16
    ea = torch.linspace(0, 1, 16, dtype=torch.float32) / 7.0
    sd = {"state": {0: {"momentum_buffer": mom.clone()},
                    1: {"step": 4, "exp_avg": ea.clone(), "exp_avg_sq": ea.clone() ** 2}},
          "param_groups": opt.state_dict()["param_groups"]}
    opt.load_state_dict(sd)
    st_w, st_b = opt.state[w], opt.state[b]
    assert st_w["momentum_buffer"].dtype == torch.float32 and torch.equal(st_w["momentum_buffer"], mom)
    assert st_b["exp_avg"].dtype == torch.float32 and torch.equal(st_b["exp_avg"], ea)
    assert torch.equal(st_b["exp_avg_sq"], ea ** 2) and st_b["step"] == 4
    assert st_w["momentum_buffer"].data_ptr() != sd["state"][0]["momentum_buffer"].data_ptr()
