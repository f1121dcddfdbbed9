"""GPU tests of the torch.optim wrapper MuonAdamW on a small transformer-shaped
model: routing through split_params, one step against the oracle (float32
path) and against the functional calls (bitwise), and a checkpoint round trip
through state_dict() / load_state_dict() that must continue bit for bit.
"""

import copy

import numpy as np
import pytest
import torch

from gpu_util import need_gpu, to_np
from oracle import muon_oracle as O
from workloads import host_normal

pytestmark = pytest.mark.gpu

F32_TOL = 1e-4
LR, WD, ALR, AWD, BETAS, EPS = 0.02, 0.01, 3e-3, 0.01, (0.9, 0.95), 1e-8


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    import newton_schulz_orthogonalized_amd as nso  # noqa: F401  (fails loudly without the library)
    yield


class Block(torch.nn.Module):
    def __init__(self, d):
        super().__init__()
        self.ln = torch.nn.LayerNorm(d)
        self.qkv = torch.nn.Linear(d, 3 * d, bias=False)   # tall: 3d x d
        self.proj = torch.nn.Linear(d, d, bias=False)
        self.up = torch.nn.Linear(d, 4 * d, bias=True)
        self.down = torch.nn.Linear(4 * d, d, bias=False)  # wide: d x 4d


class Tiny(torch.nn.Module):
    def __init__(self, vocab=97, d=64, layers=2):
        super().__init__()
        self.wte = torch.nn.Embedding(vocab, d)
        self.blocks = torch.nn.ModuleList([Block(d) for _ in range(layers)])
        self.lm_head = torch.nn.Linear(d, vocab, bias=False)


def _model(dtype, seed=0):
    torch.manual_seed(seed)
    m = Tiny().to(device="cuda", dtype=dtype)
    for i, p in enumerate(m.parameters()):   # seeded, synthetic weights
        p.data.copy_(torch.from_numpy(host_normal(tuple(p.shape), 31000 + i, 0.02)).to(p.device, dtype))
    return m


def _set_grads(model, step):
    for i, p in enumerate(model.parameters()):
        p.grad = torch.from_numpy(host_normal(tuple(p.shape), 32000 + 100 * step + i, 1e-3)).to(p.device, p.dtype)


def _opt(model, precision):
    import newton_schulz_orthogonalized_amd as nso
    muon, adamw = nso.split_params(model)
    return nso.MuonAdamW([{"params": muon, "kind": "muon"}, {"params": adamw, "kind": "adamw"}], lr=LR,
                         weight_decay=WD, adamw_lr=ALR, adamw_weight_decay=AWD, betas=BETAS, eps=EPS,
                         precision=precision)


def test_routing_of_the_tiny_model():
    import newton_schulz_orthogonalized_amd as nso
    model = _model(torch.float32)
    muon, adamw = nso.split_params(model)
    names = {id(p): n for n, p in model.named_parameters()}
    assert sorted(names[id(p)].split(".")[-2] for p in muon) == sorted(["qkv", "proj", "up", "down"] * 2)
    for p in adamw:
        n = names[id(p)]
        assert p.dim() < 2 or n.startswith("wte") or n.startswith("lm_head"), n


def test_one_step_matches_the_oracle_f32():
    import newton_schulz_orthogonalized_amd as nso
    model = _model(torch.float32)
    opt = _opt(model, "f32")
    before = {n: to_np(p.detach()) for n, p in model.named_parameters()}
    _set_grads(model, 0)
    grads = {n: to_np(p.grad) for n, p in model.named_parameters()}
    opt.step()
    torch.cuda.synchronize()
    muon, _ = nso.split_params(model)
    muon_ids = {id(p) for p in muon}
    for n, p in model.named_parameters():
        w0, g0 = before[n], grads[n]
        if id(p) in muon_ids:
            ref = O.muon_step_ref(w0, g0, np.zeros_like(w0), lr=LR, weight_decay=WD)
            assert O.rel_fro(to_np(p.detach()) - w0, ref["w"] - w0) <= F32_TOL, n
            assert O.rel_fro(to_np(opt.state[p]["momentum_buffer"]), ref["m"]) <= 1e-6, n
        else:
            pr, mr, vr = O.adamw_ref(w0, g0, np.zeros_like(w0), np.zeros_like(w0), lr=ALR, weight_decay=AWD,
                                     beta1=BETAS[0], beta2=BETAS[1], eps=EPS, step=1)
            assert O.rel_fro(to_np(p.detach()) - w0, pr - w0) <= F32_TOL, n
            assert opt.state[p]["step"] == 1


@pytest.mark.parametrize("dtype,precision", [(torch.bfloat16, "bf16"), (torch.float32, "f32")])
def test_one_step_equals_the_functional_calls(dtype, precision):
    import newton_schulz_orthogonalized_amd as nso
    a, b = _model(dtype), _model(dtype)
    opt = _opt(a, precision)
    _set_grads(a, 0)
    _set_grads(b, 0)
    opt.step()
    muon, adamw = nso.split_params(b)
    moms = [torch.zeros(p.shape, dtype=torch.float32, device="cuda") for p in muon]
    nso.muon_step([p.data for p in muon], [p.grad for p in muon], moms, lr=LR, weight_decay=WD, precision=precision)
    ms = [torch.zeros(p.shape, dtype=torch.float32, device="cuda") for p in adamw]
    vs = [torch.zeros(p.shape, dtype=torch.float32, device="cuda") for p in adamw]
    nso.adamw_step([p.data for p in adamw], [p.grad for p in adamw], ms, vs, lr=ALR, weight_decay=AWD,
                   beta1=BETAS[0], beta2=BETAS[1], eps=EPS, step=1)
    torch.cuda.synchronize()
    for (n, pa), pb in zip(a.named_parameters(), b.parameters()):
        assert torch.equal(pa, pb), n


def test_checkpoint_round_trip_continues_bitwise():
    """k steps, state_dict() to the host and into a fresh optimizer over a copy
    of the parameters, one more step: equal, bit for bit, to k+1 steps."""
    k = 3
    a = _model(torch.bfloat16)
    opt_a = _opt(a, "bf16")
    for s in range(k):
        _set_grads(a, s)
        opt_a.step()
    torch.cuda.synchronize()
    state = copy.deepcopy(opt_a.state_dict())
    state = {"state": {i: {key: (v.cpu() if torch.is_tensor(v) else v) for key, v in st.items()}
                       for i, st in state["state"].items()},
             "param_groups": state["param_groups"]}
    b = _model(torch.bfloat16)
    b.load_state_dict(a.state_dict())
    opt_b = _opt(b, "bf16")
    opt_b.load_state_dict(state)
    _set_grads(a, k)
    _set_grads(b, k)
    opt_a.step()
    opt_b.step()
    torch.cuda.synchronize()
    for (n, pa), pb in zip(a.named_parameters(), b.parameters()):
        assert torch.equal(pa, pb), n
        sa, sb = opt_a.state[pa], opt_b.state[pb]
        for key in sa:
            if torch.is_tensor(sa[key]):
                assert torch.equal(sa[key], sb[key].to(sa[key].device)), (n, key)
            else:
                assert sa[key] == sb[key], (n, key)
