"""Full-size parity: each transformer-shaped parameter set runs as one Muon call
and one AdamW call over the whole set (the launch configuration bench.py
times), and sampled matrices / tensor slices are compared with the CPU oracle.
O of the sampled matrices comes from the step's optional float32 ortho_out.
"""

import gc

import numpy as np
import pytest
import torch

from gpu_util import bf16_ulp, check_w_against_oracle, need_gpu, tile_rel_fro, to_np
from oracle import muon_oracle as O
from workloads import PARAM_SETS, device_normal, seed_for

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
MOM_TOL = 1e-6


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    yield
    gc.collect()
    torch.cuda.empty_cache()


SAMPLES = {
    "gpt2_small": ["h0.attn.c_attn", "h0.attn.c_proj", "h5.mlp.c_fc", "h11.mlp.c_proj"],
    "per_head_wq": ["l0.wq", "l23.wq"],
    "llama_1b": ["l0.wk", "l23.up", "l11.down"],
    "llama_8b": ["l0.wk", "l0.wq", "l31.gate", "l0.down"],
}


# quintic steps as `bench.py --coeffs quintic` runs them: the second-order
# Newton-Schulz polynomial for the polar factor, five times
QUINTIC = [(1.875, -1.25, 0.375)] * 5


@pytest.mark.parametrize("set_name", ["gpt2_small", "per_head_wq", "llama_1b", "llama_8b"])
def test_full_set_muon_step(set_name):
    _full_set_muon_step(set_name, None)


@pytest.mark.parametrize("set_name", ["llama_1b", "llama_8b"])
def test_full_set_muon_step_quintic(set_name):
    _full_set_muon_step(set_name, QUINTIC)


def _full_set_muon_step(set_name, coeffs):
    import newton_schulz_orthogonalized_amd as nso
    idx = list(PARAM_SETS).index(set_name)
    ps = PARAM_SETS[set_name]()
    print(f"[fullsize muon] {set_name}: {len(ps.muon)} matrices, {ps.muon_elems()} elements, "
          f"{'cubic' if coeffs is None else 'quintic'} steps", flush=True)
    dt = torch.bfloat16
    ws, gs, ms, oo, keep = [], [], [], [], {}
    for j, e in enumerate(ps.muon):
        s = seed_for(idx, j)
        w = device_normal(e.shape, s, ps.weight_std, dt, "cuda")
        g = device_normal(e.shape, s + 500000, ps.grad_std, dt, "cuda")
        m = device_normal(e.shape, s + 900000, ps.mom_std, torch.float32, "cuda")
        o = None
        if e.name in SAMPLES[set_name]:
            keep[j] = (to_np(w), to_np(g), to_np(m))
            o = torch.zeros(e.shape, dtype=torch.float32, device="cuda")
        ws.append(w); gs.append(g); ms.append(m); oo.append(o)
    nso.muon_step(ws, gs, ms, lr=0.02, weight_decay=0.01, heads=[e.heads for e in ps.muon], ortho_outs=oo,
                  coeffs=coeffs)
    torch.cuda.synchronize()
    for j, (w0, g0, m0) in keep.items():
        e = ps.muon[j]
        print(f"  oracle for {e.name} {e.shape} heads={e.heads}", flush=True)
        ref = O.muon_step_ref(w0, g0, m0, lr=0.02, weight_decay=0.01, heads=e.heads, coeffs=coeffs)
        o = to_np(oo[j])
        err = O.rel_fro(o, ref["o"])
        terr = tile_rel_fro(o, ref["o"])
        print(f"    O relF {err:.3e}, worst 256x256 tile {terr:.3e}", flush=True)
        assert err <= BF16_TOL, e.name
        assert terr <= BF16_TOL, e.name
        assert O.rel_fro(to_np(ms[j]), ref["m"]) <= MOM_TOL, e.name
        w1 = to_np(ws[j])
        # the update arithmetic: W1 is the bf16 rounding of W0 - lr wd W0 - lr O, with the GPU's O
        want = w0 - 0.02 * 0.01 * w0 - 0.02 * o
        tol = bf16_ulp(want) * 0.5 + 8 * 2.0 ** -24 * (np.abs(w0) + 0.02 * np.abs(o))
        assert np.all(np.abs(w1 - want) <= tol), e.name
        # and W1 against the oracle's W
        frac = check_w_against_oracle(w1, w0, o, ref["w"], ref["o"], 0.02)
        print(f"    W within 1 bf16 ulp of RNE(oracle W): {100 * frac:.2f} %", flush=True)
    # every matrix moved and stayed finite
    for j, w in enumerate(ws):
        assert torch.isfinite(w).all(), ps.muon[j].name
    del ws, gs, ms, oo


@pytest.mark.parametrize("set_name", ["gpt2_small", "llama_8b"])
def test_full_set_adamw_step(set_name):
    import newton_schulz_orthogonalized_amd as nso
    idx = list(PARAM_SETS).index(set_name)
    ps = PARAM_SETS[set_name]()
    print(f"[fullsize adamw] {set_name}: {len(ps.adamw)} tensors, {ps.adamw_elems()} elements", flush=True)
    p_, g_, m_, v_, keep = [], [], [], [], {}
    rng = np.random.default_rng(idx)
    for j, e in enumerate(ps.adamw):
        s = seed_for(idx, 100 + j)
        p = device_normal(e.shape, s, ps.weight_std, torch.bfloat16, "cuda")
        g = device_normal(e.shape, s + 500000, ps.grad_std, torch.bfloat16, "cuda")
        m = device_normal(e.shape, s + 900000, 1e-3, torch.float32, "cuda")
        v = device_normal(e.shape, s + 700000, 1e-3, torch.float32, "cuda").square_()
        n = p.numel()
        lo = int(rng.integers(0, max(1, n - 1_000_000)))
        sl = slice(lo, min(n, lo + 1_000_000))
        keep[j] = (sl, to_np(p.view(-1)[sl]), to_np(g.view(-1)[sl]), to_np(m.view(-1)[sl]), to_np(v.view(-1)[sl]))
        p_.append(p); g_.append(g); m_.append(m); v_.append(v)
    nso.adamw_step(p_, g_, m_, v_, lr=0.02, weight_decay=0.01, beta1=0.9, beta2=0.95, eps=1e-8, step=10)
    torch.cuda.synchronize()
    for j, (sl, p0, g0, m0, v0) in keep.items():
        f32 = lambda x: float(np.float32(x))  # noqa: E731  (the C ABI's float32 hyper-parameters)
        pr, mr, vr = O.adamw_ref(p0, g0, m0, v0, lr=f32(0.02), weight_decay=f32(0.01), beta1=f32(0.9),
                                 beta2=f32(0.95), eps=f32(1e-8), step=10)
        p1 = to_np(p_[j].view(-1)[sl])
        # one rounding to bf16 of a float32 result: half an ulp of the result plus
        # float32 rounding of the operands (the update can cancel p to near zero)
        ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(pr), 2.0 ** -126))) - 7)
        tol = 0.5 * ulp + 8 * 2.0 ** -24 * (np.abs(p0) + np.abs(pr - p0))
        bad = np.abs(p1 - pr) > tol
        assert not bad.any(), (ps.adamw[j].name, int(bad.sum()), p0[bad][:3], pr[bad][:3], p1[bad][:3])
        assert O.rel_fro(to_np(m_[j].view(-1)[sl]), mr) <= 1e-6
        assert O.rel_fro(to_np(v_[j].view(-1)[sl]), vr) <= 1e-6
