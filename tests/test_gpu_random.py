"""Seeded random lists: shapes across every tile group and orientation, with
head counts, precisions and coefficient schedules drawn per call, in one
Muon call each. Every matrix is compared with the float64 oracle, and the
whole call with one call per matrix, bit for bit: the launches walk a call's
problems in an order of their own (sorted by K for the Gram, the reverse for
the apply) and deal the tiles to the XCDs in windows, none of which may
change any value.
"""

import numpy as np
import pytest
import torch

from gpu_util import make_matrix_inputs, need_gpu, to_np
from oracle import muon_oracle as O

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
MOM_TOL = 1e-6
SIDES = [1, 5, 64, 127, 128, 129, 255, 256, 300, 512, 640, 768, 1000, 1024, 1536]
SCHEDULES = [
    None,                                                         # 5 cubic steps
    [(1.875, -1.25, 0.375)] * 2 + [(1.5, -0.5, 0.0)] * 3,         # quintic, then cubic
    [(3.4445, -4.775, 2.0315)] * 5,                               # a tuned quintic schedule
]


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()
    yield
    torch.cuda.empty_cache()


def _draw(seed):
    rng = np.random.default_rng(seed)
    specs = []
    while len(specs) < int(rng.integers(5, 10)):
        r, c = (int(x) for x in rng.choice(SIDES, 2))
        if r * c > 1_600_000:
            continue
        heads = int(rng.choice([h for h in (1, 2, 4) if r % h == 0]))
        specs.append(((r, c), heads))
    return specs


# seed 5 adds wide and tall blocks that take Gram-side steps (m >= 1024, n > m)
GRAM_SIDE = [((1024, 1536), 1), ((1536, 1024), 1), ((1000, 1500), 1)]


@pytest.mark.parametrize("seed,prec,sched", [(0, "bf16", 0), (1, "f32", 0), (2, "bf16", 1), (3, "f32", 2),
                                             (4, "bf16", 2), (5, "bf16", 0)])
def test_random_list(seed, prec, sched):
    import newton_schulz_orthogonalized_amd as nso
    specs = _draw(1000 + seed) + (GRAM_SIDE if seed == 5 else [])
    coeffs = SCHEDULES[sched]
    print(f"[random list] seed={seed} prec={prec} schedule={sched} specs={specs}", flush=True)
    dt = torch.bfloat16 if prec == "bf16" else torch.float32
    std = (1e-3, 0.02, 1e-3) if prec == "bf16" else (1.0, 1.0, 1.0)
    ins = [make_matrix_inputs(sh, 40000 + 100 * seed + 10 * i, dt, *std) for i, (sh, _) in enumerate(specs)]
    host = [(to_np(w), to_np(g), to_np(m)) for w, g, m in ins]
    nest = seed % 2 == 0
    kw = dict(lr=0.02, weight_decay=0.01, mu=0.95, nesterov=nest, coeffs=coeffs, precision=prec)

    w1 = [w.clone() for w, _, _ in ins]
    m1 = [m.clone() for _, _, m in ins]
    o1 = [torch.zeros(sh, dtype=torch.float32, device="cuda") for sh, _ in specs]
    nso.muon_step(w1, [g for _, g, _ in ins], m1, heads=[h for _, h in specs], ortho_outs=o1, **kw)
    torch.cuda.synchronize()

    for i, ((sh, heads), (w0, g0, m0)) in enumerate(zip(specs, host)):
        ref = O.muon_step_ref(w0, g0, m0, lr=0.02, weight_decay=0.01, nesterov=nest, heads=heads, coeffs=coeffs)
        assert O.rel_fro(to_np(o1[i]), ref["o"]) <= TOL[prec], (sh, heads)
        assert O.rel_fro(to_np(m1[i]), ref["m"]) <= MOM_TOL, (sh, heads)

    for i, ((sh, heads), (w, g, m)) in enumerate(zip(specs, ins)):
        w2, m2 = w.clone(), m.clone()
        o2 = torch.zeros(sh, dtype=torch.float32, device="cuda")
        nso.muon_step([w2], [g], [m2], heads=[heads], ortho_outs=[o2], **kw)
        torch.cuda.synchronize()
        assert torch.equal(w1[i], w2), (sh, heads)
        assert torch.equal(m1[i], m2), (sh, heads)
        assert torch.equal(o1[i], o2), (sh, heads)
