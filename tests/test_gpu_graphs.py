"""Repeated calls: from the second call with the same structure (list,
workspace, steps, coefficients) on, the library replays its launch sequence
from a HIP graph and uploads only the call's table, whose header carries the
per-call scalars. Every replay must give bit for bit the result of the eager
launch sequence (which the library uses while its profiler is on), for
changing learning rate, weight decay, momentum and scales, with the program's
own eager work and synchronisations between the replays.
"""

import pytest
import torch

from gpu_util import make_matrix_inputs, need_gpu, to_np
from oracle import muon_oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    import newton_schulz_orthogonalized_amd  # noqa: F401  (fails loudly without the library)
    yield


def _lib():
    from newton_schulz_orthogonalized_amd import _lib as L
    return L


def _eager(fn):
    """Run fn with the library's profiler on, which makes every call launch
    its kernels one by one."""
    L = _lib()
    L.mu_profile_enable(True)
    try:
        fn()
        torch.cuda.synchronize()
    finally:
        L.mu_profile_enable(False)


SETS = [
    ([(768, 2304), (2304, 768), (768, 768)], [1, 1, 4], torch.bfloat16, "bf16"),
    ([(128, 256)], [1], torch.float32, "f32"),
    ([(256 * 128, 256)], [256], torch.bfloat16, "bf16"),   # the fused short-block path
]


@pytest.mark.parametrize("si", range(len(SETS)))
def test_replays_match_eager_with_changing_scalars(si):
    import newton_schulz_orthogonalized_amd as nso
    shapes, heads, dtype, prec = SETS[si]
    print(f"[graphs] {shapes} heads={heads} {prec}", flush=True)
    ins = [make_matrix_inputs(sh, 40000 + 10 * i, dtype, 1e-3, 0.02, 1e-3) for i, sh in enumerate(shapes)]
    w0 = [w.clone() for w, _, _ in ins]
    m0 = [m.clone() for _, _, m in ins]
    W = [w for w, _, _ in ins]
    G = [g for _, g, _ in ins]
    M = [m for _, _, m in ins]
    oo = [torch.zeros(sh, dtype=torch.float32, device="cuda") for sh in shapes]
    L = _lib()
    ws = L.workspace(nso.muon_workspace_bytes(W, G, M, heads=heads, precision=prec), "cuda")
    # per call: lr, weight decay, mu, nesterov, scales
    calls = [(0.02, 0.01, 0.95, True, 1.0), (0.05, 0.1, 0.9, False, 2.0), (0.01, 0.0, 0.95, True, 0.5),
             (0.03, 0.02, 0.8, True, 1.5), (0.02, 0.01, 0.95, True, 1.0)]

    def run(lr, wd, mu, nest, sc):
        nso.muon_step(W, G, M, lr=lr, weight_decay=wd, mu=mu, nesterov=nest, heads=heads,
                      scales=[sc] * len(W), precision=prec, workspace=ws, ortho_outs=oo)

    def restore():
        for a, b in zip(W, w0):
            a.copy_(b)
        for a, b in zip(M, m0):
            a.copy_(b)

    for k, args in enumerate(calls):
        restore()
        _eager(lambda: run(*args))
        want_w = [w.clone() for w in W]
        want_m = [m.clone() for m in M]
        want_o = [o.clone() for o in oo]
        for rep in range(2):   # replayed (the first call of the structure was eager), twice
            restore()
            torch.cuda.synchronize()
            run(*args)
            junk = torch.randn(1 << 20, device="cuda").sum()   # the program's own work in between
            torch.cuda.synchronize()
            del junk
            for i in range(len(W)):
                assert torch.equal(W[i], want_w[i]), (k, rep, i)
                assert torch.equal(M[i], want_m[i]), (k, rep, i)
                assert torch.equal(oo[i], want_o[i]), (k, rep, i)
    # and one matrix of the last call against the oracle
    restore()
    host = [to_np(t) for t in (W[0], G[0], M[0])]
    run(*calls[-1])
    torch.cuda.synchronize()
    lr, wd, mu, nest, sc = calls[-1]
    ref = O.muon_step_ref(*host, lr=lr, weight_decay=wd, mu=mu, nesterov=nest, heads=heads[0], scale=sc)
    assert O.rel_fro(to_np(oo[0]), ref["o"]) <= (1e-4 if prec == "f32" else 2e-2)


def test_two_lists_alternating_share_a_workspace():
    """Two different lists on one workspace, alternating: each is replayed
    from its own graph after uploading its own table."""
    import newton_schulz_orthogonalized_amd as nso
    a = [make_matrix_inputs((512, 1024), 41000, torch.bfloat16, 1e-3, 0.02, 1e-3)]
    b = [make_matrix_inputs((1024, 384), 41100, torch.bfloat16, 1e-3, 0.02, 1e-3),
         make_matrix_inputs((300, 77), 41200, torch.bfloat16, 1e-3, 0.02, 1e-3)]
    sets = [a, b]
    snap = [[(w.clone(), m.clone()) for w, _, m in s] for s in sets]
    need = max(nso.muon_workspace_bytes([w for w, _, _ in s], [g for _, g, _ in s], [m for _, _, m in s])
               for s in sets)
    ws = _lib().workspace(need, "cuda")

    def run(s):
        nso.muon_step([w for w, _, _ in s], [g for _, g, _ in s], [m for _, _, m in s], lr=0.02, weight_decay=0.01,
                      workspace=ws)

    def restore(j):
        for (w, _, m), (w0, m0) in zip(sets[j], snap[j]):
            w.copy_(w0)
            m.copy_(m0)

    want = []
    for j in range(2):
        restore(j)
        _eager(lambda: run(sets[j]))
        want.append([(w.clone(), m.clone()) for w, _, m in sets[j]])
    for rep in range(3):
        for j in range(2):
            restore(j)
            run(sets[j])
            torch.cuda.synchronize()
            for (w, _, m), (ww, wm) in zip(sets[j], want[j]):
                assert torch.equal(w, ww) and torch.equal(m, wm), (rep, j)


def test_more_structures_than_the_cache_holds():
    """Twenty list structures, each called three times (eager, capture,
    replay), then the first five again after they were evicted from the
    16-entry cache: every call bit for bit the eager result."""
    import newton_schulz_orthogonalized_amd as nso
    shapes = [(64 + 32 * i, 96 + 40 * i) for i in range(20)]
    ins = [make_matrix_inputs(sh, 43000 + i, torch.bfloat16, 1e-3, 0.02, 1e-3) for i, sh in enumerate(shapes)]
    snap = [(w.clone(), m.clone()) for w, _, m in ins]
    want = []
    for i, (w, g, m) in enumerate(ins):
        _eager(lambda: nso.muon_step([w], [g], [m], lr=0.02, weight_decay=0.01))
        want.append((w.clone(), m.clone()))
        w.copy_(snap[i][0])
        m.copy_(snap[i][1])

    def check(i):
        w, g, m = ins[i]
        w.copy_(snap[i][0])
        m.copy_(snap[i][1])
        nso.muon_step([w], [g], [m], lr=0.02, weight_decay=0.01)
        torch.cuda.synchronize()
        assert torch.equal(w, want[i][0]) and torch.equal(m, want[i][1]), i

    for i in range(20):
        for _ in range(3):
            check(i)
    for i in range(5):
        for _ in range(3):
            check(i)
