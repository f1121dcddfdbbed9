"""mu_muon_step_noalloc (the entry point for callers that cannot allocate)
against mu_muon_step, through the C ABI: four calls in a row on one GPU, each
smaller than the one before, each compared bit for bit with mu_muon_step on
clones of the same inputs (same kernels, so the results must be identical),
and one matrix of each call against the oracle. The scratch array keeps the
previous call's contents, so the later calls also show that nothing stale is
read.
"""

import numpy as np
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


# (shape, heads) lists, largest first; dtype and Newton-Schulz precision
CALLS = [
    ([((32768, 256), 256), ((768, 2304), 1)], torch.bfloat16, "bf16"),   # fused short blocks + a tiled matrix
    ([((1024, 2048), 1)], torch.bfloat16, "bf16"),                         # Gram-side steps
    ([((768, 768), 1), ((2304, 768), 1), ((300, 77), 1)], torch.bfloat16, "bf16"),
    ([((128, 256), 1)], torch.float32, "f32"),
]


def _run(entry, specs, dtype, prec, seed):
    from newton_schulz_orthogonalized_amd import _lib
    ins = [make_matrix_inputs(sh, seed + 10 * i, dtype, 1e-3, 0.02, 1e-3) for i, (sh, _) in enumerate(specs)]
    host = [tuple(to_np(t) for t in x) for x in ins]
    ws_, gs_, ms_ = [x[0] for x in ins], [x[1] for x in ins], [x[2] for x in ins]
    oo = [torch.zeros(sh, dtype=torch.float32, device="cuda") for sh, _ in specs]
    mats, n = _lib.matrices(ws_, gs_, ms_, [h for _, h in specs], None, None, oo)
    hp, keep = _lib.muon_hparams(0.02, 0.01, 0.95, True, 1e-7, 5, None, prec)
    if entry == "noalloc":
        need = _lib.mu_muon_workspace_size(mats, n, hp)
        assert need <= _lib.MU_NOALLOC_SCRATCH_BYTES, need
        _lib.mu_muon_step_noalloc(mats, n, hp)
    else:
        ws = _lib.workspace(_lib.mu_muon_workspace_size(mats, n, hp), "cuda")
        _lib.mu_muon_step(mats, n, hp, ws)
    torch.cuda.synchronize()
    del keep
    return ws_, ms_, oo, host


def test_noalloc_matches_step_on_calls_of_falling_size():
    for k, (specs, dtype, prec) in enumerate(CALLS):
        print(f"[noalloc] call {k}: {specs} {prec}", flush=True)
        seed = 32000 + 100 * k
        w_a, m_a, o_a, host = _run("noalloc", specs, dtype, prec, seed)
        w_b, m_b, o_b, _ = _run("step", specs, dtype, prec, seed)
        for i in range(len(specs)):
            assert torch.equal(w_a[i], w_b[i]), (k, i)
            assert torch.equal(m_a[i], m_b[i]), (k, i)
            assert torch.equal(o_a[i], o_b[i]), (k, i)
        # one matrix of the call against the oracle
        (sh, heads) = specs[-1]
        w0, g0, m0 = host[-1]
        ref = O.muon_step_ref(w0, g0, m0, lr=0.02, weight_decay=0.01, heads=heads)
        tol = 1e-4 if prec == "f32" else 2e-2
        assert O.rel_fro(to_np(o_a[-1]), ref["o"]) <= tol, (k, sh)
        assert O.rel_fro(to_np(m_a[-1]), ref["m"]) <= 1e-6, (k, sh)


def test_noalloc_rejects_a_list_beyond_the_scratch():
    import newton_schulz_orthogonalized_amd as nso
    from newton_schulz_orthogonalized_amd import _lib
    w, g, m = make_matrix_inputs((4096, 4096), 32900, torch.bfloat16, 1e-3, 0.02, 1e-3)
    w0, m0 = w.clone(), m.clone()
    with pytest.raises(_lib.MuonError) as e:
        nso.muon_step([w], [g], [m], lr=0.02, weight_decay=0.01, noalloc=True)
    assert e.value.status == _lib.MU_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.equal(w, w0) and torch.equal(m, m0)
