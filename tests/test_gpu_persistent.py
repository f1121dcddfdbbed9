"""Persistent launches: a Gram or apply launch (but not the last apply) of at
least 8 tiles per compute unit runs one workgroup per compute unit, and each
takes tiles from its XCD's queue (the tiles that XCD would run in a
one-workgroup-per-tile launch, in the same order), then from the other XCDs'
queues. Every tile is computed by one workgroup with the same arithmetic, so
the result must be bit for bit that of the one-workgroup-per-tile launch
(MU_PERSIST=0), for cubic steps and for quintic steps (whose A A^T pass is a
Gram launch as well). Sixteen 4096 x 4096 matrices give 16 x 136 = 2176 Gram
tiles and 4096 apply tiles of 256 x 256, above the threshold of 8 x 256
compute units. (The one-workgroup-per-tile path is held to the
oracle by every other parity test, among them the 8B-shaped set, whose Gram
launches are persistent by default.)
"""

import pytest
import torch

from gpu_util import make_matrix_inputs, need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    import newton_schulz_orthogonalized_amd  # noqa: F401  (fails loudly without the library)
    yield


QUINTIC = [(1.875, -1.25, 0.375)] * 5


@pytest.mark.parametrize("coeffs", [None, QUINTIC], ids=["cubic", "quintic"])
def test_persistent_launches_match_one_workgroup_per_tile(coeffs, monkeypatch):
    import newton_schulz_orthogonalized_amd as nso
    from newton_schulz_orthogonalized_amd import _lib as L
    props = torch.cuda.get_device_properties(0)
    shapes = [(4096, 4096)] * 16
    if 16 * 136 < 8 * props.multi_processor_count:
        pytest.skip("fewer Gram tiles than the persistent threshold on this device")
    print(f"[persistent] 16 x (4096, 4096) coeffs={'quintic' if coeffs else 'cubic'}", flush=True)
    ins = [make_matrix_inputs(sh, 45000 + i, torch.bfloat16, 1e-3, 0.02, 1e-3) for i, sh in enumerate(shapes)]
    w0 = [w.clone() for w, _, _ in ins]
    m0 = [m.clone() for _, _, m in ins]
    oo = [torch.zeros(sh, dtype=torch.float32, device="cuda") for sh in shapes]

    def run(persist):
        monkeypatch.setenv("MU_PERSIST", "1" if persist else "0")
        for (w, _, m), a, b in zip(ins, w0, m0):
            w.copy_(a)
            m.copy_(b)
        L.mu_profile_enable(True)   # eager launches: the switch is read when the sequence is planned
        try:
            nso.muon_step([x[0] for x in ins], [x[1] for x in ins], [x[2] for x in ins], lr=0.02,
                          weight_decay=0.01, coeffs=coeffs, ortho_outs=oo)
            torch.cuda.synchronize()
        finally:
            L.mu_profile_enable(False)
        return [w.clone() for w, _, _ in ins], [o.clone() for o in oo]

    w_tile, o_tile = run(False)
    w_pers, o_pers = run(True)
    for i in range(len(shapes)):
        assert torch.equal(o_pers[i], o_tile[i]), i
        assert torch.equal(w_pers[i], w_tile[i]), i


def test_persistent_128_tiles_match_one_workgroup_per_tile(monkeypatch):
    """The 128 x 128 tile kernel (two workgroups per compute unit) in a
    persistent apply: 256 blocks of 200 x 4096 (short side padded to 256,
    tile 128, not the fused path) give 256 x 64 = 16384 apply tiles, above
    8 x 512 slots; the Gram (768 tiles) stays one workgroup per tile. Tall
    and wide blocks alike."""
    import newton_schulz_orthogonalized_amd as nso
    from newton_schulz_orthogonalized_amd import _lib as L
    props = torch.cuda.get_device_properties(0)
    shapes = [(200, 4096) if i % 2 else (4096, 200) for i in range(256)]
    if 256 * 64 < 8 * 2 * props.multi_processor_count:
        pytest.skip("fewer apply tiles than the persistent threshold on this device")
    print("[persistent] 256 x (200, 4096) / (4096, 200), 128 tiles", flush=True)
    ins = [make_matrix_inputs(sh, 46000 + i, torch.bfloat16, 1e-3, 0.02, 1e-3) for i, sh in enumerate(shapes)]
    w0 = [w.clone() for w, _, _ in ins]
    m0 = [m.clone() for _, _, m in ins]
    oo = [torch.zeros(sh, dtype=torch.float32, device="cuda") for sh in shapes]

    def run(persist):
        monkeypatch.setenv("MU_PERSIST", "1" if persist else "0")
        for (w, _, m), a, b in zip(ins, w0, m0):
            w.copy_(a)
            m.copy_(b)
        L.mu_profile_enable(True)
        try:
            nso.muon_step([x[0] for x in ins], [x[1] for x in ins], [x[2] for x in ins], lr=0.02,
                          weight_decay=0.01, ortho_outs=oo)
            torch.cuda.synchronize()
        finally:
            L.mu_profile_enable(False)
        return [w.clone() for w, _, _ in ins], [o.clone() for o in oo]

    w_tile, o_tile = run(False)
    w_pers, o_pers = run(True)
    for i in range(len(shapes)):
        assert torch.equal(o_pers[i], o_tile[i]), i
        assert torch.equal(w_pers[i], w_tile[i]), i


def test_persistent_gram_side_launches_match_one_workgroup_per_tile(monkeypatch):
    """Gram-side blocks in persistent launches: 16 blocks of 4096 x 8192 (eight
    wide, eight tall) give 16 x 136 = 2176 upper tiles per m x m product set and
    per first Gram, and 8192 restart tiles, all above 8 x 256 slots."""
    import newton_schulz_orthogonalized_amd as nso
    from newton_schulz_orthogonalized_amd import _lib as L
    props = torch.cuda.get_device_properties(0)
    shapes = [(4096, 8192) if i % 2 else (8192, 4096) for i in range(16)]
    if 16 * 136 < 8 * props.multi_processor_count:
        pytest.skip("fewer tiles than the persistent threshold on this device")
    print("[persistent] 16 x (4096, 8192) / (8192, 4096), Gram-side steps", flush=True)
    ins = [make_matrix_inputs(sh, 47000 + i, torch.bfloat16, 1e-3, 0.02, 1e-3) for i, sh in enumerate(shapes)]
    w0 = [w.clone() for w, _, _ in ins]
    m0 = [m.clone() for _, _, m in ins]
    oo = [torch.zeros(sh, dtype=torch.float32, device="cuda") for sh in shapes]

    def run(persist):
        monkeypatch.setenv("MU_PERSIST", "1" if persist else "0")
        for (w, _, m), a, b in zip(ins, w0, m0):
            w.copy_(a)
            m.copy_(b)
        L.mu_profile_enable(True)
        try:
            nso.muon_step([x[0] for x in ins], [x[1] for x in ins], [x[2] for x in ins], lr=0.02,
                          weight_decay=0.01, ortho_outs=oo)
            torch.cuda.synchronize()
        finally:
            L.mu_profile_enable(False)
        return [w.clone() for w, _, _ in ins], [o.clone() for o in oo]

    w_tile, o_tile = run(False)
    w_pers, o_pers = run(True)
    for i in range(len(shapes)):
        assert torch.equal(o_pers[i], o_tile[i]), i
        assert torch.equal(w_pers[i], w_tile[i]), i
