"""The C-ABI library loads on a machine without a GPU, exports every symbol the
header declares, and rejects bad arguments before any HIP call (status codes
only; nothing here enqueues work or touches device memory)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "muon_mi355x.h")
LIB = os.path.join(ROOT, "newton_schulz_orthogonalized_amd", "libmuon_mi355x.so")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(mu_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libmuon_mi355x.so is not built (run __graft_entry__.build())")
    from newton_schulz_orthogonalized_amd import _lib
    return _lib


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("mu_muon_workspace_size", "mu_muon_step", "mu_muon_orthogonalize", "mu_ortho_workspace_size",
              "mu_adamw_workspace_size", "mu_adamw_step", "mu_status_string", "mu_last_error", "mu_version"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    raw = ctypes.CDLL(LIB)
    for n in _declared():
        assert hasattr(raw, n), n
    assert set(lib.EXPORTED) == set(_declared())


def test_header_constants_match_the_binding(lib):
    """The kernel-class ids, status codes and dtypes the binding uses are the
    header's, and every kernel class has a name in the library."""
    text = open(HEADER).read()
    defs = {k: int(v) for k, v in re.findall(r"^#define\s+(MU_\w+)\s+\(?(-?\d+)\)?", text, re.M)}
    for k, v in defs.items():
        if k.startswith("MU_K_") or k.startswith("MU_ERR_") or k in ("MU_OK", "MU_F32", "MU_BF16"):
            if hasattr(lib, k):
                assert getattr(lib, k) == v, k
    assert lib.MU_K_COUNT == defs["MU_K_COUNT"]
    names = [lib.mu_kernel_name(k) for k in range(lib.MU_K_COUNT)]
    assert "unknown" not in names and len(set(names)) == len(names)
    assert lib.mu_kernel_name(lib.MU_K_COUNT) == "unknown"


def test_version_and_status_strings(lib):
    assert lib.mu_version() == 2
    assert lib.mu_status_string(0) == "ok"
    assert "workspace" in lib.mu_status_string(lib.MU_ERR_WORKSPACE)
    assert lib.mu_status_string(99) == "unknown status"


# Fake, never-dereferenced device addresses: validation must reject these
# calls before any HIP call is made.
A = 0x7f0000000000


def _mat(lib, **kw):
    d = dict(param=A, grad=A + (1 << 24), momentum=A + (2 << 24), rows=64, cols=32, dtype=lib.MU_F32,
             num_heads=1, scale=1.0, norm_out=None, ortho_out=None)
    d.update(kw)
    return lib.MuMatrix(**d)


def _hp(lib, **kw):
    d = dict(lr=0.02, weight_decay=0.01, mu=0.95, nesterov=1, norm_eps=1e-7, ns_steps=5, coeffs=None,
             ns_precision=lib.MU_NS_BF16, cautious_wd=0)
    d.update(kw)
    return lib.MuMuonHparams(**d)


def _step(lib, mats, hp, ws=None, nbytes=0):
    arr = (lib.MuMatrix * len(mats))(*mats)
    return lib.LIB.mu_muon_step(arr, len(mats), ctypes.byref(hp), ws, nbytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(num_heads=3), 1), (dict(num_heads=0), 1), (dict(rows=0), 1), (dict(cols=-4), 1),
    (dict(param=None), 1), (dict(dtype=7), 2), (dict(grad=A + 1), 3),
    (dict(rows=(1 << 21) + 1, cols=8), 1), (dict(rows=8, cols=(1 << 21) + 1), 1),
])
def test_bad_matrix_rejected(lib, kw, code):
    assert _step(lib, [_mat(lib, **kw)], _hp(lib)) == code
    assert lib.mu_last_error() != ""


def test_bad_hparams_rejected(lib):
    assert _step(lib, [_mat(lib)], _hp(lib, ns_steps=-1)) == lib.MU_ERR_INVALID_ARG
    assert _step(lib, [_mat(lib)], _hp(lib, cautious_wd=2)) == lib.MU_ERR_INVALID_ARG
    assert _step(lib, [_mat(lib)], _hp(lib, ns_precision=9)) == lib.MU_ERR_DTYPE
    assert _step(lib, [_mat(lib)], _hp(lib, lr=float("nan"))) == lib.MU_ERR_INVALID_ARG


def test_overlap_and_mixed_dtype_rejected(lib):
    assert _step(lib, [_mat(lib, grad=A + 100)], _hp(lib)) == lib.MU_ERR_LAYOUT
    m2 = _mat(lib, param=A + (3 << 24), grad=A + (4 << 24), momentum=A + (5 << 24), dtype=lib.MU_BF16)
    assert _step(lib, [_mat(lib), m2], _hp(lib)) == lib.MU_ERR_DTYPE


def test_workspace_checks(lib):
    need = ctypes.c_size_t(0)
    arr = (lib.MuMatrix * 1)(_mat(lib))
    assert lib.LIB.mu_muon_workspace_size(arr, 1, ctypes.byref(_hp(lib)), ctypes.byref(need)) == 0
    # 64x32 float32 -> X is 32x64, 128-tiles on the bf16 path: 2 x 128x128 x 2 B + 128x128 x 2 B + tables
    assert need.value >= 3 * 128 * 128 * 2
    assert _step(lib, [_mat(lib)], _hp(lib)) == lib.MU_ERR_WORKSPACE
    assert _step(lib, [_mat(lib)], _hp(lib), ws=A + (9 << 24), nbytes=need.value - 1) == lib.MU_ERR_WORKSPACE
    assert _step(lib, [_mat(lib)], _hp(lib), ws=A + (9 << 24) + 16, nbytes=need.value) == lib.MU_ERR_WORKSPACE


def test_gram_side_workspace(lib, monkeypatch):
    """Gram-side steps (wide bf16 blocks, n > m, m >= 1024, three or more cubic
    steps) add exactly six m x m buffers per block (the unfolded B0 and a
    second B, two Q, S and one A) plus their descriptors and tile maps; every
    other block and schedule plans as with MU_GRAMSIDE=0."""
    def need(rows, cols, **kw):
        arr = (lib.MuMatrix * 1)(_mat(lib, rows=rows, cols=cols, dtype=lib.MU_BF16))
        n = ctypes.c_size_t(0)
        assert lib.LIB.mu_muon_workspace_size(arr, 1, ctypes.byref(_hp(lib, **kw)), ctypes.byref(n)) == 0
        return n.value

    cases = [((1024, 4096), {}, True), ((4096, 1024), {}, True), ((1000, 2600), {}, True),
             ((1024, 4096), dict(ns_steps=3), True), ((1024, 1024), {}, False), ((512, 4096), {}, False),
             ((1024, 2048), {}, True), ((1024, 1280), {}, True), ((1024, 4096), dict(ns_steps=2), False),
             ((1024, 4096), dict(ns_precision=lib.MU_NS_F32), False)]
    for (r, c), kw, gains in cases:
        monkeypatch.delenv("MU_GRAMSIDE", raising=False)
        on = need(r, c, **kw)
        monkeypatch.setenv("MU_GRAMSIDE", "0")
        off = need(r, c, **kw)
        mp = 1024
        extra = 6 * mp * mp * 2
        if gains:
            assert extra <= on - off < extra + (64 << 10), ((r, c), kw, on - off)
        else:
            assert on == off, ((r, c), kw)
    # quintic steps: no Gram-side steps
    co = (ctypes.c_float * 15)(*([1.875, -1.25, 0.375] * 5))
    monkeypatch.delenv("MU_GRAMSIDE", raising=False)
    on = need(1024, 4096, coeffs=co)
    monkeypatch.setenv("MU_GRAMSIDE", "0")
    assert need(1024, 4096, coeffs=co) == on


def test_empty_list_is_ok_without_device(lib):
    arr = (lib.MuMatrix * 1)()
    assert lib.LIB.mu_muon_step(arr, 0, ctypes.byref(_hp(lib)), None, 0, None) == 0
    need = ctypes.c_size_t(123)
    assert lib.LIB.mu_muon_workspace_size(arr, 0, ctypes.byref(_hp(lib)), ctypes.byref(need)) == 0
    assert need.value == 0


def test_adamw_validation(lib):
    t = lib.MuTensor(A, A + (1 << 24), A + (2 << 24), A + (3 << 24), 100, lib.MU_F32, 0.1, 0.0)
    arr = (lib.MuTensor * 1)(t)
    for hp, code in [((0.9, 0.95, 1e-8, 0), 1), ((1.0, 0.95, 1e-8, 1), 1), ((0.9, 0.95, float("inf"), 1), 1)]:
        h = lib.MuAdamwHparams(*hp)
        assert lib.LIB.mu_adamw_step(arr, 1, ctypes.byref(h), None, 0, None) == code
    h = lib.MuAdamwHparams(0.9, 0.95, 1e-8, 1)
    assert lib.LIB.mu_adamw_step(arr, 1, ctypes.byref(h), None, 0, None) == lib.MU_ERR_WORKSPACE
    bad = (lib.MuTensor * 1)(lib.MuTensor(A, A + 2, A + (2 << 24), A + (3 << 24), 100, lib.MU_F32, 0.1, 0.0))
    assert lib.LIB.mu_adamw_step(bad, 1, ctypes.byref(h), None, 0, None) == lib.MU_ERR_LAYOUT


def test_ortho_validation(lib):
    x = lib.MuOrtho(A, A + (1 << 24), 10, 20, lib.MU_BF16, 3, None)
    arr = (lib.MuOrtho * 1)(x)
    assert lib.LIB.mu_muon_orthogonalize(arr, 1, ctypes.byref(_hp(lib)), None, 0, None) == lib.MU_ERR_INVALID_ARG
    x = lib.MuOrtho(A, A, 10, 20, lib.MU_BF16, 1, None)
    arr = (lib.MuOrtho * 1)(x)
    assert lib.LIB.mu_muon_orthogonalize(arr, 1, ctypes.byref(_hp(lib)), None, 0, None) == lib.MU_ERR_LAYOUT


def _qk(lib, **kw):
    d = dict(wq=A, wk=A + (1 << 24), q_rows=64, k_rows=16, cols=32, q_heads=8, k_heads=2, dtype=lib.MU_BF16,
             pad0=0, max_logit=A + (2 << 24), gamma_out=None)
    d.update(kw)
    return lib.MuQkPair(**d)


def _clip(lib, pairs, tau=100.0, ws=None, nbytes=0):
    arr = (lib.MuQkPair * max(len(pairs), 1))(*pairs)
    return lib.LIB.mu_qk_clip(arr, len(pairs), tau, ws, nbytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q_heads=3), 1), (dict(k_heads=3), 1), (dict(q_heads=4, k_heads=8, k_rows=16), 1), (dict(cols=0), 1),
    (dict(wq=None), 1), (dict(max_logit=None), 1), (dict(dtype=5), 2), (dict(wk=A + 2), 3),
    (dict(max_logit=A + 3), 3), (dict(gamma_out=A + (2 << 24) + 16), 3),
])
def test_qk_clip_bad_pair_rejected(lib, kw, code):
    assert _clip(lib, [_qk(lib, **kw)]) == code
    assert lib.mu_last_error() != ""


def test_qk_clip_tau_and_workspace_checks(lib):
    for tau in (0.0, -1.0, float("nan"), float("inf")):
        assert _clip(lib, [_qk(lib)], tau=tau) == lib.MU_ERR_INVALID_ARG
    assert _clip(lib, [_qk(lib)]) == lib.MU_ERR_WORKSPACE
    arr = (lib.MuQkPair * 2)(_qk(lib), _qk(lib, wq=A + (4 << 24), wk=A + (5 << 24), max_logit=A + (6 << 24)))
    need = ctypes.c_size_t(0)
    assert lib.LIB.mu_qk_clip_workspace_size(arr, 2, ctypes.byref(need)) == 0
    assert need.value >= 2 * (8 + 2) * 8   # one segment per head of each matrix
    assert lib.LIB.mu_qk_clip(arr, 2, 100.0, A + (9 << 24), need.value - 1, None) == lib.MU_ERR_WORKSPACE
    assert _clip(lib, []) == 0                               # empty list: no-op without a device


def test_qk_clip_overlapping_pairs_rejected(lib):
    a = _qk(lib)
    b = _qk(lib, wq=A + (1 << 24) + 64, wk=A + (4 << 24), max_logit=A + (6 << 24))   # b.wq inside a.wk
    assert _clip(lib, [a, b]) == lib.MU_ERR_LAYOUT


def test_noalloc_scratch_limit_and_empty_list(lib):
    """mu_muon_step_noalloc: the header's scratch size is the binding's, a list
    beyond it is rejected before any HIP call, an empty list is a no-op, and
    validation runs as for mu_muon_step."""
    text = open(HEADER).read()
    m = re.search(r"#define\s+MU_NOALLOC_SCRATCH_BYTES\s+\((\d+)u\s*<<\s*(\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == lib.MU_NOALLOC_SCRATCH_BYTES
    big = _mat(lib, rows=8192, cols=8192, dtype=lib.MU_BF16, grad=A + (1 << 30), momentum=A + (2 << 30))
    arr = (lib.MuMatrix * 1)(big)
    need = ctypes.c_size_t(0)
    assert lib.LIB.mu_muon_workspace_size(arr, 1, ctypes.byref(_hp(lib)), ctypes.byref(need)) == 0
    assert need.value > lib.MU_NOALLOC_SCRATCH_BYTES
    assert lib.LIB.mu_muon_step_noalloc(arr, 1, ctypes.byref(_hp(lib)), None) == lib.MU_ERR_WORKSPACE
    assert "scratch" in lib.mu_last_error()
    assert lib.LIB.mu_muon_step_noalloc(arr, 0, ctypes.byref(_hp(lib)), None) == 0
    bad = (lib.MuMatrix * 1)(_mat(lib, num_heads=3))
    assert lib.LIB.mu_muon_step_noalloc(bad, 1, ctypes.byref(_hp(lib)), None) == lib.MU_ERR_INVALID_ARG
    assert lib.LIB.mu_muon_step_noalloc(arr, 1, ctypes.byref(_hp(lib, ns_steps=-2)), None) == lib.MU_ERR_INVALID_ARG


def test_tie_to_stream_records_only_other_streams(lib):
    """A workspace allocated on the current stream is recorded on the launch
    stream when that is another stream, so the caching allocator keeps it
    until the library's kernels there are done."""
    class FakeStream:
        def __init__(self, h):
            self.cuda_stream = h

    class FakeBuf:
        def __init__(self):
            self.recorded = []
            self.device = "cuda:0"

        def record_stream(self, s):
            self.recorded.append(s.cuda_stream)

    import torch
    orig = torch.cuda.Stream
    try:
        torch.cuda.Stream = FakeStream   # the helper takes any torch stream object as it is
        cur = FakeStream(11)
        b = FakeBuf()
        lib.tie_to_stream(b, FakeStream(22), current=cur)
        assert b.recorded == [22]
        b = FakeBuf()
        lib.tie_to_stream(b, FakeStream(11), current=cur)
        assert b.recorded == []
        b = FakeBuf()
        lib.tie_to_stream(b, None, current=cur)
        assert b.recorded == []
        lib.tie_to_stream(None, FakeStream(22), current=cur)
    finally:
        torch.cuda.Stream = orig



def test_ceiling_probe_library_loads_and_is_separate():
    """The benchmark's MFMA ceiling probe is a library of its own: it loads
    without a GPU, exports its one entry point, and the optimizer library
    exports nothing of it."""
    path = os.path.join(ROOT, "newton_schulz_orthogonalized_amd", "libmuon_probe.so")
    if not os.path.exists(path):
        pytest.fail("libmuon_probe.so is not built (run __graft_entry__.build())")
    probe = ctypes.CDLL(path)
    assert hasattr(probe, "probe_mfma_bf16")
    assert not hasattr(ctypes.CDLL(LIB), "probe_mfma_bf16")
