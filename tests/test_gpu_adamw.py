"""GPU parity of the multi-tensor AdamW step against the CPU oracle."""

import numpy as np
import pytest
import torch

from gpu_util import bf16_ulp, need_gpu, to_np
from oracle import muon_oracle as O
from workloads import as_dtype, host_normal

pytestmark = pytest.mark.gpu

# around the chunk (8192 elements) and the band of the tiled layout (65536
# elements): whole bands, bands plus whole and ragged chunks
SIZES = [1, 7, 8, 9, 4095, 4096, 4097, 10000, 65536, 70001, 131072 + 12293, 3 * 65536 + 1]


def f32(x):
    return float(np.float32(x))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()
    yield


def _case(dtype, step, seed, random_state):
    import newton_schulz_orthogonalized_amd as nso
    ps, gs, ms, vs, ref_in = [], [], [], [], []
    lrs = [0.02 * (1 + i % 3) for i in range(len(SIZES))]
    wds = [0.01 * (i % 2) for i in range(len(SIZES))]
    for i, n in enumerate(SIZES):
        p = as_dtype(host_normal(n, seed + 10 * i, 0.5), dtype)
        g = as_dtype(host_normal(n, seed + 10 * i + 1, 1e-2), dtype)
        if random_state:
            m = as_dtype(host_normal(n, seed + 10 * i + 2, 1e-2), torch.float32)
            v = as_dtype(host_normal(n, seed + 10 * i + 3, 1e-2) ** 2, torch.float32)
        else:
            m = torch.zeros(n)
            v = torch.zeros(n)
        ref_in.append((to_np(p), to_np(g), to_np(m), to_np(v)))
        ps.append(p.cuda()); gs.append(g.cuda()); ms.append(m.cuda()); vs.append(v.cuda())
    nso.adamw_step(ps, gs, ms, vs, lr=lrs, weight_decay=wds, beta1=0.9, beta2=0.95, eps=1e-8, step=step)
    torch.cuda.synchronize()
    for i in range(len(SIZES)):
        p0, g0, m0, v0 = ref_in[i]
        # the C ABI takes float32 hyper-parameters: give the oracle those same values
        pr, mr, vr = O.adamw_ref(p0, g0, m0, v0, lr=f32(lrs[i]), weight_decay=f32(wds[i]), beta1=f32(0.9),
                                 beta2=f32(0.95), eps=f32(1e-8), step=step)
        yield i, to_np(ps[i]), to_np(ms[i]), to_np(vs[i]), pr, mr, vr, (p0, g0, m0, v0)


U32 = 2.0 ** -24  # float32 unit roundoff


def check_states(m, v, mr, vr, ins):
    """Moments against the oracle: relative Frobenius error 1e-6, and per element
    within a few float32 roundings of the operands of each update."""
    p0, g0, m0, v0 = ins
    assert O.rel_fro(m, mr) <= 1e-6
    assert O.rel_fro(v, vr) <= 1e-6
    assert np.all(np.abs(m - mr) <= 4 * U32 * (0.9 * np.abs(m0) + 0.1 * np.abs(g0)) + 1e-30)
    assert np.all(np.abs(v - vr) <= 6 * U32 * (0.95 * np.abs(v0) + 0.05 * g0 * g0) + 1e-30)


@pytest.mark.parametrize("step,random_state", [(1, False), (10, True), (1000, True)])
def test_adamw_f32(step, random_state):
    for i, p, m, v, pr, mr, vr, ins in _case(torch.float32, step, 20000 + step, random_state):
        check_states(m, v, mr, vr, ins)
        # the step p - p0 is lr-sized; compare it, not p, so the check has teeth
        p0 = ins[0]
        assert O.rel_fro(p - p0, pr - p0) <= 1e-4, i


@pytest.mark.parametrize("step,random_state", [(1, False), (10, True)])
def test_adamw_bf16(step, random_state):
    for i, p, m, v, pr, mr, vr, ins in _case(torch.bfloat16, step, 21000 + step, random_state):
        check_states(m, v, mr, vr, ins)
        # one rounding to bf16 of a float32 result: half an ulp of the result plus
        # float32 rounding of the operands (the update can cancel p to near zero)
        p0 = ins[0]
        tol = 0.5 * bf16_ulp(pr) + 8 * U32 * (np.abs(p0) + np.abs(pr - p0))
        assert np.all(np.abs(p - pr) <= tol), i


def test_adamw_empty_tensor_and_list():
    import newton_schulz_orthogonalized_amd as nso
    nso.adamw_step([], [], [], [], lr=0.1, weight_decay=0.0)
    z = torch.zeros(0, device="cuda")
    nso.adamw_step([z], [z.clone()], [z.clone()], [z.clone()], lr=0.1, weight_decay=0.0, step=1)


def test_adamw_rejects_step_zero():
    import newton_schulz_orthogonalized_amd as nso
    from newton_schulz_orthogonalized_amd import _lib
    p = torch.ones(10, device="cuda")
    with pytest.raises(_lib.MuonError):
        nso.adamw_step([p], [p.clone()], [p.clone()], [p.clone()], lr=0.1, weight_decay=0.0, step=0)
    assert torch.all(p == 1)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_adamw_unaligned_views_take_the_contiguous_path(dtype):
    """Buffers that are not 16-byte aligned (views one element into a larger
    allocation) are taken in contiguous chunks; the same values, aligned, go
    through the band tiles. Both must equal the oracle, and each other bit for bit."""
    import newton_schulz_orthogonalized_amd as nso
    n = 2 * 65536 + 8192 + 37
    p0 = as_dtype(host_normal(n, 23001, 0.5), dtype)
    g0 = as_dtype(host_normal(n, 23002, 1e-2), dtype)
    m0 = as_dtype(host_normal(n, 23003, 1e-2), torch.float32)
    v0 = as_dtype(host_normal(n, 23004, 1e-2) ** 2, torch.float32)
    outs = []
    for off in (0, 1):
        bufs = [torch.zeros(n + 1, dtype=t.dtype, device="cuda") for t in (p0, g0, m0, v0)]
        views = [b[off:off + n] for b in bufs]
        for vw, t in zip(views, (p0, g0, m0, v0)):
            vw.copy_(t.cuda())
        nso.adamw_step([views[0]], [views[1]], [views[2]], [views[3]], lr=0.03, weight_decay=0.01, beta1=0.9,
                       beta2=0.95, eps=1e-8, step=7)
        torch.cuda.synchronize()
        outs.append([to_np(vw) for vw in (views[0], views[2], views[3])])
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(a, b)
    ins = tuple(to_np(t) for t in (p0, g0, m0, v0))
    pr, mr, vr = O.adamw_ref(*ins, lr=f32(0.03), weight_decay=f32(0.01), beta1=f32(0.9), beta2=f32(0.95),
                             eps=f32(1e-8), step=7)
    p, m, v = outs[0]
    check_states(m, v, mr, vr, ins)
    if dtype == torch.float32:
        assert O.rel_fro(p - ins[0], pr - ins[0]) <= 1e-4
    else:
        tol = 0.5 * bf16_ulp(pr) + 8 * U32 * (np.abs(ins[0]) + np.abs(pr - ins[0]))
        assert np.all(np.abs(p - pr) <= tol)
