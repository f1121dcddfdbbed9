"""ctypes binding of libmuon_mi355x.so: argument marshalling only.

Every entry point of ``include/muon_mi355x.h`` has a function of the same name
here that takes torch tensors, fills the C structs with their device pointers
and calls the library on the current HIP stream. All arithmetic runs in the
library's kernels; there is no fallback path, and importing this module fails
loudly when the shared library is missing.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmuon_mi355x.so")

MU_F32 = 0
MU_BF16 = 1
MU_NS_F32 = 0
MU_NS_BF16 = 1

MU_OK = 0
MU_ERR_INVALID_ARG = 1
MU_ERR_DTYPE = 2
MU_ERR_LAYOUT = 3
MU_ERR_WORKSPACE = 4
MU_ERR_HIP = 5

(MU_K_PREP, MU_K_NORM, MU_K_GRAM, MU_K_GRAM2, MU_K_APPLY, MU_K_FINISH, MU_K_ADAMW, MU_K_QKCLIP, MU_K_FUSED,
 MU_K_RESCALE, MU_K_TILEMAP) = range(11)
MU_K_COUNT = 11

EXPORTED = (
    "mu_muon_workspace_size", "mu_muon_step", "mu_muon_step_noalloc", "mu_ortho_workspace_size",
    "mu_muon_orthogonalize",
    "mu_adamw_workspace_size", "mu_adamw_step", "mu_qk_clip_workspace_size", "mu_qk_clip",
    "mu_status_string", "mu_last_error", "mu_version", "mu_profile_enable", "mu_profile_read", "mu_kernel_name",
)


class MuMatrix(ctypes.Structure):
    _fields_ = [
        ("param", ctypes.c_void_p), ("grad", ctypes.c_void_p), ("momentum", ctypes.c_void_p),
        ("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("dtype", ctypes.c_int32),
        ("num_heads", ctypes.c_int32), ("scale", ctypes.c_float), ("norm_out", ctypes.c_void_p),
        ("ortho_out", ctypes.c_void_p),
    ]


class MuMuonHparams(ctypes.Structure):
    _fields_ = [
        ("lr", ctypes.c_float), ("weight_decay", ctypes.c_float), ("mu", ctypes.c_float),
        ("nesterov", ctypes.c_int32), ("norm_eps", ctypes.c_float), ("ns_steps", ctypes.c_int32),
        ("coeffs", ctypes.POINTER(ctypes.c_float)), ("ns_precision", ctypes.c_int32),
        ("cautious_wd", ctypes.c_int32),
    ]


class MuOrtho(ctypes.Structure):
    _fields_ = [
        ("input", ctypes.c_void_p), ("output", ctypes.c_void_p), ("rows", ctypes.c_int64),
        ("cols", ctypes.c_int64), ("dtype", ctypes.c_int32), ("num_heads", ctypes.c_int32),
        ("norm_out", ctypes.c_void_p),
    ]


class MuTensor(ctypes.Structure):
    _fields_ = [
        ("param", ctypes.c_void_p), ("grad", ctypes.c_void_p), ("exp_avg", ctypes.c_void_p),
        ("exp_avg_sq", ctypes.c_void_p), ("numel", ctypes.c_int64), ("dtype", ctypes.c_int32),
        ("lr", ctypes.c_float), ("weight_decay", ctypes.c_float),
    ]


class MuAdamwHparams(ctypes.Structure):
    _fields_ = [("beta1", ctypes.c_float), ("beta2", ctypes.c_float), ("eps", ctypes.c_float),
                ("step", ctypes.c_int64)]


class MuQkPair(ctypes.Structure):
    _fields_ = [
        ("wq", ctypes.c_void_p), ("wk", ctypes.c_void_p), ("q_rows", ctypes.c_int64), ("k_rows", ctypes.c_int64),
        ("cols", ctypes.c_int64), ("q_heads", ctypes.c_int32), ("k_heads", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("pad0", ctypes.c_int32), ("max_logit", ctypes.c_void_p),
        ("gamma_out", ctypes.c_void_p),
    ]


class MuonError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{_status_text(status)} (status {status}): {detail}")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m newton_schulz_orthogonalized_amd.build` "
            "(there is no fallback path)")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    sz = ctypes.c_size_t
    lib.mu_muon_workspace_size.argtypes = [P(MuMatrix), ctypes.c_int32, P(MuMuonHparams), P(sz)]
    lib.mu_muon_step.argtypes = [P(MuMatrix), ctypes.c_int32, P(MuMuonHparams), ctypes.c_void_p, sz, ctypes.c_void_p]
    lib.mu_muon_step_noalloc.argtypes = [P(MuMatrix), ctypes.c_int32, P(MuMuonHparams), ctypes.c_void_p]
    lib.mu_ortho_workspace_size.argtypes = [P(MuOrtho), ctypes.c_int32, P(MuMuonHparams), P(sz)]
    lib.mu_muon_orthogonalize.argtypes = [P(MuOrtho), ctypes.c_int32, P(MuMuonHparams), ctypes.c_void_p, sz,
                                          ctypes.c_void_p]
    lib.mu_adamw_workspace_size.argtypes = [ctypes.c_int32, P(sz)]
    lib.mu_adamw_step.argtypes = [P(MuTensor), ctypes.c_int32, P(MuAdamwHparams), ctypes.c_void_p, sz,
                                  ctypes.c_void_p]
    lib.mu_qk_clip_workspace_size.argtypes = [P(MuQkPair), ctypes.c_int32, P(sz)]
    lib.mu_qk_clip.argtypes = [P(MuQkPair), ctypes.c_int32, ctypes.c_float, ctypes.c_void_p, sz, ctypes.c_void_p]
    lib.mu_status_string.argtypes = [ctypes.c_int]
    lib.mu_status_string.restype = ctypes.c_char_p
    lib.mu_last_error.argtypes = []
    lib.mu_last_error.restype = ctypes.c_char_p
    lib.mu_version.restype = ctypes.c_int
    lib.mu_profile_enable.argtypes = [ctypes.c_int]
    lib.mu_profile_read.argtypes = [ctypes.c_int, P(ctypes.c_double), P(ctypes.c_int64), P(ctypes.c_double),
                                    P(ctypes.c_double)]
    lib.mu_kernel_name.argtypes = [ctypes.c_int]
    lib.mu_kernel_name.restype = ctypes.c_char_p
    for name in ("mu_muon_workspace_size", "mu_muon_step", "mu_muon_step_noalloc", "mu_ortho_workspace_size",
                 "mu_muon_orthogonalize",
                 "mu_adamw_workspace_size", "mu_adamw_step", "mu_profile_enable", "mu_profile_read"):
        getattr(lib, name).restype = ctypes.c_int
    return lib


LIB = _load()


def _status_text(status: int) -> str:
    return LIB.mu_status_string(status).decode()


def _check(status: int) -> None:
    if status != MU_OK:
        raise MuonError(status, LIB.mu_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MU_BF16
    if t.dtype == torch.float32:
        return MU_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _require(t: torch.Tensor, what: str) -> None:
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous (the library takes dense row-major buffers)")


def muon_hparams(lr: float, weight_decay: float, mu: float = 0.95, nesterov: bool = True, norm_eps: float = 1e-7,
                 ns_steps: int = 5, coeffs: Optional[Sequence[Sequence[float]]] = None,
                 precision: str = "bf16", cautious_wd: bool = False):
    """Build mu_muon_hparams. Returns (struct, keepalive) - keep both alive for the call."""
    buf = None
    if coeffs is not None:
        flat = []
        for c in coeffs:
            c = list(c)
            if len(c) == 2:
                c.append(0.0)
            flat.extend(float(v) for v in c)
        if len(flat) != 3 * ns_steps:
            raise ValueError("coeffs must give (a, b[, c]) for each of ns_steps steps")
        buf = (ctypes.c_float * len(flat))(*flat)
    hp = MuMuonHparams(lr, weight_decay, mu, 1 if nesterov else 0, norm_eps, ns_steps,
                       ctypes.cast(buf, ctypes.POINTER(ctypes.c_float)) if buf is not None else None,
                       MU_NS_BF16 if precision == "bf16" else MU_NS_F32, 1 if cautious_wd else 0)
    return hp, buf


def matrices(params, grads, moms, heads=None, scales=None, norm_outs=None, ortho_outs=None):
    """Array of mu_matrix for lists of 2-D tensors."""
    n = len(params)
    arr = (MuMatrix * max(n, 1))()
    for i in range(n):
        p, g, m = params[i], grads[i], moms[i]
        for t, what in ((p, "param"), (g, "grad"), (m, "momentum")):
            _require(t, what)
        if p.dim() != 2 or g.shape != p.shape or m.shape != p.shape:
            raise ValueError("param, grad and momentum must be 2-D and of one shape")
        if m.dtype != torch.float32 or g.dtype != p.dtype:
            raise TypeError("momentum must be float32 and grad must share the param dtype")
        no = None if norm_outs is None else norm_outs[i]
        oo = None if ortho_outs is None else ortho_outs[i]
        if oo is not None and (oo.dtype != torch.float32 or oo.shape != p.shape or not oo.is_contiguous()):
            raise ValueError("ortho_out must be a contiguous float32 tensor of the param's shape")
        arr[i] = MuMatrix(_ptr(p), _ptr(g), _ptr(m), p.shape[0], p.shape[1], _dtype_code(p),
                          1 if heads is None else int(heads[i]), 1.0 if scales is None else float(scales[i]),
                          _ptr(no), _ptr(oo))
    return arr, n


def mu_muon_workspace_size(mats, n, hp) -> int:
    out = ctypes.c_size_t(0)
    _check(LIB.mu_muon_workspace_size(mats, n, ctypes.byref(hp), ctypes.byref(out)))
    return out.value


def mu_muon_step(mats, n, hp, workspace: Optional[torch.Tensor], stream=None) -> None:
    ws = 0 if workspace is None else workspace.data_ptr()
    nb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(LIB.mu_muon_step(mats, n, ctypes.byref(hp), ws, nb, _stream(stream)))


MU_NOALLOC_SCRATCH_BYTES = 64 << 20


def mu_muon_step_noalloc(mats, n, hp, stream=None) -> None:
    """mu_muon_step with the library's static per-GPU scratch as workspace."""
    _check(LIB.mu_muon_step_noalloc(mats, n, ctypes.byref(hp), _stream(stream)))


def orthos(inputs, outputs, heads=None, norm_outs=None):
    n = len(inputs)
    arr = (MuOrtho * max(n, 1))()
    for i in range(n):
        x, o = inputs[i], outputs[i]
        _require(x, "input")
        _require(o, "output")
        if x.dim() != 2 or o.shape != x.shape or o.dtype != x.dtype:
            raise ValueError("input and output must be 2-D, of one shape and dtype")
        no = None if norm_outs is None else norm_outs[i]
        arr[i] = MuOrtho(_ptr(x), _ptr(o), x.shape[0], x.shape[1], _dtype_code(x),
                         1 if heads is None else int(heads[i]), _ptr(no))
    return arr, n


def mu_ortho_workspace_size(xs, n, hp) -> int:
    out = ctypes.c_size_t(0)
    _check(LIB.mu_ortho_workspace_size(xs, n, ctypes.byref(hp), ctypes.byref(out)))
    return out.value


def mu_muon_orthogonalize(xs, n, hp, workspace: Optional[torch.Tensor], stream=None) -> None:
    ws = 0 if workspace is None else workspace.data_ptr()
    nb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(LIB.mu_muon_orthogonalize(xs, n, ctypes.byref(hp), ws, nb, _stream(stream)))


def tensors(params, grads, exp_avgs, exp_avg_sqs, lrs, wds):
    n = len(params)
    arr = (MuTensor * max(n, 1))()
    for i in range(n):
        p, g, m, v = params[i], grads[i], exp_avgs[i], exp_avg_sqs[i]
        for t, what in ((p, "param"), (g, "grad"), (m, "exp_avg"), (v, "exp_avg_sq")):
            _require(t, what)
        if g.shape != p.shape or m.shape != p.shape or v.shape != p.shape:
            raise ValueError("param, grad and states must share a shape")
        if m.dtype != torch.float32 or v.dtype != torch.float32 or g.dtype != p.dtype:
            raise TypeError("states must be float32 and grad must share the param dtype")
        arr[i] = MuTensor(_ptr(p), _ptr(g), _ptr(m), _ptr(v), p.numel(), _dtype_code(p), float(lrs[i]),
                          float(wds[i]))
    return arr, n


def mu_adamw_workspace_size(n: int) -> int:
    out = ctypes.c_size_t(0)
    _check(LIB.mu_adamw_workspace_size(n, ctypes.byref(out)))
    return out.value


def mu_adamw_step(ts, n, beta1: float, beta2: float, eps: float, step: int,
                  workspace: Optional[torch.Tensor], stream=None) -> None:
    hp = MuAdamwHparams(beta1, beta2, eps, step)
    ws = 0 if workspace is None else workspace.data_ptr()
    nb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(LIB.mu_adamw_step(ts, n, ctypes.byref(hp), ws, nb, _stream(stream)))


def qk_pairs(wqs, wks, max_logits, q_heads, k_heads, gamma_outs=None):
    n = len(wqs)
    arr = (MuQkPair * max(n, 1))()
    for i in range(n):
        wq, wk, ml = wqs[i], wks[i], max_logits[i]
        for t, what in ((wq, "wq"), (wk, "wk"), (ml, "max_logit")):
            _require(t, what)
        if wq.dim() != 2 or wk.dim() != 2 or wq.shape[1] != wk.shape[1]:
            raise ValueError("wq and wk must be 2-D with the same number of columns")
        if wk.dtype != wq.dtype or ml.dtype != torch.float32:
            raise TypeError("wk must share wq's dtype and max_logit must be float32")
        go = None if gamma_outs is None else gamma_outs[i]
        if go is not None:
            _require(go, "gamma_out")
        arr[i] = MuQkPair(_ptr(wq), _ptr(wk), wq.shape[0], wk.shape[0], wq.shape[1], int(q_heads[i]),
                          int(k_heads[i]), _dtype_code(wq), 0, _ptr(ml), _ptr(go))
    return arr, n


def mu_qk_clip_workspace_size(pairs, n) -> int:
    out = ctypes.c_size_t(0)
    _check(LIB.mu_qk_clip_workspace_size(pairs, n, ctypes.byref(out)))
    return out.value


def mu_qk_clip(pairs, n, tau: float, workspace: Optional[torch.Tensor], stream=None) -> None:
    ws = 0 if workspace is None else workspace.data_ptr()
    nb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(LIB.mu_qk_clip(pairs, n, float(tau), ws, nb, _stream(stream)))


def mu_version() -> int:
    return LIB.mu_version()


def mu_status_string(status: int) -> str:
    return _status_text(status)


def mu_last_error() -> str:
    return LIB.mu_last_error().decode()


def mu_profile_enable(on: bool) -> None:
    _check(LIB.mu_profile_enable(1 if on else 0))


def mu_profile_read(kernel: int) -> dict:
    ms = ctypes.c_double(0)
    n = ctypes.c_int64(0)
    fl = ctypes.c_double(0)
    by = ctypes.c_double(0)
    _check(LIB.mu_profile_read(kernel, ctypes.byref(ms), ctypes.byref(n), ctypes.byref(fl), ctypes.byref(by)))
    return {"kernel": LIB.mu_kernel_name(kernel).decode(), "ms": ms.value, "launches": n.value,
            "flops": fl.value, "bytes": by.value}


def mu_kernel_name(kernel: int) -> str:
    return LIB.mu_kernel_name(kernel).decode()


def workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    """A 256-byte aligned uint8 device buffer of at least nbytes (None for 0)."""
    if nbytes == 0:
        return None
    buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    off = (-buf.data_ptr()) % 256
    return buf[off:off + nbytes]


def tie_to_stream(buf: Optional[torch.Tensor], stream, current=None) -> None:
    """Keep a buffer allocated on the current stream alive for work queued on
    `stream` (a torch stream or a raw hipStream_t value): the caching
    allocator may otherwise hand its memory to the next allocation on the
    current stream as soon as the caller drops it, while the library's kernels
    on `stream` still read it. No-op for None or for the current stream."""
    if buf is None or stream is None:
        return
    if not isinstance(stream, torch.cuda.Stream):
        stream = torch.cuda.ExternalStream(int(stream), device=buf.device)
    cur = torch.cuda.current_stream(buf.device) if current is None else current
    if stream.cuda_stream != cur.cuda_stream:
        buf.record_stream(stream)
