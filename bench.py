#!/usr/bin/env python3
"""Benchmark of one optimizer step (Muon over every 2-D hidden weight + AdamW
over the rest) on a transformer-shaped parameter set, on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config llama_8b] [--coeffs cubic|quintic]

A step is one mu_muon_step over the whole Muon list (momentum, normalisation,
five Newton-Schulz steps, update) plus one mu_adamw_step over the whole AdamW
list, with every input resident in HBM. W untimed steps (by default at
least 3 and at least one second of them, so that short steps are timed at the
clocks a training loop settles at; the JSON reports the number run), then K timed steps
between two device synchronisations (`value`, ms per step; repeated calls
replay their launch sequence from a HIP graph, as in a training loop), then K
more timed steps with the library's profiler on, whose HIP events around each
launch on its launch stream give the per-kernel durations and the roofline.
Prints one JSON line.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Muon step ms per param set; NS TFLOP/s (% MFMA peak); AdamW GB/s"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 matrix
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E

# Per-step (a, b, c) of X <- a X + b (X X^T) X + c (X X^T)^2 X. cubic: the
# Newton-Schulz step of the Muon pages, 1.5 X - 0.5 X X^T X. quintic: the
# second-order Newton-Schulz iteration for the polar factor (the series of
# (X^T X)^(-1/2) about I cut after the quadratic term: 15/8, -10/8, 3/8), which
# exercises the A A^T pass of a quintic step with coefficients of known
# convergence; the pages name tuned quintic schedules but print no values.
COEFF_SCHEDULES = {"cubic": (1.5, -0.5, 0.0), "quintic": (1.875, -1.25, 0.375)}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps (default: at least 3, and at least --warmup-s seconds)")
    ap.add_argument("--warmup-s", type=float, default=1.0,
                    help="without --warmup: warm up for at least this long, so that the timed steps run at the "
                         "clocks a training loop settles at (short steps start at lower clocks)")
    ap.add_argument("--config", default="llama_8b")
    ap.add_argument("--ns-steps", type=int, default=5)
    ap.add_argument("--coeffs", default="cubic", choices=sorted(COEFF_SCHEDULES),
                    help="Newton-Schulz polynomial of every step")
    ap.add_argument("--precision", default="bf16", choices=["bf16", "f32"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the copy / library-GEMM ceiling measurement")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run a plain device copy of this many MiB first (counter calibration)")
    return ap.parse_args()


# the library's sources that decide what runs on the GPU: the kernels and the
# host planner (tile groups, schedules, launch shapes)
KERNEL_SOURCES = ("ns_gemm.hip", "elementwise.hip", "common.hpp", "launch.hpp", "capi.hip")
# the sources each profiled kernel class is built from, with the host planner
# that decides its launches (tile groups, schedule, persistent mode)
KERNEL_FILES = {"apply": ("ns_gemm.hip", "common.hpp", "launch.hpp", "capi.hip"),
                "gram": ("ns_gemm.hip", "common.hpp", "launch.hpp", "capi.hip")}


def source_digest(files=KERNEL_SOURCES) -> str:
    """Digest of kernel sources with comments and all whitespace removed, so
    that recorded counter figures stay attached to the code they measured
    (and survive reformatting)."""
    import re
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "newton_schulz_orthogonalized_amd", "csrc", f)) as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update("".join(src.split()).encode())
    return h.hexdigest()[:16]


def run_key(args) -> dict:
    """What decides a run's launches besides the sources: the parameter set and
    the Newton-Schulz schedule."""
    return {"workload": args.config, "coeffs": args.coeffs, "ns_steps": args.ns_steps, "precision": args.precision,
            "gramside": os.environ.get("MU_GRAMSIDE", "1")[:1] != "0"}


def traffic_from_profiles(kernel: str, run: dict):
    """HBM bytes per launch from committed counter summaries, if they were taken
    on the current sources of that kernel and on a run of the same parameter set
    and schedule; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{run['workload']}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_digest") != source_digest(KERNEL_FILES[kernel]):
        return None
    if d.get("run") != run:
        return None
    return d.get("bytes_per_launch")


def measure_ceilings(torch, device):
    """Measured ceilings on this GPU, next to the spec peaks: the HBM rate of a
    plain 2 GiB device-to-device copy (read + write bytes), and the vendor
    library's dense bf16 GEMM (torch.matmul, hipBLASLt) on the two product
    shapes of one Newton-Schulz step on a 4096 x 14336 matrix (the Gram
    X X^T counted as a full 2 m^2 n product here; operands contiguous)."""
    out = {}
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(reps):
            fn()
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / reps

    a = torch.empty(1 << 30, dtype=torch.bfloat16, device=device)
    b = torch.empty_like(a)
    a.fill_(1)
    ms = timed(lambda: b.copy_(a), 10)
    out["hbm_copy_gbs"] = 2 * a.numel() * 2 / (ms * 1e-3) / 1e9
    del a, b
    m, n = 4096, 14336
    x = torch.randn(m, n, device=device).to(torch.bfloat16)
    xt = x.t().contiguous()
    bm = torch.randn(m, m, device=device).to(torch.bfloat16)
    ms_g = timed(lambda: torch.matmul(x, xt), 10)
    ms_a = timed(lambda: torch.matmul(bm, x), 10)
    out["library_gemm_tflops"] = {"gram_4096x14336": 2.0 * m * m * n / (ms_g * 1e-3) / 1e12,
                                  "apply_4096x4096x14336": 2.0 * m * m * n / (ms_a * 1e-3) / 1e12}
    del x, xt, bm
    torch.cuda.empty_cache()
    out["mfma_bf16_loop"] = mfma_loop_ceiling()
    return out


def mfma_loop_ceiling(target_ms: float = 200.0):
    """The dense bf16 MFMA rate this GPU sustains with no memory traffic at all
    (every compute unit, one wave per SIMD, 16 independent 16x16x32 MFMA
    chains), and the shader clock during that loop (s_memtime cycles over the
    100 MHz s_memrealtime ticks, mean over waves). None if the probe library
    is not built."""
    import ctypes
    path = os.path.join(ROOT, "newton_schulz_orthogonalized_amd", "libmuon_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.probe_mfma_bf16.argtypes = [ctypes.c_double] + [ctypes.POINTER(ctypes.c_double)] * 3
    lib.probe_mfma_bf16.restype = ctypes.c_int
    tf, ms, ghz = ctypes.c_double(0), ctypes.c_double(0), ctypes.c_double(0)
    rc = lib.probe_mfma_bf16(target_ms, ctypes.byref(tf), ctypes.byref(ms), ctypes.byref(ghz))
    if rc != 0:
        return {"error": f"hip error {rc}"}
    return {"tflops": tf.value, "frac_of_spec": tf.value / PEAK_BF16_TFLOPS, "ms": ms.value,
            "shader_clock_ghz": ghz.value}


def time_qk_clip(ps, mu, args, torch, head_dim: int = 128):
    """QK-Clip (post-update per-head rescale) over the set's attention layers,
    timed on its own after the steps: every query head is given a max logit
    above tau, so every head is rescaled and the algorithmic traffic is one read
    and one write of all query and key weights. None if the set has no wq/wk."""
    import newton_schulz_orthogonalized_amd as nso
    from newton_schulz_orthogonalized_amd import _lib
    names = [e.name for e in ps.muon]
    pairs = [(names.index(n), names.index(n[:-2] + "wk")) for n in names
             if n.endswith(".wq") and n[:-2] + "wk" in names]
    if not pairs:
        return None
    wqs = [mu["p"][i] for i, _ in pairs]
    wks = [mu["p"][j] for _, j in pairs]
    qh = [w.shape[0] // head_dim for w in wqs]
    kh = [w.shape[0] // head_dim for w in wks]
    gen = torch.Generator(device=wqs[0].device).manual_seed(77)
    mls = [150.0 + 100.0 * torch.rand(h, generator=gen, device=wqs[0].device) for h in qh]
    ws = _lib.workspace(_lib.mu_qk_clip_workspace_size(*_lib.qk_pairs(wqs, wks, mls, qh, kh)), wqs[0].device)
    run = lambda: nso.qk_clip(wqs, wks, mls, q_heads=qh, k_heads=kh, tau=100.0, workspace=ws)
    run()
    torch.cuda.synchronize()
    _lib.mu_profile_enable(True)
    reps = max(1, args.steps)
    for _ in range(reps):
        run()
    torch.cuda.synchronize()
    _lib.mu_profile_enable(False)
    pr = _lib.mu_profile_read(_lib.MU_K_QKCLIP)
    nbytes = sum(2.0 * (a.numel() + b.numel()) * a.element_size() for a, b in zip(wqs, wks))
    ms = pr["ms"] / max(1, pr["launches"])
    gbs = nbytes / (ms * 1e-3) / 1e9 if ms > 0 else None
    return {"layers": len(pairs), "q_heads": qh[0], "k_heads": kh[0], "ms_per_launch": ms,
            "bytes_per_launch": nbytes, "gbs": gbs, "frac_hbm": (gbs / PEAK_HBM_GBS) if gbs else None}


def build_set(ps, set_index, device, torch):
    from workloads import device_normal, seed_for
    dt = torch.bfloat16 if ps.dtype == "bf16" else torch.float32
    mu = {"p": [], "g": [], "m": [], "heads": []}
    for j, e in enumerate(ps.muon):
        s = seed_for(set_index, j)
        mu["p"].append(device_normal(e.shape, s, ps.weight_std, dt, device))
        mu["g"].append(device_normal(e.shape, s + 500000, ps.grad_std, dt, device))
        mu["m"].append(device_normal(e.shape, s + 900000, ps.mom_std, torch.float32, device))
        mu["heads"].append(e.heads)
    aw = {"p": [], "g": [], "m": [], "v": []}
    for j, e in enumerate(ps.adamw):
        s = seed_for(set_index, 100 + j)
        aw["p"].append(device_normal(e.shape, s, ps.weight_std, dt, device))
        aw["g"].append(device_normal(e.shape, s + 500000, ps.grad_std, dt, device))
        aw["m"].append(torch.zeros(e.shape, dtype=torch.float32, device=device))
        aw["v"].append(torch.zeros(e.shape, dtype=torch.float32, device=device))
    return mu, aw


def cpu_baseline(ps, set_index, ns_steps, coeffs):
    """The CPU oracle, as it stands, on a bounded sample of the same workload,
    scaled to one whole parameter set by algorithmic work."""
    import numpy as np
    from oracle import muon_oracle as O
    from workloads import host_normal
    try:
        from threadpoolctl import threadpool_info
        cores = max([int(i.get("num_threads", 1)) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    # sample: the set's Muon matrices in order (layer 0 first) until about 15 s
    # of float64 work (all seven of layer 0 but the last on the 8B set), plus
    # 8M AdamW elements
    from workloads import MuonEntry, ParamSet
    budget_s, t_muon, picked = 15.0, 0.0, []
    for k, e in enumerate(ps.muon):
        if t_muon >= budget_s:
            break
        w = host_normal(e.shape, 777 + k, ps.weight_std)
        g = host_normal(e.shape, 778 + k, ps.grad_std)
        m = host_normal(e.shape, 779 + k, ps.mom_std)
        t0 = time.perf_counter()
        O.muon_step_ref(w, g, m, lr=0.02, weight_decay=0.01, heads=e.heads, coeffs=coeffs)
        t_muon += time.perf_counter() - t0
        picked.append(e)
    sample = ParamSet("sample", [MuonEntry(e.name, e.shape, e.heads) for e in picked])
    n_aw = min(8 << 20, max(1, ps.adamw_elems()))
    t_aw = 0.0
    if ps.adamw:
        p, g = host_normal(n_aw, 1, 0.02), host_normal(n_aw, 2, 1e-3)
        z = np.zeros(n_aw)
        t0 = time.perf_counter()
        O.adamw_ref(p, g, z, z, lr=0.02, weight_decay=0.01, beta1=0.9, beta2=0.95, eps=1e-8, step=1)
        t_aw = time.perf_counter() - t0
    nq = sum(1 for c in coeffs if c[2] != 0.0)
    muon_scale = ps.ns_flops(ns_steps, nq) / sample.ns_flops(ns_steps, nq)
    aw_scale = ps.adamw_elems() / n_aw if ps.adamw else 0.0
    est_ms = 1e3 * (t_muon * muon_scale + t_aw * aw_scale)
    counts = {}
    for e in picked:
        key = f"{e.shape[0]}x{e.shape[1]}" + (f"/{e.heads}h" if e.heads > 1 else "")
        counts[key] = counts.get(key, 0) + 1
    desc = ", ".join(f"{c} x {k}" for k, c in counts.items())
    desc = f"the first {len(picked)} of {len(ps.muon)}: {desc}"
    return {"value": est_ms, "unit": "ms", "cores": cores, "kind": "oracle",
            "sample": (f"float64 numpy oracle on Muon matrices [{desc}] ({t_muon:.2f} s) scaled by Newton-Schulz "
                       f"flops x{muon_scale:.1f}, plus AdamW on {n_aw} elements ({t_aw:.2f} s) scaled by "
                       f"element count x{aw_scale:.1f}; measured {t_muon + t_aw:.1f} s of CPU work")}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark times one GPU: the library has no multi-GPU path "
                                   "(each GPU would run its own share of the matrices)",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)
    import newton_schulz_orthogonalized_amd as nso
    from newton_schulz_orthogonalized_amd import _lib
    from workloads import PARAM_SETS

    device = torch.device("cuda", 0)
    torch.cuda.set_device(device)
    set_index = list(PARAM_SETS).index(args.config)
    ps = PARAM_SETS[args.config]()
    precision = args.precision if ps.dtype == "bf16" else "f32"
    print(f"[bench] building {args.config}: {len(ps.muon)} Muon matrices ({ps.muon_elems()} elems), "
          f"{len(ps.adamw)} AdamW tensors ({ps.adamw_elems()} elems)", file=sys.stderr, flush=True)
    mu, aw = build_set(ps, set_index, device, torch)
    coeffs = [COEFF_SCHEDULES[args.coeffs]] * args.ns_steps
    ws_bytes = nso.muon_workspace_bytes(mu["p"], mu["g"], mu["m"], heads=mu["heads"], ns_steps=args.ns_steps,
                                        coeffs=coeffs, precision=precision)
    ws = _lib.workspace(ws_bytes, device)
    aw_ws = _lib.workspace(_lib.mu_adamw_workspace_size(len(aw["p"])), device)
    torch.cuda.synchronize()
    print(f"[bench] workspace {ws_bytes / 2**30:.1f} GiB, allocated {torch.cuda.memory_allocated() / 2**30:.1f} GiB",
          file=sys.stderr, flush=True)

    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device=device)
        b = torch.empty_like(a)
        a.fill_(1)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    state = {"t": 0}

    def step():
        state["t"] += 1
        nso.muon_step(mu["p"], mu["g"], mu["m"], lr=0.02, weight_decay=0.01, heads=mu["heads"],
                      ns_steps=args.ns_steps, coeffs=coeffs, precision=precision, workspace=ws)
        if aw["p"]:
            nso.adamw_step(aw["p"], aw["g"], aw["m"], aw["v"], lr=0.02, weight_decay=0.01, beta1=0.9,
                           beta2=0.95, eps=1e-8, step=state["t"], workspace=aw_ws)

    tw = time.perf_counter()
    done = 0
    while True:
        step()
        torch.cuda.synchronize()
        done += 1
        if args.warmup is not None:
            print(f"[bench] warmup step {done}/{args.warmup} done", file=sys.stderr, flush=True)
            if done >= args.warmup:
                break
        elif done >= 3 and time.perf_counter() - tw >= args.warmup_s:
            break
    args.warmup = done
    print(f"[bench] {done} warm-up steps in {time.perf_counter() - tw:.3f} s", file=sys.stderr, flush=True)

    # Timed region 1: the steps as a training loop runs them (a repeated call
    # replays its launch sequence from a HIP graph). `value` comes from here.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    print(f"[bench] {args.steps} timed steps in {elapsed:.3f} s", file=sys.stderr, flush=True)
    # Timed region 2: the same number of steps with the library's profiler on,
    # which records HIP events around every kernel on its launch stream (and
    # launches each kernel itself instead of replaying a graph); the
    # per-kernel durations and the roofline come from here.
    _lib.mu_profile_enable(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed_prof = time.perf_counter() - t1
    _lib.mu_profile_enable(False)
    prof = {_lib.mu_kernel_name(k): _lib.mu_profile_read(k) for k in range(_lib.MU_K_COUNT)}
    # host time to issue one step with the GPU idle (no wait on earlier work)
    issue = []
    for _ in range(5):
        torch.cuda.synchronize()
        ti = time.perf_counter()
        step()
        issue.append(time.perf_counter() - ti)
    torch.cuda.synchronize()
    host_ms = 1e3 * sorted(issue)[len(issue) // 2]
    print(f"[bench] {args.steps} profiled steps in {elapsed_prof:.3f} s", file=sys.stderr, flush=True)

    ms_step = 1e3 * elapsed / max(1, args.steps)
    K = max(1, args.steps)
    ns_kinds = ("gram", "gram2", "apply", "ns_fused")
    ns_ms = sum(prof[k]["ms"] for k in ns_kinds) / K
    ns_flops = sum(prof[k]["flops"] for k in ns_kinds) / K
    peak = PEAK_BF16_TFLOPS if precision == "bf16" else PEAK_F32_TFLOPS
    ns_tflops = ns_flops / (ns_ms * 1e-3) / 1e12 if ns_ms > 0 else 0.0
    # the plain iteration's flops (every step a Gram and an apply on X); the
    # library's Gram-side steps reach the same result with fewer, so this
    # rate is the method's work retired per second, not a kernel's rate
    method_flops = ps.ns_flops(args.ns_steps, sum(1 for c in coeffs if c[2] != 0.0))
    ns_method_tflops = method_flops / (ns_ms * 1e-3) / 1e12 if ns_ms > 0 else 0.0
    adamw_gbs = prof["adamw"]["bytes"] / (prof["adamw"]["ms"] * 1e-3) / 1e9 if prof["adamw"]["ms"] > 0 else None
    prep_gbs = prof["prep"]["bytes"] / (prof["prep"]["ms"] * 1e-3) / 1e9 if prof["prep"]["ms"] > 0 else None
    kernels = {k: {"ms_per_launch": (v["ms"] / v["launches"]) if v["launches"] else None,
                   "launches_per_step": v["launches"] / K, "ms_per_step": v["ms"] / K} for k, v in prof.items()}
    # dominant kernel: the class with the most time
    dom = max(("gram", "apply", "gram2", "ns_fused", "prep", "adamw"), key=lambda k: prof[k]["ms"])
    d = prof[dom]
    if dom in ("gram", "apply", "gram2"):
        achieved = d["flops"] / (d["ms"] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak}
    else:
        achieved = d["bytes"] / (d["ms"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS}
    roof["kernel"] = dom
    roof["ms_per_launch"] = d["ms"] / max(1, d["launches"])
    roof["traffic"] = traffic_from_profiles(dom, run_key(args))

    out = {
        "metric": METRIC, "value": ms_step, "unit": "ms", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": precision, "data": "synthetic",
        "config": {"workload": f"{args.config}: Muon over {len(ps.muon)} matrices ({ps.muon_elems()} elements), "
                               f"AdamW over {len(ps.adamw)} tensors ({ps.adamw_elems()} elements)"
                               + ("" if args.coeffs == "cubic" else f"; {args.coeffs} Newton-Schulz steps"),
                   "muon_matrices": len(ps.muon), "adamw_tensors": len(ps.adamw),
                   "ns_steps": args.ns_steps, "ns_coeffs": list(COEFF_SCHEDULES[args.coeffs]),
                   "ns_precision": precision, "parallelism": "single-gpu"},
        "ms_per_step_profiled": 1e3 * elapsed_prof / max(1, args.steps),
        # host time to issue one step (Python binding + C ABI + launches, median
        # of five issued onto an idle GPU) and the summed kernel time of one
        # step: host_ms_per_step below kernel_ms_per_step means the timed
        # steps were bound by the GPU, not by issuing them
        "host_ms_per_step": host_ms,
        "kernel_ms_per_step": sum(v["ms"] for v in prof.values()) / K,
        "muon_ms_per_step": sum(prof[k]["ms"] for k in ("prep", "norm", "rescale", "gram", "gram2", "apply", "finish",
                                                          "ns_fused")) / K,
        "adamw_ms_per_step": prof["adamw"]["ms"] / K,
        "ns_ms_per_step": ns_ms, "ns_tflops": ns_tflops, "ns_frac_peak": ns_tflops / peak,
        "ns_flops_per_step": ns_flops, "ns_method_flops_per_step": method_flops,
        "ns_method_tflops": ns_method_tflops,
        "adamw_gbs": adamw_gbs, "adamw_frac_hbm": (adamw_gbs / PEAK_HBM_GBS) if adamw_gbs else None,
        "prep_gbs": prep_gbs, "prep_frac_hbm": (prep_gbs / PEAK_HBM_GBS) if prep_gbs else None,
        "kernels": kernels, "roofline": roof, "source_digest": source_digest(),
    }
    out["qk_clip"] = time_qk_clip(ps, mu, args, torch)
    if not args.no_ceilings:
        print("[bench] measuring copy, library-GEMM and MFMA-loop ceilings", file=sys.stderr, flush=True)
        out["ceilings"] = measure_ceilings(torch, device)
        loop = out["ceilings"].get("mfma_bf16_loop") or {}
        if roof["bound"] == "mfma" and precision == "bf16" and loop.get("tflops"):
            # the same kernel against the rate a pure MFMA loop reaches on this GPU
            roof["frac_of_measured_ceiling"] = roof["achieved"] / loop["tflops"]
            out["ns_frac_of_measured_ceiling"] = ns_tflops / loop["tflops"]
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(ps, set_index, args.ns_steps, coeffs)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
