"""Builds libmuon_mi355x.so (gfx950) in the package directory with hipcc.

    python -m newton_schulz_orthogonalized_amd.build
    python -m newton_schulz_orthogonalized_amd.build --host-asan OUT.so

The second form builds a debugging variant whose host code (the C ABI:
validation, planning, table upload) is compiled with AddressSanitizer; the
device code is the same. Load it with the clang ASan runtime preloaded, e.g.
LD_PRELOAD=<rocm>/lib/llvm/lib/clang/<ver>/lib/linux/libclang_rt.asan-x86_64.so
ASAN_OPTIONS=detect_leaks=0, in place of the regular library.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmuon_mi355x.so")
SOURCES = ["capi.hip", "elementwise.hip", "ns_gemm.hip"]
# The benchmark's ceiling probe (an MFMA loop with clock stamps), a library of
# its own so that the optimizer library holds only the optimizer.
PROBE_LIB = os.path.join(HERE, "libmuon_probe.so")
PROBE_SOURCES = ["probe.hip"]
ARCH = "gfx950"
# Per-source extra flags. The Newton-Schulz GEMMs keep 256 accumulator AGPRs
# and two fragment buffers live; the register-minimising scheduler keeps the
# accumulators in place (no spills, no copies in the K loop).
EXTRA = {"ns_gemm.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-minreg"]}


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 instructions in any kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def compile_commands(objdir: str, sources=None) -> list:
    cmds = []
    for src in (SOURCES if sources is None else sources):
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmds.append([hipcc()] + COMMON + EXTRA.get(src, []) +
                    ["-I", os.path.join(os.path.dirname(HERE), "include"), "-c", os.path.join(CSRC, src), "-o", obj])
    return cmds


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}")
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l and "target-feature" not in l)
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = True, out: str = LIB, host_asan: bool = False, sources=None) -> str:
    import tempfile
    with tempfile.TemporaryDirectory(prefix="mu_build_") as objdir:
        cmds = compile_commands(objdir, sources)
        if host_asan:   # the host half of the C ABI only; the sanitizer never reaches device code
            for c in cmds:
                if c[c.index("-c") + 1].endswith("capi.hip"):
                    c[1:1] = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
        for c in cmds:
            _run(c, verbose)
        tmp = out + ".tmp"
        objs = [c[c.index("-o") + 1] for c in cmds]
        link = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
        if host_asan:
            link[1:1] = ["-Xarch_host", "-fsanitize=address", "-shared-libasan"]
        _run(link, verbose)
        os.replace(tmp, out)
    return out


if __name__ == "__main__":
    if len(sys.argv) == 3 and sys.argv[1] == "--host-asan":
        build(verbose=True, out=os.path.abspath(sys.argv[2]), host_asan=True)
    elif len(sys.argv) == 1:
        build(verbose=True)
        build(verbose=True, out=PROBE_LIB, sources=PROBE_SOURCES)
    else:
        sys.exit("usage: python -m newton_schulz_orthogonalized_amd.build [--host-asan OUT.so]")
    sys.exit(0)
