"""The benchmark's host-side contract, on the CPU: it refuses more than one
GPU with a message, and the HBM-traffic figure it reports comes from the
committed counter summary only while the apply kernel's sources are the ones
that summary was taken on (comments and formatting aside) and only for the
parameter set and schedule it was taken on."""

import json
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


@pytest.fixture
def tree(tmp_path, monkeypatch):
    """A copy of the kernel sources and the traffic summary, with bench.ROOT on it."""
    src = os.path.join(ROOT, "newton_schulz_orthogonalized_amd", "csrc")
    dst = tmp_path / "newton_schulz_orthogonalized_amd" / "csrc"
    shutil.copytree(src, dst)
    (tmp_path / "profiles").mkdir()
    shutil.copy(os.path.join(ROOT, "profiles", "traffic_apply_llama_8b.json"), tmp_path / "profiles")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    return dst


def test_digest_ignores_comments_and_whitespace_only(tree):
    before = bench.source_digest(bench.KERNEL_FILES["apply"])
    p = tree / "ns_gemm.hip"
    s = p.read_text()
    p.write_text("// a new comment\n" + s.replace("    ", "\t").replace("\n", "  \n\n") + "\n/* trailing */\n")
    assert bench.source_digest(bench.KERNEL_FILES["apply"]) == before
    p.write_text(s.replace("constexpr int NS = 4;", "constexpr int NS = 3;", 1))
    assert bench.source_digest(bench.KERNEL_FILES["apply"]) != before


def test_traffic_figure_follows_the_apply_sources(tree):
    with open(os.path.join(ROOT, "profiles", "traffic_apply_llama_8b.json")) as f:
        recorded = json.load(f)
    if recorded["kernel_source_digest"] != bench.source_digest(bench.KERNEL_FILES["apply"]):
        pytest.skip("the committed traffic summary predates the current apply sources")
    run = recorded["run"]
    assert bench.traffic_from_profiles("apply", run) == pytest.approx(recorded["bytes_per_launch"])
    # another parameter set or schedule has other launches: no figure
    for k, v in (("workload", "gpt2_small"), ("coeffs", "quintic"), ("ns_steps", 6), ("gramside", False)):
        assert bench.traffic_from_profiles("apply", dict(run, **{k: v})) is None
    # a change to a file the apply kernel is built from drops the figure ...
    p = tree / "common.hpp"
    p.write_text(p.read_text() + "\nconstexpr int UNUSED_FOR_TEST = 1;\n")
    assert bench.traffic_from_profiles("apply", run) is None
    # ... a change to a file it is not built from does not
    p.write_text(p.read_text().replace("\nconstexpr int UNUSED_FOR_TEST = 1;\n", ""))
    e = tree / "elementwise.hip"
    e.write_text(e.read_text() + "\n// unrelated\nstatic int unrelated_for_test;\n")
    assert bench.traffic_from_profiles("apply", run) == pytest.approx(recorded["bytes_per_launch"])
