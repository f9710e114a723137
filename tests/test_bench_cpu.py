"""Host-side logic of bench.py (no GPU): the one-GPU guard, and the lookup of
recorded HBM traffic, which must follow the GEMM kernel source (a comment
edit keeps the record, a code edit voids it)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.fixture()
def tree(tmp_path, monkeypatch):
    csrc = tmp_path / "muon_newton_schulz_03_amd" / "csrc"
    csrc.mkdir(parents=True)
    for name in ("kernels.hip", "layout.h"):
        shutil.copy(os.path.join(ROOT, "muon_newton_schulz_03_amd", "csrc", name), csrc / name)
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    return tmp_path


def write_profile(tree, digest):
    (tree / "profiles" / "muon_step_w.md").write_text(
        "# summary\n\nkernel_code_sha256: %s\ntraffic_bytes_per_launch gemm_bf16_kernel<2>: 123\n"
        "traffic_bytes_per_launch gemm_bf16_kernel<0>: 45\n" % digest)


def test_recorded_traffic_follows_the_kernel_source(tree):
    assert bench.recorded_traffic("w", "gemm_bf16_kernel<2>") is None  # no summary
    write_profile(tree, bench.kernel_code_hash())
    assert bench.recorded_traffic("w", "gemm_bf16_kernel<2>") == 123
    assert bench.recorded_traffic("w", "gemm_bf16_kernel<0>") == 45
    assert bench.recorded_traffic("w", "gemm_bf16_kernel<1>") is None  # not recorded
    src = tree / "muon_newton_schulz_03_amd" / "csrc" / "kernels.hip"
    text = src.read_text()
    src.write_text(text + "\n// a comment changes nothing\n")
    assert bench.recorded_traffic("w", "gemm_bf16_kernel<2>") == 123
    src.write_text(text + "\nstatic int changed_code;\n")
    assert bench.recorded_traffic("w", "gemm_bf16_kernel<2>") is None


def test_committed_profiles_are_well_formed():
    """Every committed summary that records traffic carries a source digest
    and one line per GEMM kernel."""
    import re
    for name in os.listdir(os.path.join(ROOT, "profiles")):
        text = open(os.path.join(ROOT, "profiles", name)).read()
        if "traffic_bytes_per_launch" not in text:
            continue
        assert re.search(r"^kernel_code_sha256: [0-9a-f]{64}$", text, re.M), name
        for k in ("gemm_bf16_kernel<0>", "gemm_bf16_kernel<1>", "gemm_bf16_kernel<2>"):
            assert re.search(r"^traffic_bytes_per_launch " + re.escape(k) + r": \d+$", text, re.M), (name, k)
