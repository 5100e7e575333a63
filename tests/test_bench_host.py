"""Host-side logic of bench.py (no GPU): the one-GPU guard, the kernel-source
hash that keys the committed traffic profiles, the profile lookup, and the
algorithmic byte and operation counts the rooflines divide by."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


def test_kernel_hash_ignores_comments_and_whitespace(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("int a = 1;  // one\n\n__global__ void k() {}\n")
    monkeypatch.setattr(bench, "KERNEL_SRC", str(src))
    h0 = bench.kernel_hash()
    src.write_text("// a comment\nint a = 1;\n   __global__ void k() {}   // other\n")
    assert bench.kernel_hash() == h0
    src.write_text("int a = 2;\n__global__ void k() {}\n")
    assert bench.kernel_hash() != h0


def test_traffic_is_read_only_for_the_current_source_and_kernel(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    h = bench.kernel_hash()
    (tmp_path / "traffic_w.txt").write_text(f"# header: not a field\nkernels_hip_sha256_16: {h}\nkernel: k_fused\n"
                                            "hbm_bytes_per_launch: 12345\n")
    assert bench.load_traffic("k_fused", "w") == 12345.0
    assert bench.load_traffic("k_stats", "w") is None      # another kernel
    assert bench.load_traffic("k_fused", "missing") is None  # no profile
    (tmp_path / "traffic_w.txt").write_text("kernels_hip_sha256_16: 0000000000000000\nkernel: k_fused\n"
                                            "hbm_bytes_per_launch: 12345\n")
    assert bench.load_traffic("k_fused", "w") is None      # taken on other kernel source


def test_committed_traffic_profiles_match_the_kernel_source():
    """Every committed traffic profile was taken on the current kernel source,
    so the benchmark reports measured traffic rather than null."""
    names = [f for f in os.listdir(os.path.join(ROOT, "profiles")) if f.startswith("traffic_")]
    assert names
    for f in names:
        wl = f[len("traffic_"):-len(".txt")]
        kv = dict(l.split(":", 1) for l in open(os.path.join(ROOT, "profiles", f)) if ":" in l and not l.startswith("#"))
        assert kv["kernels_hip_sha256_16"].strip() == bench.kernel_hash(), f
        assert bench.load_traffic(kv["kernel"].strip(), wl) is not None, f


class _W:
    def __init__(self, mode, gamma, V, dtype="bf16"):
        self.mode, self.gamma, self.vocab, self.dtype = mode, np.asarray(gamma), V, dtype
        self.batch, self.total_draft_rows = len(gamma), int(np.sum(gamma))


@pytest.mark.parametrize("dtype,s", [("bf16", 2), ("f32", 4)])
def test_algorithmic_bytes(dtype, s):
    V = 1000
    w = _W(0, [3, 0, 2], V, dtype)
    # stochastic: both rows of every drafted position, then 2 rows per
    # rejection and 1 per bonus for the draw
    rows, step = bench.algorithmic_bytes(w, np.array([1, 0, 2]))
    assert rows == 2 * 5 * V * s
    assert step == rows + (2 * 1 + 2) * V * s  # request 0 rejects; 1 and 2 take a bonus token
    # NKL: both rows of every position plus each request's bonus row
    w.mode = 2
    assert bench.algorithmic_bytes(w, None) == ((2 * 5 + 3) * V * s,) * 2
    # greedy family: the target rows only
    for mode in (1, 3, 4):
        w.mode = mode
        assert bench.algorithmic_bytes(w, None) == ((5 + 3) * V * s,) * 2


def test_consensus_operation_count():
    # K = 3: 3 rows x 4 plus 3 pairs x 9
    assert bench.cons_flops_per_element(3) == 39
    assert bench.cons_flops_per_element(2) == 17
    assert bench.cons_flops_per_element(4) == 70
