"""The benchmark's contract pieces that need no GPU: the one-GPU refusal, the roofline bound
choice and its fractions, and the algorithmic byte counts of the row kernels."""
import os
import subprocess
import sys

import pytest

import bench
import workloads as wk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "--gpus must be 1" in r.stderr and not r.stdout.strip()


@pytest.mark.parametrize("name,role,bound", [
    ("dsv3_ep64", "bwd_gate_up", "mfma"),      # 4 experts of thousands of rows: flop-bound
    ("dsv3_ep64", "gemm2_down", "mfma"),
    ("mid_t2048", "bwd_gate_up", "hbm"),       # weights and their gradients outweigh flops
    ("dsv3_e256_zipf", "gemm1_swiglu", "hbm"),
    ("dsv3_ep64_mxfp8", "mx_gemm1_swiglu", "mfma"),
])
def test_roofline_takes_the_binding_bound(name, role, bound):
    wl = wk.WORKLOADS[name]
    kind, flops = bench.step_work(wl, role)
    assert kind == "flop"
    ms = 1.0
    r = bench.roofline_of(wl, role, ms, 1.0, None)
    assert r["bound"] == bound
    peak = bench.PEAK_MXFP8_TFLOPS if role.startswith("mx_") else bench.PEAK_BF16_TFLOPS
    mfma_frac = flops / 1e-3 / 1e12 / peak
    if role.startswith("mx_"):           # no byte model for the MXFP8 products
        assert r["unit"] == "TFLOP/s" and r["frac"] == pytest.approx(mfma_frac, rel=1e-3)
        return
    nbytes = bench.gemm_bytes(wl, role, False)
    if wl.S and not wl.local_share:
        nbytes += bench.gemm_bytes(wl, role, True)
    hbm_frac = nbytes / 1e-3 / 1e9 / bench.PEAK_HBM_GBS
    assert r["mfma_frac"] == pytest.approx(mfma_frac, rel=1e-3)
    assert r["hbm_frac"] == pytest.approx(hbm_frac, rel=1e-3)
    # the binding bound is the one whose ideal time is longer, i.e. the larger fraction
    assert r["frac"] == pytest.approx(max(mfma_frac, hbm_frac), rel=1e-3)


def test_gemm_bytes_count_each_operand_once():
    wl = wk.WORKLOADS["dsv3_ep64"]
    H, I, R, E = wl.H, wl.I, wl.R, wl.E
    w1 = E * 2 * I * H * 2
    # dXp = dGU W1 and dW1 = dGU^T Xp: dGU, W1, Xp read; dXp, dW1 written
    assert bench.gemm_bytes(wl, "bwd_gate_up", False) == R * 2 * I * 2 + w1 + 2 * R * H * 2 + w1
    # GEMM1 + SwiGLU: Xp, W1 read; h and the g|u save written
    assert bench.gemm_bytes(wl, "gemm1_swiglu", False) == R * H * 2 + w1 + R * I * 2 + R * 2 * I * 2


def test_row_kernel_bytes():
    wl = wk.WORKLOADS["dsv3_ep64"]
    T, H, R, k = wl.T, wl.H, wl.R, wl.R // wl.T
    # each source row read once, every routed row written, pos read
    assert bench.role_work(wl, "dispatch", False) == ("byte", float(T * H * 2 + R * H * 2 + R * 4))
    # every routed row read once, the output written, pos and weights read
    assert bench.role_work(wl, "combine", False) == ("byte", float(R * H * 2 + T * H * 2 + T * k * 8))


def test_traffic_needs_matching_sources(tmp_path, monkeypatch):
    """Stored HBM traffic counts are reported only for the HIP sources they were taken on."""
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    (tmp_path / "mixture_experts_layer_39_amd" / "csrc").mkdir(parents=True)
    (tmp_path / "mixture_experts_layer_39_amd" / "csrc" / "k.hip").write_text("a")
    import json
    entry = {"workloads": {"w": {"r": {"hbm_bytes_per_launch": 123}}}}
    (tmp_path / "profiles" / "hbm_traffic.json").write_text(
        json.dumps({"kernel_source_digest": bench.kernel_source_digest(), **entry}))
    assert bench.measured_traffic("w", "r") == 123
    (tmp_path / "mixture_experts_layer_39_amd" / "csrc" / "k.hip").write_text("b")
    assert bench.measured_traffic("w", "r") is None


def test_traffic_needs_matching_ring_depth(tmp_path, monkeypatch):
    """Counts taken through the ring at one depth are not reported for another depth."""
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    (tmp_path / "mixture_experts_layer_39_amd" / "csrc").mkdir(parents=True)
    (tmp_path / "mixture_experts_layer_39_amd" / "csrc" / "k.hip").write_text("a")
    import json
    entry = {"ring_depth": {"w": 16}, "workloads": {"w": {"r": {"hbm_bytes_per_launch": 7}}}}
    (tmp_path / "profiles" / "hbm_traffic.json").write_text(
        json.dumps({"kernel_source_digest": bench.kernel_source_digest(), **entry}))
    assert bench.measured_traffic("w", "r", 16) == 7
    assert bench.measured_traffic("w", "r", 4) is None
    assert bench.measured_traffic("w", "r") is None
