"""The benchmark's output contract: one JSON line with the fields the
measurement reports (throughput, the attention kernel's roofline object and
the oracle's CPU baseline), checked on the tiny workload (GPU), and its
refusal of more than one GPU (CPU)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args, timeout=240):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=timeout)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2", timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_kernel_instance_names():
    sys.path.insert(0, ROOT)
    import bench
    assert bench.attn_kernel_name(128, 4, 75600) == "bsa::attn_fwd_kernel<128, true, false, false>"
    assert bench.attn_kernel_name(128, 4, 144126) == "bsa::attn_fwd_kernel<128, true, true, false>"
    assert bench.attn_kernel_name(128, 2, 139262) == "bsa::attn_fwd_kernel<128, true, false, true>"
    assert bench.attn_kernel_name(128, 2, 139263) == "bsa::attn_fwd_kernel<128, false, false, false>"
    assert bench.attn_kernel_name(128, 1, 139262) == "bsa::attn_fwd_kernel<128, false, false, false>"
    assert bench.attn_kernel_name(64, 8, 2048) == "bsa::attn_fwd_kernel<64, true, false, false>"
    assert bench.attn_kernel_name(64, 4, 2048) == "bsa::attn_fwd_kernel<64, true, false, true>"
    assert bench.attn_kernel_name(64, 4, 2046) == "bsa::attn_fwd_kernel<64, false, false, false>"
    assert bench.attn_kernel_name(64, 2, 2048) == "bsa::attn_fwd_kernel<64, false, false, false>"


@pytest.mark.gpu
def test_bench_line_on_the_tiny_workload():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("case bench line tiny_2x32x32", flush=True)
    r = _run("--workload", "tiny_2x32x32", "--steps", "3", "--warmup", "1")
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1
    rec = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config"):
        assert key in rec, key
    assert rec["n_gpus"] == 1 and rec["steps"] == 3 and rec["warmup"] == 1
    assert rec["ms_per_step_graph"] > 0    # the step replayed from a captured graph
    assert rec["value"] > 0 and rec["ms_per_step"] > 0 and rec["higher_is_better"] is True
    assert rec["config"]["workload"].startswith("tiny_2x32x32")
    roof = rec["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in roof, key
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s"
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert roof["traffic"] is None  # the counter runs cover the headline workload only
    assert roof["peak_measured"] > 0 and roof["peak_measured_low_entropy"] > 0
    assert abs(roof["frac_measured"] - roof["achieved"] / roof["peak_measured"]) < 1e-3
    p10, p50, p90 = rec["attn_ms_p10_p50_p90"]
    assert rec["attn_ms_per_call"] == p50                     # the median
    cpu = rec["cpu_baseline"]
    for key in ("value", "unit", "cores", "kind", "sample", "seconds_per_head",
                "extrapolated_seconds_all_heads", "extrapolation", "one_thread"):
        assert key in cpu, key
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["unit"] == rec["unit"]
    assert cpu["one_thread"]["cores"] == 1 and cpu["one_thread"]["value"] > 0


def test_traffic_record_keyed_on_code(tmp_path, monkeypatch):
    """The committed counter runs stay valid across comment edits of the
    attention source and are dropped by any code change."""
    sys.path.insert(0, ROOT)
    import bench
    src = open(bench.ATTN_SRC).read()
    base = bench.attn_build_sha()
    p = tmp_path / "attn_fwd.hip"
    monkeypatch.setattr(bench, "ATTN_SRC", str(p))
    p.write_text(src.replace("// ", "// (reworded) ", 3) + "\n// a trailing note\n\n")
    assert bench.attn_build_sha() == base
    p.write_text(src.replace("constexpr int NBUF = 3;", "constexpr int NBUF = 4;"))
    assert bench.attn_build_sha() != base


@pytest.mark.gpu
def test_mfma_peak_report():
    """The matrix-instruction probe's report: a rate per grid size, none
    above the published peak."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("case bench --mfma-peak", flush=True)
    r = _run("--mfma-peak", "--reps", "2")
    assert r.returncode == 0, r.stderr[-2000:]
    rep = json.loads(r.stdout.strip().splitlines()[-1])
    assert set(rep["best_tflops"]) == {"random", "low entropy"}
    assert all(v > 100 for v in rep["best_tflops"].values())
    assert all(0 < p["tflops"] <= rep["peak_spec"] for p in rep["points"])
    assert {p["operands"] for p in rep["points"]} == {"random", "low entropy"}
