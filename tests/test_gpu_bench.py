"""bench.py end to end on the GPU: the one JSON line it prints keeps its
contract (fields, units, the value recomputable from the step time, the
roofline fraction from its own achieved and peak, the CPU baseline timed from
the oracle), for the headline workload and for the small fp32 one with the
CPU baseline leg enabled. Short runs: a few steps each."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def run_bench(*args, timeout=240):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, capture_output=True,
                       text=True, timeout=timeout)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [ln for ln in r.stdout.strip().splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    return json.loads(lines[0])


def common(d, steps, warmup):
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == steps and d["warmup"] == warmup
    assert d["higher_is_better"] is True and d["scaling"] == "weak" and d["vs_baseline"] is None
    assert "workload" in d["config"]
    r = d["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in r, key
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    assert d["value"] > 0 and d["ms_per_step"] > 0


def test_headline_line():
    d = run_bench("--steps", "5", "--warmup", "2", "--no-cpu-baseline", "--no-sclk")
    common(d, 5, 2)
    c = d["config"]
    assert c["workload"] == "gpt2_small_causal" and (c["B"], c["H"], c["N"], c["d"]) == (8, 12, 1024, 64)
    assert d["dtype"] == "bf16" and c["causal"] is True
    flop = 10 * 8 * 12 * 1024 ** 2 * 64 / 2
    assert abs(d["value"] - flop / (d["ms_per_step"] * 1e-3) / 1e12) <= 1e-3 * d["value"] + 1e-3
    r = d["roofline"]
    assert r["kernel"] == "bwd_fused_kernel" and r["peak"] == pytest.approx(2516.6, rel=1e-3)
    assert r["flop_per_launch"] == pytest.approx(flop)
    # the dominant launch is part of a step, so it cannot take longer than the step
    assert r["avg_launch_ms"] < d["ms_per_step"]


def test_fp32_line_with_cpu_baseline():
    d = run_bench("--workload", "tiny_fp32", "--steps", "3", "--warmup", "1", "--no-sclk", timeout=400)
    common(d, 3, 1)
    assert d["dtype"] == "fp32" and d["roofline"]["peak"] == pytest.approx(157.3, rel=1e-3)
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1 and cpu["unit"] == d["unit"]
    assert cpu["sample"]
