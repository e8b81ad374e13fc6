"""bench.py's output contract: one JSON line with the fields the measurement record relies on.

The one-GPU refusal runs on the CPU; the full line needs the GPU (a short run on the smallest
workload, in a child process).
"""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def run_bench(*args, timeout=600):
    res = subprocess.run([sys.executable, BENCH, *args], cwd=ROOT, capture_output=True, text=True, timeout=timeout)
    lines = [ln for ln in res.stdout.splitlines() if ln.startswith("{")]
    return res, lines


def test_more_than_one_gpu_is_refused():
    res, lines = run_bench("--gpus", "2", timeout=120)
    assert res.returncode == 2
    assert len(lines) == 1
    out = json.loads(lines[0])
    assert out["n_gpus"] == 2 and "one GPU only" in out["error"]


@pytest.mark.gpu
def test_bench_line_carries_the_contract():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("[gpu-case] bench.py --workload b1 --steps 2 --warmup 1 --no-probe", flush=True)
    res, lines = run_bench("--workload", "b1", "--steps", "2", "--warmup", "1", "--no-probe")
    assert res.returncode == 0, res.stderr[-2000:]
    assert len(lines) == 1, res.stdout[-2000:]
    out = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in out, key
    assert out["n_gpus"] == 1 and out["steps"] == 2 and out["warmup"] == 1
    assert out["unit"] == "frames/s" and out["higher_is_better"] is True and out["vs_baseline"] is None
    # value is frames over the timed region: B·T·K over K·ms_per_step
    frames = out["config"]["batch"] * out["config"]["seq_len"]
    assert out["value"] == pytest.approx(frames / (out["ms_per_step"] / 1e3), rel=1e-6)
    assert out["config"]["workload"].startswith("b1:")
    roof = out["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in roof, key
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"], rel=1e-9)
    assert 0.0 < roof["frac"] < 1.0
    cpu = out["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1 and cpu["sample"]
    assert 0.0 < out["projection"]["frac"] < 2.0
