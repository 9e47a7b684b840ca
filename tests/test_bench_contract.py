"""bench.py's output contract: one JSON line with the metric, throughput,
timing, configuration, roofline and CPU-baseline fields, and a refusal of
more than one GPU.  The refusal is checked on the CPU; the JSON line comes
from a short default run (the long workload, 1 x 2^20 x 512 x 16 bf16) on the
GPU: the headline is the median of K steps each run right after a cache
flush, and the warm (back-to-back) figures ride along.  The CPU baseline of
that default run is skipped here (--no-cpu-baseline keeps the test short);
a separate short run checks the CPU-baseline fields."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.gpu
def test_default_run_prints_one_contract_line():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3",
                        "--warmup", "1", "--no-cpu-baseline"], capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["unit"] == "elem/s" and d["higher_is_better"] is True
    assert d["data"] == "synthetic" and d["vs_baseline"] is None
    cfg = d["config"]
    assert cfg["workload"] == "long"
    assert (cfg["batch"], cfg["seqlen"], cfg["dim"], cfg["dstate"]) == (1, 1 << 20, 512, 16)
    elems = cfg["batch"] * cfg["seqlen"] * cfg["dim"] * cfg["dstate"]
    assert d["value"] == pytest.approx(elems / (d["ms_per_step"] * 1e-3), rel=1e-6)
    assert d["warm_value"] == pytest.approx(elems / (d["warm_ms_per_step"] * 1e-3), rel=1e-6)
    roof = d["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in roof, k
    assert roof["bound"] in ("hbm", "mfma", "alu")
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"], rel=1e-9)
    assert 0.0 < roof["frac"] < 1.0
    assert d["cpu_baseline"] is None


@pytest.mark.gpu
def test_cpu_baseline_fields():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny",
                        "--steps", "3", "--warmup", "1"], capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    d = json.loads([ln for ln in r.stdout.splitlines() if ln.strip()][-1])
    cpu = d["cpu_baseline"]
    for k in ("value", "unit", "cores", "kind", "sample"):
        assert k in cpu, k
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1
