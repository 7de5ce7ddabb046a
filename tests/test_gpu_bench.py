"""bench.py on a small workload, in a child process on the GPU: it prints
exactly one JSON line carrying the fields of the measurement record (the
metric, the step, the roofline of the dominant kernel with its traffic
field, the per-stage rooflines, the realized sparsity, the clocks)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_line_on_a_small_workload():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("case bench.py --workload tiny --steps 3 --warmup 1", flush=True)
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--workload", "tiny",
                        "--steps", "3", "--warmup", "1", "--no-cpu-baseline"],
                       cwd=ROOT, capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "stages", "realized", "warm", "dense", "hipblaslt_dense",
              "hipblaslt_bare_gemms", "clocks"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert d["config"]["workload"] == "tiny"
    roof = d["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in roof, k
    assert roof["bound"] in ("hbm", "mfma") and roof["achieved"] > 0 and roof["peak"] > 0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-9
    assert roof["traffic"] is None  # no counter profile is committed for this workload
    assert d["configs"] is None and d["cpu_baseline"] is None
