"""bench.py measures one GPU: asked for more, it exits with a message (CPU)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(args, env):
    e = dict(os.environ)
    e.update(env)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, env=e,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2, (r.returncode, r.stderr)
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_counter_traffic_only_for_profiled_workloads():
    """The roofline's counter traffic comes from the committed profiles only
    for a workload exactly as profiled: a density, batch-size or capacity
    override (whose traffic differs) reports none."""
    sys.path.insert(0, ROOT)
    import bench
    from activation_sparse_feed_gate_amd import synth

    W = synth.WORKLOADS
    w = W["ffn-2b"]
    got = bench._traffic("gate_twell", "gate_twell.hip", w, W)
    if got is None:
        pytest.skip("the committed profile predates the current gate_twell.hip")
    assert got > 0
    assert bench._traffic("gate_twell", "gate_twell.hip", w.with_(density=0.05), W) is None
    assert bench._traffic("gate_twell", "gate_twell.hip", w.with_(M=1024), W) is None
    assert bench._traffic("gate_twell", "gate_twell.hip", w, W, r_max_override=64) is None
    assert bench._traffic("no_such_kernel", "gate_twell.hip", w, W) is None
