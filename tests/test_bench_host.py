"""Host-side checks of bench.py's contract that need no GPU."""
import subprocess
import sys
from pathlib import Path

ROOT = Path(__file__).resolve().parents[1]


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_cpu_baseline_times_the_whole_oracle_forward():
    """The CPU baseline runs the oracle over every head and query tile of the workload and
    reports its wall-clock, the pairs it covered and the worker count it used."""
    sys.path.insert(0, str(ROOT))
    import bench
    from workloads.synth import WORKLOADS, make_inputs
    w = WORKLOADS["tiny"]
    r = bench.cpu_baseline(w, make_inputs(w), max_workers=2)
    assert r["kind"] == "oracle" and r["cores"] == 2 and r["seconds"] > 0
    assert r["ms_per_layer"] is not None and r["value"] > 0
    assert "216 executed pairs" in r["sample"]
