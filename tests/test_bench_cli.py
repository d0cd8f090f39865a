"""bench.py's host-side contract: the one-GPU refusal and the oracle baseline
record (on a tiny sample, so no GPU is needed)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_cpu_baseline_record():
    sys.path.insert(0, ROOT)
    import bench
    from synth import workloads
    wl = workloads.qwen_32b()
    rec = bench.cpu_baseline(wl, 2, 2)
    assert rec["kind"] == "oracle" and rec["unit"] == "tokens/s"
    assert rec["value"] > 0 and rec["cores"] >= 1 and rec["live_kv_gbps"] > 0
    assert rec["cpu_model"] and "2 of 512" in rec["sample"]
    # tokens/s of a full step from the sampled per-unit time
    assert abs(rec["value"] * rec["seconds_per_step"] - wl.batch) < 1e-6 * wl.batch
