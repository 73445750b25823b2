"""Host-side checks of bench.py: the oracle baseline leg (forked host workers) and the
one-GPU contract.  No GPU is used."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_oracle_baseline_workers_report_a_rate():
    """The baseline forks one worker per host core (at most 16), each generating its slices on
    the host and timing the oracle; on the single-slice workload every field is filled in."""
    import bench
    import kvsynth
    w = kvsynth.workload(1)
    r = bench.cpu_baseline(w, 1)
    assert r["kind"] == "oracle" and r["unit"] == "slice-tokens/s"
    assert 1 <= r["cores"] <= 16 and r["cores"] <= r["host_cpus"]
    assert r["value"] > 0 and r["csm_s"] > 0 and r["decode_us_per_step"] > 0
    assert "1 of 1 compressible" in r["sample"]


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU only" in p.stderr
