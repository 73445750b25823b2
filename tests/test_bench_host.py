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


def test_round_byte_counts():
    """The roofline's algorithmic bytes: a compressed slice reads its rows after the sinks once
    and writes its kept rows once, an outlier slice counts nothing; the out-of-place extras are
    the sinks of compressed slices and every row of outlier slices, read and written."""
    import bench
    from oracle import schedule as osched
    row = 2 * 128 * 2 + 4
    assert bench.ROW_BYTES == row
    lens_in = [65536, 65536, 1000]
    s_out = osched.round_length(65536, 16, 64, 256, 0.5)
    lens_out = [s_out, 65536, osched.round_length(1000, 16, 64, 256, 0.5)]
    mask = [0, 1, 0]
    want = ((65536 - 16) + (s_out - 16)) * row + ((1000 - 16) + (lens_out[2] - 16)) * row
    assert bench.csm_bytes(lens_in, lens_out, mask, 16) == want
    assert bench.csm_copy_bytes(lens_in, mask, 16) == 2 * (16 + 65536 + 16) * row
    # the 64K workload's round: 246 compressed slices, 14.5565 GB
    assert bench.csm_bytes([65536] * 256, [s_out] * 256, [0] * 246 + [1] * 10, 16) == 14556512736
