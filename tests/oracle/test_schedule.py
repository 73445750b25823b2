"""Pins for oracle.schedule against lengths derived by hand from Algorithm 1 (golden file)."""
import json
import os

import numpy as np

from oracle import csm, schedule


def _golden(golden_dir):
    with open(os.path.join(golden_dir, "schedule_trajectories.json")) as f:
        return json.load(f)


def test_single_rounds(golden_dir):
    for row in _golden(golden_dir)["single_round"]:
        assert schedule.round_length(row["s"], 16, 64, 256, row["r"]) == row["out"]


def test_algorithm1_trajectories(golden_dir):
    for row in _golden(golden_dir)["algorithm1"]:
        out = schedule.run_algorithm1(row["n"], row["R"], row["Gamma"], row["g"])
        assert abs(out["budget"] - row["budget"]) < 1e-9
        if "prefill" in row:
            assert out["prefill"] == row["prefill"]
        if "prefill_final" in row:
            assert len(out["prefill"]) - 1 == row["prefill_rounds"]
            assert out["prefill"][-1] == row["prefill_final"]
        assert [t[0] for t in out["triggers"]] == row["trigger_steps"]
        for t in out["triggers"]:
            assert abs(t[3] - row.get("trigger_r", 0.1)) < 1e-12
        if "final" in row:
            assert out["final"] == row["final"]


def test_round_length_agrees_with_a_real_round():
    rng = np.random.default_rng(9)
    for s, c, r in [(700, 64, 0.5), (531, 32, 0.19999999999999996), (333, 256, 0.35)]:
        K = rng.standard_normal((s, 4)); V = rng.standard_normal((s, 4)); N = np.ones(s, np.int64)
        _, _, _, s2, _ = csm.csm_round_slice(K, V, N, s, 16, 64, c, r, storage="f64")
        assert s2 == schedule.round_length(s, 16, 64, c, r)


def test_annealing():
    assert [round(schedule.annealed_r(j), 12) for j in range(10)] == \
        [0.5, 0.45, 0.4, 0.35, 0.3, 0.25, 0.2, 0.15, 0.1, 0.1]
