"""Pins for oracle.csm (one CSM round): hand-worked cases and invariants.

Sources: Chelsea review, section 三, 分块软匹配算法 steps 1-4; CentroidKV page,
分块软匹配 (CSM) and 聚合.
"""
import json
import os

import numpy as np
import pytest
from scipy.spatial.distance import cdist

from oracle import bf16, csm, schedule


def _load_cases(golden_dir):
    with open(os.path.join(golden_dir, "csm_tiny_cases.json")) as f:
        return json.load(f)["cases"]


def test_hand_worked_cases(golden_dir):
    for case in _load_cases(golden_dir):
        K = np.array(case["K"], dtype=np.float64)
        V = np.array(case["V"], dtype=np.float64)
        N = np.array(case["N"], dtype=np.int64)
        s = K.shape[0]
        exp = case["expect"]
        K2, V2, N2, s2, taps = csm.csm_round_slice(K, V, N, s, case["n1"], case["n2"],
                                                   case["c"], case["r"], storage="f64")
        name = case["name"]
        assert s2 == exp["s"], name
        assert taps["src_pos"].tolist() == exp["src_pos"], name
        assert N2[:s2].tolist() == exp["N"], name
        np.testing.assert_allclose(K2[:s2], np.array(exp["K"]), rtol=0, atol=1e-12, err_msg=str(name))
        np.testing.assert_allclose(V2[:s2], np.array(exp["V"]), rtol=0, atol=1e-12, err_msg=str(name))
        got_b = [t["best_b"].tolist() for t in taps["chunks"] if "best_b" in t]
        got_sel = [t["selected"].tolist() for t in taps["chunks"] if "selected" in t]
        assert got_b == exp["best_b"], name
        assert got_sel == exp["selected"], name


def test_cosine_matches_scipy():
    rng = np.random.default_rng(1)
    a = rng.standard_normal((37, 16))
    b = rng.standard_normal((29, 16))
    S = csm.cosine_matrix(a, b)
    np.testing.assert_allclose(S, 1.0 - cdist(a, b, metric="cosine"), atol=1e-13)


def test_equal_rows_score_identically():
    """The similarity depends on the two rows' values only, so rows with equal values score
    bit-identically against everything (ties in the definition stay exact ties), whatever
    their position and the block shapes (fp32-valued data, whose products are not exact)."""
    rng = np.random.default_rng(7)
    for _ in range(200):
        nA, nB, d = int(rng.integers(2, 257)), int(rng.integers(2, 257)), int(rng.choice([64, 128]))
        a = rng.standard_normal((nA, d)).astype(np.float32).astype(np.float64)
        b = rng.standard_normal((nB, d)).astype(np.float32).astype(np.float64)
        j, j2 = sorted(rng.choice(nB, 2, replace=False))
        i, i2 = sorted(rng.choice(nA, 2, replace=False))
        b[j2], a[i2] = b[j], a[i]
        S = csm.cosine_matrix(a, b)
        assert np.array_equal(S[:, j], S[:, j2]) and np.array_equal(S[i], S[i2])


def test_cosine_special_values_and_scale_invariance():
    e = np.eye(4)
    S = csm.cosine_matrix(e, np.vstack([e[0] * 3.0, -e[0], e[1]]))
    assert S[0, 0] == pytest.approx(1.0) and S[0, 1] == pytest.approx(-1.0)
    assert S[0, 2] == 0.0 and S[1, 2] == pytest.approx(1.0)
    rng = np.random.default_rng(2)
    a, b = rng.standard_normal((8, 5)), rng.standard_normal((6, 5))
    np.testing.assert_allclose(csm.cosine_matrix(a * 7.5, b * 0.01),
                               csm.cosine_matrix(a, b), atol=1e-14)


def test_merge_count_guard():
    # 0.5 - 0.05*6 is 0.19999999999999996 in fp64; the guard keeps floor(0.2*L/2) exact.
    r6 = 0.5 - 0.05 * 6
    assert r6 < 0.2
    for L in (10, 20, 40, 80, 100, 160, 200, 256):
        assert csm.merge_count(r6, L) == (L // 10)
    assert csm.merge_count(0.5, 256) == 64
    assert csm.merge_count(0.5, 176) == 44
    assert csm.merge_count(1.0, 1) == 0
    assert csm.merge_count(1.0, 3) == 1


def _random_slice(rng, s, d, cap=None, rho=0.9, degrees=False):
    cap = s if cap is None else cap
    K = np.zeros((cap, d))
    k = rng.standard_normal(d)
    for t in range(s):
        k = rho * k + np.sqrt(1 - rho * rho) * rng.standard_normal(d)
        K[t] = k
    V = np.zeros((cap, d))
    V[:s] = rng.standard_normal((s, d))
    N = np.zeros(cap, dtype=np.int64)
    N[:s] = rng.integers(1, 6, size=s) if degrees else 1
    return K, V, N


@pytest.mark.parametrize("s,c", [(600, 64), (1000, 256), (97, 16), (81, 8)])
def test_r0_is_identity(s, c):
    rng = np.random.default_rng(s)
    K, V, N = _random_slice(rng, s, 16, cap=s + 5)
    K = bf16.round_to_bf16(K)
    V = bf16.round_to_bf16(V)
    K2, V2, N2, s2, _ = csm.csm_round_slice(K, V, N, s, 16, 64 if s > 200 else 4, c, 0.0)
    assert s2 == s
    assert np.array_equal(K2, K) and np.array_equal(V2, V) and np.array_equal(N2, N)


@pytest.mark.parametrize("r", [0.1, 0.3, 0.5, 0.77, 1.0])
def test_degree_sum_first_moments_and_compaction(r):
    rng = np.random.default_rng(int(r * 100))
    s, n1, n2, c, d = 1500, 16, 64, 128, 8
    K, V, N = _random_slice(rng, s, d, cap=s, degrees=True)
    K2, V2, N2, s2, taps = csm.csm_round_slice(K, V, N, s, n1, n2, c, r, storage="f64")
    # sum of degrees conserved exactly
    assert int(N2[:s2].sum()) == int(N[:s].sum())
    # first moments conserved (degree-weighted mean is the only weighting that does this)
    np.testing.assert_allclose((N2[:s2, None] * K2[:s2]).sum(0), (N[:s, None] * K[:s]).sum(0),
                               rtol=1e-10, atol=1e-9)
    np.testing.assert_allclose((N2[:s2, None] * V2[:s2]).sum(0), (N[:s, None] * V[:s]).sum(0),
                               rtol=1e-10, atol=1e-9)
    src = taps["src_pos"]
    assert np.all(np.diff(src) > 0)
    assert np.array_equal(src[:n1], np.arange(n1))
    assert np.array_equal(src[-n2:], np.arange(s - n2, s))
    assert np.array_equal(K2[:n1], K[:n1]) and np.array_equal(K2[s2 - n2:s2], K[s - n2:s])
    assert np.array_equal(V2[s2 - n2:s2], V[s - n2:s]) and np.array_equal(N2[s2 - n2:s2], N[s - n2:s])
    assert s2 == schedule.round_length(s, n1, n2, c, r)
    assert (s - s2) <= (s - n1 - n2) // 2 + 1
    # removed rows are exactly the selected A rows (even chunk offsets)
    removed = sorted(set(range(s)) - set(src.tolist()))
    for t in taps["chunks"]:
        if "selected" in t:
            rows_a = t["start"] + csm.partition(t["L"])[0]
            assert set(rows_a[t["selected"]].tolist()) <= set(removed)
            assert int(t["selected"].sum()) == t["m"] == csm.merge_count(r, t["L"])
    for x in removed:          # every removed row sits at an even offset of its chunk
        start = max(t["start"] for t in taps["chunks"] if t["start"] <= x)
        assert (x - start) % 2 == 0


def _check_match_and_rank(K, taps):
    """best_b is the lowest B attaining the row maximum; the selected set is the first m by
    (score descending, A index ascending)."""
    ties = 0
    for t in taps["chunks"]:
        if "best_b" not in t:
            continue
        A, B = csm.partition(t["L"])
        S = csm.cosine_matrix(K[t["start"] + A], K[t["start"] + B])
        for i, b in enumerate(t["best_b"]):
            assert S[i, b] == S[i].max()
            assert np.all(S[i, :b] < S[i, b])          # lowest index among maxima
            assert t["score"][i] == S[i, b]
            ties += int(np.sum(S[i] == S[i, b]) > 1)
        sel = t["selected"]
        if sel.any() and (~sel).any():
            lo_sel = t["score"][sel].min()
            hi_uns = t["score"][~sel].max()
            assert lo_sel >= hi_uns
            # at an exact tie the lower A index is the selected one
            for i in np.nonzero(~sel)[0]:
                if t["score"][i] == lo_sel:
                    ties += 1
                    assert np.nonzero(sel & (t["score"] == lo_sel))[0].max() < i
    return ties


def test_match_and_rank_properties():
    rng = np.random.default_rng(5)
    s, n1, n2, c = 2000, 16, 64, 256
    K, V, N = _random_slice(rng, s, 32, rho=0.97)
    K = bf16.round_to_bf16(K)
    _, _, _, _, taps = csm.csm_round_slice(K, V, N, s, n1, n2, c, 0.5)
    _check_match_and_rank(K, taps)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_planted_exact_ties_follow_the_rules(dt):
    """Copies of B rows make an A row tie two B rows exactly (the lower B must win); copies
    of A rows give equal best scores, some straddling the selection cut (the lower A must be
    selected).  Checked on fp32-valued data (inexact products) and bf16-valued data."""
    rng = np.random.default_rng(13)
    s, n1, n2, c = 3000, 16, 64, 128
    K, V, N = _random_slice(rng, s, 64, rho=0.9)
    K = K.astype(np.float32).astype(np.float64) if dt == "f32" else bf16.round_to_bf16(K)
    for start in range(n1, s - n2 - c, c):
        for _ in range(6):                     # B copies (odd offsets) inside the chunk
            j, j2 = sorted(rng.choice(c // 2, 2, replace=False))
            K[start + 2 * j2 + 1] = K[start + 2 * j + 1]
        for _ in range(6):                     # A copies (even offsets)
            i, i2 = sorted(rng.choice(c // 2, 2, replace=False))
            K[start + 2 * i2] = K[start + 2 * i]
    total = 0
    for r in (0.5, 0.3, 0.77):
        _, _, _, _, taps = csm.csm_round_slice(K, V, N, s, n1, n2, c, r)
        total += _check_match_and_rank(K, taps)
    assert total > 50


def test_centroids_are_means_of_their_members_over_rounds():
    rng = np.random.default_rng(11)
    s, n1, n2, c, d = 1200, 16, 64, 64, 6
    K, V, N = _random_slice(rng, s, d)
    orig_K, orig_V = K[:s].copy(), V[:s].copy()
    members = [[t] for t in range(s)]      # original tokens each current row stands for
    for j, r in enumerate([0.5, 0.45, 0.4, 0.35]):
        K2, V2, N2, s2, taps = csm.csm_round_slice(K, V, N, s, n1, n2, c, r, storage="f64")
        new_members = {}
        for t in taps["chunks"]:
            if "selected" not in t:
                continue
            A, B = csm.partition(t["L"])
            for i in np.nonzero(t["selected"])[0]:
                tb = t["start"] + B[t["best_b"][i]]
                new_members.setdefault(tb, list(members[tb]))
                new_members[tb] += members[t["start"] + A[i]]
        members = [new_members.get(int(p), members[int(p)]) for p in taps["src_pos"]]
        K, V, N, s = K2, V2, N2, s2
        for row in range(s):
            mem = members[row]
            assert N[row] == len(mem)
            np.testing.assert_allclose(K[row], orig_K[mem].mean(0), atol=1e-12)
            np.testing.assert_allclose(V[row], orig_V[mem].mean(0), atol=1e-12)


def test_outlier_slices_untouched_and_short_slices():
    rng = np.random.default_rng(3)
    S, cap, d = 4, 400, 8
    K = np.zeros((S, cap, d)); V = np.zeros((S, cap, d)); N = np.zeros((S, cap), np.int64)
    lens = np.array([400, 300, 81, 60])
    for z in range(S):
        k, v, n = _random_slice(rng, lens[z], d, cap=cap)
        K[z], V[z], N[z] = k, v, n
    mask = np.array([0, 1, 0, 0], np.uint8)
    K2, V2, N2, lens2, taps = csm.csm_compress(K, V, N, lens, 16, 64, 64, 0.5, mask, storage="f64")
    assert np.array_equal(K2[1], K[1]) and np.array_equal(N2[1], N[1]) and lens2[1] == 300
    assert lens2[2] == 81 and np.array_equal(K2[2], K[2])     # middle of length 1: untouched
    assert lens2[3] == 60 and np.array_equal(K2[3], K[3])     # middle negative: untouched
    assert lens2[0] < 400
