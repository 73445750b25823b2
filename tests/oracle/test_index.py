"""Pins for oracle.index (hierarchical centroid index and the attention over what it keeps).

Source: LycheeCluster page, 方法论 §2 层次 KV 索引 and §3 流式懒更新; log-N attention from the
Chelsea review, section 三, 核心公式.  The page prints no worked example, so the index is pinned
by what the readings make true by mathematics: the ball bound holds for every row (brute force),
a zero-radius ball bounds exactly and a centred pair is tight, the tree walk keeps exactly the
leaves the direct test keeps, tau = inf is full attention, the dropped-mass error bound holds,
and lazy appends keep bounds valid with a kept set that contains a rebuild's.
"""
import numpy as np
import pytest

from oracle import attention as oatt
from oracle import index as oix


def _slice(rng, s, d=32, rho=0.9, degrees=True):
    K = np.zeros((s, d))
    k = rng.standard_normal(d)
    for t in range(s):
        k = rho * k + np.sqrt(1 - rho * rho) * rng.standard_normal(d)
        K[t] = k
    V = rng.standard_normal((s, d))
    N = rng.integers(1, 6, s) if degrees else np.ones(s, np.int64)
    return K, V, N


def _clustered(rng, s, B, d=64, spread=0.05):
    """Keys in tight clusters, one per block of B rows, cluster centres random directions of norm
    sqrt(d): the structure under which ball bounds can drop whole blocks."""
    nb = -(-s // B)
    C = rng.standard_normal((nb, d))
    C *= np.sqrt(d) / np.linalg.norm(C, axis=1, keepdims=True)
    K = np.repeat(C, B, axis=0)[:s] + spread * rng.standard_normal((s, d))
    V = rng.standard_normal((s, d))
    N = rng.integers(1, 6, s)
    return K, V, N


def _queries(rng, K, G=4, peaked=True):
    """Random queries, or queries aligned with a few keys (peaked attention)."""
    d = K.shape[1]
    if not peaked:
        return rng.standard_normal((G, d))
    js = rng.integers(0, K.shape[0], G)
    return 6.0 * K[js] / np.linalg.norm(K[js], axis=1, keepdims=True) * np.sqrt(d) ** 0.5


@pytest.mark.parametrize("s,B", [(1000, 64), (257, 16), (64, 64), (5, 4)])
def test_every_row_is_under_its_leaf_and_ancestor_bounds(s, B):
    rng = np.random.default_rng(s + B)
    K, V, N = _slice(rng, s)
    idx = oix.build(K, N, s, B)
    for q in np.vstack([_queries(rng, K), _queries(rng, K, peaked=False)]):
        z = oix.logits(q, K[:s], N[:s])
        for r in range(s):
            u = idx["P"] + r // B
            while u >= 1:
                assert z[r] <= oix.bound(idx, u, q) + 1e-9, (r, u)
                u //= 2


def test_closed_form_bounds():
    # a block of identical keys has radius 0: its bound is that key's exact logit
    k = np.array([0.3, -1.2, 0.5, 2.0])
    K = np.vstack([k] * 4)
    N = np.array([1, 2, 3, 4])
    idx = oix.build(K, N, 4, 4)
    q = np.array([1.0, 0.5, -0.25, 0.125])
    assert idx["rho"][1] == 0.0
    assert oix.bound(idx, 1, q) == pytest.approx(oix.logits(q, K, N).max(), abs=1e-12)
    # +e1 and -e1: centre 0, radius 1; for q = e1 the bound is attained
    K = np.array([[1.0, 0.0], [-1.0, 0.0]])
    idx = oix.build(K, np.ones(2, np.int64), 2, 2)
    assert np.allclose(idx["mu"][1], 0.0) and idx["rho"][1] == pytest.approx(1.0)
    q = np.array([3.0, 0.0])
    assert oix.bound(idx, 1, q) == pytest.approx(oix.logits(q, K, np.ones(2)).max(), abs=1e-12)


@pytest.mark.parametrize("tau", [0.5, 2.0, 4.0, 8.0, np.inf])
def test_tree_walk_keeps_exactly_the_leaves_the_direct_test_keeps(tau):
    rng = np.random.default_rng(int(10 * min(tau, 99)))
    for s, B in [(3000, 64), (1111, 32), (70, 16)]:
        K, V, N = _slice(rng, s, d=64) if s != 3000 else _clustered(rng, s, B)
        idx = oix.build(K, N, s, B, cap=s + 500)
        for peaked in (True, False):
            qs = _queries(rng, K, peaked=peaked)
            T = oix.thresholds(qs, K, N, s, 16, 64, tau, B)
            forced = oix.protected_blocks(s, 16, 64, B)
            a = oix.kept_direct(idx, qs, T, forced)
            b = oix.kept_tree(idx, qs, T, forced)
            assert np.array_equal(a, b)


def test_tau_inf_is_full_logn_attention():
    rng = np.random.default_rng(3)
    s = 2000
    K, V, N = _slice(rng, s)
    qs = _queries(rng, K)
    O, keep = oix.pruned_attention(qs, K, V, N, s, 16, 64, 64, np.inf)
    assert keep.all()
    for h, q in enumerate(qs):
        assert np.array_equal(O[h], oatt.logn_attention_one(q, K, V, N))


@pytest.mark.parametrize("tau", [1.0, 3.0, 6.0, 10.0])
def test_dropped_mass_error_bound(tau):
    """|O_kept - O_full| <= 2 e^-tau (rows dropped) max|v|, and peaked queries drop rows."""
    rng = np.random.default_rng(int(tau * 7))
    s, B = 4096, 64
    dropped_any = False
    for peaked, (K, V, N) in ((True, _clustered(rng, s, B)), (False, _slice(rng, s, d=64, rho=0.8))):
        qs = _queries(rng, K, peaked=peaked)
        O, keep = oix.pruned_attention(qs, K, V, N, s, 16, 64, B, tau)
        n_drop = s - len(oix.kept_rows(keep, s, B))
        dropped_any |= n_drop > 0
        for h, q in enumerate(qs):
            full = oatt.logn_attention_one(q, K, V, N)
            err = np.abs(O[h] - full).max()
            assert err <= 2 * np.exp(-tau) * n_drop * np.abs(V).max() + 1e-12, (peaked, h, err)
    assert dropped_any


def test_lazy_appends_keep_bounds_valid_and_contain_a_rebuild():
    rng = np.random.default_rng(11)
    s0, B, extra = 700, 32, 150
    K, V, N = _slice(rng, s0 + extra, d=32)
    idx = oix.build(K, N, s0, B, cap=s0 + extra)
    for s in range(s0 + 1, s0 + extra + 1):
        oix.append_lazy(idx, K[s - 1], int(N[s - 1]), s)
        if (s - s0) % 37 and s != s0 + extra:
            continue
        qs = _queries(rng, K[:s])
        for q in qs:
            z = oix.logits(q, K[:s], N[:s])
            for r in range(s):
                u = idx["P"] + r // B
                while u >= 1:
                    assert z[r] <= oix.bound(idx, u, q) + 1e-9
                    u //= 2
        fresh = oix.build(K, N, s, B, cap=s0 + extra)
        for tau in (1.0, 4.0):
            T = oix.thresholds(qs, K, N, s, 16, 64, tau, B)
            forced = oix.protected_blocks(s, 16, 64, B)
            lazy = oix.kept_tree(idx, qs, T, forced)
            reb = oix.kept_tree(fresh, qs, T, forced)
            assert np.all(lazy[reb]), "lazy bounds dropped a block a rebuild keeps"


def test_hand_worked_tree_and_lazy_appends(golden_dir):
    """A four-row tree with unequal degrees (degree-weighted centres), its bounds for one query,
    and two lazy appends (a new leaf, then a widened one), against values worked out by hand."""
    import json
    import os
    with open(os.path.join(golden_dir, "index_tiny_case.json")) as f:
        case = json.load(f)
    K = np.array(case["K"], np.float64)
    N = np.array(case["N"], np.int64)
    B, cap = case["B"], case["cap"]
    rows = np.zeros((cap, case["d"]))
    rows[:len(K)] = K
    degs = np.zeros(cap, np.int64)
    degs[:len(N)] = N
    idx = oix.build(rows, degs, case["s"], B, cap=cap)
    exp = case["build"]
    assert idx["P"] == exp["P"]

    def check(e):
        for u, v in e.get("wt", {}).items():
            assert idx["wt"][int(u)] == v, ("wt", u)
        for u, v in e.get("mu", {}).items():
            assert np.allclose(idx["mu"][int(u)], v, atol=1e-12), ("mu", u)
        for u, v in e.get("rho", {}).items():
            assert idx["rho"][int(u)] == pytest.approx(v, abs=1e-12), ("rho", u)
        for u, v in e.get("lmax", {}).items():
            assert idx["lmax"][int(u)] == pytest.approx(v, abs=1e-12), ("lmax", u)
    check(exp)
    q = np.array(exp["bound_q"], np.float64)
    for u, v in exp["bound"].items():
        assert oix.bound(idx, int(u), q) == pytest.approx(v, abs=1e-12)
    for ap in case["appends"]:
        rows[ap["s"] - 1] = ap["row"]
        degs[ap["s"] - 1] = ap["n"]
        oix.append_lazy(idx, np.array(ap["row"], np.float64), ap["n"], ap["s"])
        check(ap["expect"])
