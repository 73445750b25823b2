"""Theorem 6.1 (Chelsea review, section 三, 理论分析) pins the oracle's chunk partition.

For every balanced partition of 2n <= 12 points and random convex non-increasing f,
the alternating partition produced by oracle.csm.partition must attain the maximum of
sum_{x in A} sum_{y in B} f(|x - y|).  A concave f is a counterexample, which shows the
check can fail.
"""
import numpy as np
import pytest

from oracle import csm, theorem


def _oracle_partition_1based(n):
    A, B = csm.partition(2 * n)
    return [int(a) + 1 for a in A], [int(b) + 1 for b in B]


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6])
def test_alternating_partition_is_a_maximiser(n):
    rng = np.random.default_rng(100 + n)
    trials = 40 if n < 6 else 12
    for t in range(trials):
        fam = ["exp", "uniform_trunc", "linear", "geometric"][t % 4]
        f = theorem.random_convex_decreasing(n, rng, fam)
        best, _ = theorem.brute_force_max(n, f)
        A, B = _oracle_partition_1based(n)
        assert theorem.objective(A, B, f) >= best - 1e-9 * max(1.0, abs(best)), (n, fam)


def test_oracle_partition_is_the_theorems_alternating_split():
    A, B = _oracle_partition_1based(4)
    assert A == [1, 3, 5, 7] and B == [2, 4, 6, 8]


def test_concave_f_breaks_it():
    f = np.array([0.0, 1.0, 0.99, 0.97, 0.9, 0.5, 0.1, 0.0])
    best, _ = theorem.brute_force_max(4, f)
    A, B = _oracle_partition_1based(4)
    assert theorem.objective(A, B, f) < best - 0.5


def test_block_partition_is_not_a_maximiser():
    # A plausible mistake (first half vs second half) loses for strictly convex f.
    rng = np.random.default_rng(7)
    f = theorem.random_convex_decreasing(4, rng, "exp")
    best, _ = theorem.brute_force_max(4, f)
    assert theorem.objective([1, 2, 3, 4], [5, 6, 7, 8], f) < best - 1e-9
