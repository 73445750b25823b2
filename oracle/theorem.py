"""Theorem 6.1 objective and brute-force search (test infrastructure only).

Chelsea review, section 三, 理论分析, 定理 6.1: over all partitions of [2n] into two sets
A, B of size n, if f on {1, ..., 2n-1} has non-increasing, non-negative successive drops
f(k) - f(k+1) (convex and non-increasing), then the alternating partition
A0 = {1, 3, ..., 2n-1}, B0 = {2, 4, ..., 2n} maximises sum_{x in A} sum_{y in B} f(|x - y|).

This module only evaluates the objective and enumerates all balanced partitions; the
test checks that the oracle's chunk partition (csm.partition) attains the maximum.
"""

import itertools

import numpy as np


def objective(A, B, f):
    """sum over x in A, y in B of f(|x - y|); positions are 1-based, f is indexed by distance."""
    return float(sum(f[abs(x - y)] for x in A for y in B))


def brute_force_max(n, f):
    """Maximum of the objective over every balanced partition of {1..2n}, and the maximisers."""
    pts = list(range(1, 2 * n + 1))
    best = -np.inf
    arg = []
    for A in itertools.combinations(pts, n):
        Aset = set(A)
        B = [p for p in pts if p not in Aset]
        v = objective(A, B, f)
        if v > best + 1e-12:
            best, arg = v, [A]
        elif abs(v - best) <= 1e-12:
            arg.append(A)
    return best, arg


def random_convex_decreasing(n, rng, family):
    """f(1..2n-1) with drops d_1 >= d_2 >= ... >= 0 (index 0 unused)."""
    k = 2 * n - 2
    if family == "exp":
        drops = np.sort(rng.exponential(1.0, size=k))[::-1]
    elif family == "uniform_trunc":
        drops = np.sort(np.maximum(rng.uniform(-0.5, 1.0, size=k), 0.0))[::-1]
    elif family == "linear":
        drops = np.full(k, rng.uniform(0.0, 1.0))
    elif family == "geometric":
        drops = rng.uniform(0.1, 1.0) * rng.uniform(0.3, 0.95) ** np.arange(k)
    else:
        raise ValueError(family)
    f = np.zeros(2 * n)
    f[1] = rng.uniform(0.0, 5.0) + drops.sum()
    for t in range(2, 2 * n):
        f[t] = f[t - 1] - drops[t - 2]
    return f
