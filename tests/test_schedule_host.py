"""Host-side facts the round kernels rely on (CPU only).

The register-resident round kernels, picked for r <= 1/2, move each chunk's merge sources into
the B rows that are not merge targets.  That needs, for every chunk length L and every r <= 1/2,
sources + targets <= floor(L/2); targets never outnumber sources, so 2 m <= floor(L/2) suffices,
with m the chunk's merge count (Chelsea review, 分块软匹配算法 step 3: the top floor(r L / 2)
matches merge).  The device computes m as chunk_merges does, in fp64 with the same 1e-9 guard.
"""
import numpy as np

from kv_cache_clustering_amd.schedule import annealed_r, chunk_merges


def test_merges_leave_enough_free_b_rows_for_r_up_to_half():
    rs = [0.0, 0.05, 0.1, 0.25, 0.49, 0.4999999999, np.nextafter(0.5, 0.0), 0.5]
    rs += list(np.random.default_rng(3).random(200) * 0.5)
    for L in range(2, 513):
        nB = L // 2
        for r in rs:
            m = chunk_merges(float(r), L)
            assert 2 * m <= nB, (L, r, m)
    # the bound is tight: at r = 1/2 a chunk of 4k rows merges exactly k rows into 2k B rows
    assert all(2 * chunk_merges(0.5, 4 * k) == 2 * k for k in range(1, 129))


def test_annealed_r_never_exceeds_its_start():
    """The host picks the kernel from the call's r (r_init for the device-side trigger); every
    annealed r = max(r_init - j delta, r_min) stays at or below it."""
    for r_init in (0.5, 0.3, 0.1):
        for delta in (0.0, 0.05, 0.1):
            for r_min in (0.0, 0.05, 0.1):
                if r_min > r_init:
                    continue
                assert all(annealed_r(j, r_init, delta, r_min) <= r_init for j in range(200))
