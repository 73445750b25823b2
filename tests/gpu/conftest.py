import numpy as np
import pytest
import torch


@pytest.fixture(scope="session")
def lib():
    # Fails loudly if the HIP library is missing: there is no fallback path.
    from kv_cache_clustering_amd import _lib
    return _lib


@pytest.fixture(scope="session")
def dev():
    return torch.device("cuda:0")


def host_cache(S, cap, lens, d=128, dtype=torch.bfloat16, rho=0.95, seed=0, degrees=False,
               mean_std=0.0):
    """Small seeded cache built on the host (AR(1) keys, N(0,1) values) -> CPU tensors."""
    from kvsynth import ar1_numpy
    rng = np.random.default_rng(seed)
    K = np.zeros((S, cap, d), np.float32)
    V = np.zeros((S, cap, d), np.float32)
    N = np.zeros((S, cap), np.int32)
    for z in range(S):
        s = int(lens[z])
        if s:
            mu = rng.normal(0, mean_std, d) if mean_std > 0 else None
            K[z, :s] = ar1_numpy(rng, s, d, rho, np.sqrt(1 - rho * rho), mu)
            V[z, :s] = rng.standard_normal((s, d))
            N[z, :s] = rng.integers(1, 6, s) if degrees else 1
    return (torch.from_numpy(K).to(dtype), torch.from_numpy(V).to(dtype), torch.from_numpy(N),
            torch.tensor(np.asarray(lens, np.int32)))
