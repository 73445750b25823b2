"""The decode step captured in a HIP graph equals the eager step, replay after replay."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def _twin_caches(dev):
    from tests.gpu.conftest import host_cache
    S, n, steps = 32, 6000, 80
    K, V, N, L = host_cache(S, n + steps, [n] * S, seed=21, rho=0.96)
    return (K.to(dev), V.to(dev), N.to(dev), L.to(dev)), (K.to(dev), V.to(dev), N.to(dev), L.to(dev)), n, steps


def test_graph_replays_match_eager_steps(lib, dev):
    from kv_cache_clustering_amd.pipeline import ClusteredKVCache
    (a, b, n, steps) = _twin_caches(dev)
    kw = dict(H_q=16, H_kv=4, n=n, R=0.25, Gamma=steps)
    A = ClusteredKVCache(*a, **kw)
    B = ClusteredKVCache(*b, **kw)
    assert A.prefill() == B.prefill()
    B.capture_decode()
    gen = torch.Generator(device=dev).manual_seed(5)
    S = a[0].shape[0]
    rounds = 0
    for i in range(1, steps):
        q = torch.randn((S // 4, 16, 128), generator=gen, device=dev).to(torch.bfloat16)
        k = torch.randn((S, 128), generator=gen, device=dev).to(torch.bfloat16)
        v = torch.randn((S, 128), generator=gen, device=dev).to(torch.bfloat16)
        Oa, ra = A.decode_step(q, k, v)
        Ob, rb = B.decode_step_graph(q, k, v)
        assert ra == rb
        rounds += ra is not None
        torch.cuda.synchronize()
        assert torch.equal(Oa, Ob), i            # every replay against the eager result
        if i % 7 == 0:                             # eager work between replays
            torch.cuda.synchronize()
            assert torch.equal(A.lens, B.lens)
    A.check_errors()
    B.check_errors()
    assert rounds >= 1
    for x, y in zip(a, b):
        assert torch.equal(x, y)
