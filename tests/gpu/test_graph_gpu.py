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


def test_device_trigger_loop_matches_host_driven(lib, dev):
    """Whole decode steps (append, attention, round on the device's own trigger) captured in
    one graph, replayed 8 times, against the host-driven eager loop and the eager
    device-trigger step: same outputs, same cache bit for bit, same rounds."""
    from kv_cache_clustering_amd.pipeline import ClusteredKVCache
    from tests.gpu.conftest import host_cache
    S, n, steps, per = 32, 6000, 400, 50
    Kh, Vh, Nh, Lh = host_cache(S, n + steps, [n] * S, seed=23, rho=0.96)
    mask = torch.zeros(S, dtype=torch.uint8)
    mask[5] = 1                                    # one outlier slice keeps growing
    kw = dict(H_q=16, H_kv=4, n=n, R=0.25, Gamma=steps, outlier_mask=mask.to(dev))
    caches = [ClusteredKVCache(Kh.to(dev), Vh.to(dev), Nh.to(dev), Lh.to(dev), **kw)
              for _ in range(3)]
    A, B, C = caches                               # host trigger / graph loop / device trigger
    pre = [x.prefill() for x in caches]
    assert pre[0] == pre[1] == pre[2] and len(pre[0]) >= 5
    B.capture_loop(per)
    gen = torch.Generator(device=dev).manual_seed(9)
    rounds_a, rounds_c = [], []
    for rep in range(steps // per):
        q = torch.randn((per, S // 4, 16, 128), generator=gen, device=dev).to(torch.bfloat16)
        k = torch.randn((per, S, 128), generator=gen, device=dev).to(torch.bfloat16)
        v = torch.randn((per, S, 128), generator=gen, device=dev).to(torch.bfloat16)
        Oa, Oc = [], []
        for i in range(per):
            O, r = A.decode_step(q[i], k[i], v[i])
            Oa.append(O.clone())
            if r is not None:
                rounds_a.append((A.step_index, r))
            O, r = C.decode_step_device(q[i], k[i], v[i])
            Oc.append(O.clone())
            if r is not None:
                rounds_c.append((C.step_index, r))
        Ob, rounds_b = B.run_loop(q, k, v)
        torch.cuda.synchronize()
        for i in range(per):
            assert torch.equal(Oa[i], Ob[i]), (rep, i)
            assert torch.equal(Oa[i], Oc[i]), (rep, i)
        assert [x for x in rounds_a if x[0] > rep * per] == rounds_b
        for X in (B, C):
            assert torch.equal(A.lens, X.lens), rep
            assert torch.equal(A.N, X.N) and torch.equal(A.K, X.K) and torch.equal(A.V, X.V)
            assert torch.equal(X.round_idx.cpu(), torch.where(mask.bool(), len(pre[0]),
                                                              A.sched.j).to(torch.int32))
    assert rounds_a == rounds_c and len(rounds_a) >= 3
    for X in caches:
        X.check_errors()
    s_host = A.sched.s
    assert int(A.lens[0]) == s_host and int(A.lens[5]) == n + steps


def test_device_trigger_bounds_and_skips(lib, dev):
    """Slices below their threshold are left as they are; a slice that would run above the
    launch bound is a device error and is left as it is; slices that do not run may exceed
    the bound."""
    from tests.gpu.conftest import host_cache
    S, cap = 4, 3000
    lens = [2000, 2500, 2999, 1000]
    K, V, N, L = (t.to(dev) for t in host_cache(S, cap, lens, seed=3))
    K0, V0, N0 = K.clone(), V.clone(), N.clone()
    thr = torch.tensor([2500, 2500, 2500, 900], dtype=torch.int32, device=dev)
    idx = torch.tensor([0, 3, 20, 1], dtype=torch.int32, device=dev)
    ws = lib.csm_compress_triggered(K, V, N, L, thr, idx, max_len=2600)
    assert lib.read_error(ws) == lib.EDEVICE       # slice 2 would run at 2999 > 2600
    assert L.cpu().tolist()[:3] == [2000, lib_round_len(2500, 0.5 - 3 * 0.05), 2999]
    assert L.cpu().tolist()[3] == lib_round_len(1000, 0.5 - 1 * 0.05)
    assert idx.cpu().tolist() == [0, 4, 20, 2]      # only slices that ran advance
    assert torch.equal(K[0], K0[0]) and torch.equal(N[0], N0[0])
    assert torch.equal(K[2], K0[2]) and torch.equal(V[2], V0[2]) and torch.equal(N[2], N0[2])
    # within the bound every running slice is processed and no error is raised
    idx2 = torch.tensor([0, 0, 0, 0], dtype=torch.int32, device=dev)
    thr2 = torch.tensor([1, 1, 1, 1 << 30], dtype=torch.int32, device=dev)
    ws = lib.csm_compress_triggered(K, V, N, L, thr2, idx2, max_len=3000)
    assert lib.read_error(ws) == lib.OK
    assert idx2.cpu().tolist() == [1, 1, 1, 0]


def lib_round_len(s, r):
    from kv_cache_clustering_amd.schedule import round_output_length
    return round_output_length(s, 16, 64, 256, max(r, 0.1))
