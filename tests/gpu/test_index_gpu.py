"""Hierarchical centroid index (csm_index_build / csm_index_append) and decode attention over the
rows it keeps (decode_attn_logn_pruned), against the oracle (oracle/index.py).

LycheeCluster page, 方法论 §2 层次 KV 索引 and §3 流式懒更新, over the cache CSM leaves.
The index is compared node by node with the oracle's (centres, radii, log-degrees, degree
totals), and every row is checked to lie under its leaf's and every ancestor's bound as the
device stored them.  The kept blocks are compared with the oracle's: they may differ only where
the oracle's bound margin is within 1e-3 (base-2 logit units) of the threshold; the output is then
compared with the oracle's attention over the device's kept rows, and with full log-N attention
within the dropped-mass bound.  tau = inf keeps every block.
"""
import numpy as np
import pytest
import torch

import kvsynth
from oracle import attention as oatt
from oracle import index as oix
from tests import parity

pytestmark = pytest.mark.gpu

NEAR = 1e-3


def _clustered(rng, S, cap, lens, B, d, spread):
    K = np.zeros((S, cap, d), np.float32)
    V = np.zeros((S, cap, d), np.float32)
    N = np.zeros((S, cap), np.int32)
    for z in range(S):
        s = int(lens[z])
        nb = -(-s // B)
        C = rng.standard_normal((nb, d))
        C *= np.sqrt(d) / np.linalg.norm(C, axis=1, keepdims=True)
        K[z, :s] = np.repeat(C, B, axis=0)[:s] + spread * rng.standard_normal((s, d))
        V[z, :s] = rng.standard_normal((s, d))
        N[z, :s] = rng.integers(1, 6, s)
    return K, V, N


def _peaked_q(rng, K, lens, groups, H_q, H_kv):
    d = K.shape[2]
    G = H_q // H_kv
    q = np.zeros((groups, H_q, d), np.float32)
    for g in range(groups):
        for kvh in range(H_kv):
            z = g * H_kv + kvh
            for h in range(G):
                j = int(rng.integers(0, max(1, int(lens[z]))))
                k = K[z, j]
                q[g, kvh * G + h] = 6.0 * k / max(np.linalg.norm(k), 1e-6) * d ** 0.25
    return q


def _setup(dev, dt, d, B, spread, seed, lens, cap, H_q=8, H_kv=2):
    rng = np.random.default_rng(seed)
    S = len(lens)
    Kf, Vf, Nf = _clustered(rng, S, cap, lens, B, d, spread)
    qf = _peaked_q(rng, Kf, lens, S // H_kv, H_q, H_kv)
    T = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dt]
    K, V, N = torch.from_numpy(Kf).to(T), torch.from_numpy(Vf).to(T), torch.from_numpy(Nf)
    q = torch.from_numpy(qf).to(T)
    L = torch.tensor(lens, dtype=torch.int32)
    return K.to(dev), V.to(dev), N.to(dev), L.to(dev), q.to(dev)


def _node_arrays(lib, index, S, P, d):
    """The device index as numpy arrays (centres, radii, log2 degree, degree totals)."""
    nodes = S * 2 * P
    b = index.cpu().numpy()

    def al(x):
        return (x + 255) // 256 * 256
    mu = b[:nodes * d * 4].view(np.float32).reshape(S, 2 * P, d)
    o = al(nodes * d * 4)
    rho = b[o:o + nodes * 4].view(np.float32).reshape(S, 2 * P)
    o += al(nodes * 4)
    lmax = b[o:o + nodes * 4].view(np.float32).reshape(S, 2 * P)
    o += al(nodes * 4)
    wt = b[o:o + nodes * 4].view(np.int32).reshape(S, 2 * P)
    return mu, rho, lmax, wt


def _check_index(K64, N64, lens, cap, B, mu, rho, lmax, wt, qs_by_slice):
    S = len(lens)
    P = mu.shape[1] // 2
    for z in range(S):
        s = int(lens[z])
        ref = oix.build(K64[z], N64[z], s, B, cap=cap)
        assert ref["P"] == P
        used = ref["wt"] > 0
        assert np.array_equal(wt[z][1:], ref["wt"][1:].astype(np.int32)), z
        np.testing.assert_allclose(mu[z][1:][used[1:]], ref["mu"][1:][used[1:]], rtol=1e-5, atol=1e-5)
        r_dev, r_ref = rho[z][1:][used[1:]], ref["rho"][1:][used[1:]]
        assert np.all(r_dev >= r_ref * (1 - 1e-6) - 1e-6) and np.all(r_dev <= r_ref * (1 + 1e-4) + 1e-5)
        np.testing.assert_allclose(lmax[z][1:][used[1:]], ref["lmax"][1:][used[1:]], atol=1e-5)
        # every row under its leaf's and every ancestor's bound, with the device's node values
        dev = {"mu": mu[z].astype(np.float64), "rho": rho[z].astype(np.float64),
               "lmax": lmax[z].astype(np.float64), "P": P}
        for q in qs_by_slice[z]:
            zr = oix.logits(q, K64[z, :s], N64[z, :s])
            for r in range(s):
                u = P + r // B
                while u >= 1:
                    assert zr[r] <= oix.bound(dev, u, q) + 1e-6, (z, r, u)
                    u //= 2


# leaves read in one pass of at most 64 rows (their rows kept in registers for the radius) and in
# several (read again): fp32 at d = 128 takes 32 rows a pass, so its 64-row leaves need two
@pytest.mark.parametrize("dt,d,B", [("bf16", 128, 64), ("f16", 64, 32), ("f32", 128, 16),
                                    ("bf16", 64, 256), ("f32", 128, 64), ("f16", 128, 128)])
def test_index_build_matches_oracle_and_bounds_hold(lib, dev, dt, d, B):
    lens = [3000, 1, 0, 777]
    cap = 3100
    K, V, N, L, q = _setup(dev, dt, d, B, 0.3, seed=B + d, lens=lens, cap=cap)
    index = lib.new_index(K, B)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    lib.index_build(K, N, L, index, err, B)
    assert lib.read_error(err) == lib.OK
    P = lib.index_leaf_slots(cap, B)
    mu, rho, lmax, wt = _node_arrays(lib, index, len(lens), P, d)
    K64, N64 = parity.to_f64(K.cpu()), N.cpu().numpy().astype(np.int64)
    qh = parity.to_f64(q.cpu())
    qs = [qh[z // 2, (z % 2) * 4:(z % 2) * 4 + 4] for z in range(len(lens))]
    _check_index(K64, N64, lens, cap, B, mu, rho, lmax, wt, qs)


@pytest.mark.parametrize("cap,B,lens,max_len", [
    (16, 16, [16, 3, 0, 9], 16),          # one leaf slot: the leaf is the root
    (32, 16, [32, 17, 1, 0], 32),         # two leaf slots
    (100, 16, [100, 64, 33, 5], 100),     # eight leaf slots: one leaf group, its whole subtree
    (300, 16, [300, 129, 200, 7], 200),   # 32 leaf slots, the length bound below the capacity
])
def test_index_build_small_trees_and_length_bound(lib, dev, cap, B, lens, max_len):
    """Trees smaller than a leaf group, exactly one group, and several groups under a length bound
    below the capacity (the build covers max_len rows; the slots past them are emptied), over an
    index filled with arbitrary bytes first, so every node must be written.  A slice longer than
    the bound sets the error word and gets an empty tree; the others match the oracle's node by
    node."""
    d = 128
    K, V, N, L, q = _setup(dev, "bf16", d, B, 0.3, seed=cap + B, lens=lens, cap=cap)
    index = lib.new_index(K, B)
    index.fill_(0x5A)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    lib.index_build(K, N, L, index, err, B, max_len=max_len)
    bad = [z for z, s in enumerate(lens) if s > max_len]
    assert (lib.read_error(err) == lib.OK) == (not bad)
    P = lib.index_leaf_slots(cap, B)
    mu, rho, lmax, wt = _node_arrays(lib, index, len(lens), P, d)
    for z in bad:
        assert np.all(wt[z][1:] == 0), z
    good = [z for z in range(len(lens)) if z not in bad]
    K64, N64 = parity.to_f64(K.cpu()), N.cpu().numpy().astype(np.int64)
    qh = parity.to_f64(q.cpu())
    qs = [qh[z // 2, (z % 2) * 4:(z % 2) * 4 + 4] for z in range(len(lens))]
    _check_index(K64[good], N64[good], [lens[z] for z in good], cap, B, mu[good], rho[good],
                 lmax[good], wt[good], [qs[z] for z in good])


def _compare_pruned(lib, K, V, N, L, q, index, tau, B, n1, n2, H_q, H_kv):
    """Pruned decode on the device against the oracle; returns (dropped rows, worst error vs the
    oracle over the device's kept rows, worst error vs full attention, bound)."""
    O, kept, ws = lib.decode_attn_logn_pruned(q, K, V, N, L, H_q, H_kv, index, tau, n1, n2, B,
                                              kept=True)
    assert lib.read_error(ws) == lib.OK
    S, cap, d = K.shape
    G = H_q // H_kv
    K64, V64 = parity.to_f64(K.cpu()), parity.to_f64(V.cpu())
    N64 = N.cpu().numpy().astype(np.int64)
    qh = parity.to_f64(q.cpu())
    Oh = O.cpu().double().numpy()
    kt = kept.cpu().numpy().astype(bool)
    near = differ = dropped = 0
    worst_follow = worst_full = 0.0
    bound_ok = True
    for z in range(S):
        s = int(L[z])
        g, kvh = divmod(z, H_kv)
        qs = qh[g, kvh * G:(kvh + 1) * G]
        if s == 0:
            assert np.all(Oh[g, kvh * G:(kvh + 1) * G] == 0)
            continue
        idx = oix.build(K64[z], N64[z], s, B, cap=cap)
        T = oix.thresholds(qs, K64[z], N64[z], s, n1, n2, tau, B)
        forced = oix.protected_blocks(s, n1, n2, B)
        ref_keep = oix.kept_tree(idx, qs, T, forced)
        dev_keep = kt[z, :idx["nleaf"]]
        assert not kt[z, idx["nleaf"]:].any()
        for b in np.nonzero(dev_keep != ref_keep)[0]:
            differ += 1
            margin = max(oix.bound(idx, idx["P"] + b, qq) - t for qq, t in zip(qs, T))
            if abs(margin) < NEAR and b not in forced:
                near += 1
            else:
                raise AssertionError(("kept block differs", z, b, margin))
        rows = oix.kept_rows(dev_keep, s, B)
        dropped += s - len(rows)
        for h in range(G):
            follow = oatt.logn_attention_one(qs[h], K64[z, rows], V64[z, rows], N64[z, rows])
            full = oatt.logn_attention_one(qs[h], K64[z, :s], V64[z, :s], N64[z, :s])
            got = Oh[g, kvh * G + h]
            worst_follow = max(worst_follow, float(np.abs(got - follow).max()))
            err_full = float(np.abs(got - full).max())
            worst_full = max(worst_full, err_full)
            lim = 2 * np.exp(-tau) * (s - len(rows)) * np.abs(V64[z, :s]).max() + 2e-4
            bound_ok &= err_full <= lim
    return dropped, near, differ, worst_follow, worst_full, bound_ok


@pytest.mark.parametrize("dt,d,B,G", [("bf16", 128, 64, 4), ("f16", 128, 32, 8), ("f32", 64, 64, 1),
                                      ("bf16", 64, 128, 2)])
def test_pruned_decode_against_oracle(lib, dev, dt, d, B, G):
    H_kv = 2
    H_q = G * H_kv
    lens = [4000, 2500, 0, 3333, 100, 4096]
    K, V, N, L, q = _setup(dev, dt, d, B, 0.05, seed=G * 7 + d, lens=lens, cap=4100, H_q=H_q,
                           H_kv=H_kv)
    index = lib.new_index(K, B)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    lib.index_build(K, N, L, index, err, B)
    assert lib.read_error(err) == lib.OK
    total_dropped = 0
    for tau in (2.0, 6.0, float("inf")):
        dropped, near, differ, wf, wfull, ok = _compare_pruned(lib, K, V, N, L, q, index, tau, B,
                                                               16, 64, H_q, H_kv)
        print(dt, d, B, G, "tau", tau, "dropped rows", dropped, "near-threshold differences", near,
              "vs oracle (device's rows)", wf, "vs full", wfull)
        assert wf < 2e-4 and ok
        if tau == float("inf"):
            assert dropped == 0 and wfull < 2e-4
        total_dropped += dropped
    assert total_dropped > 0          # the clustered keys and aligned queries do get pruned


def test_lazy_appends_track_the_oracle_and_keep_a_superset(lib, dev):
    """Rows appended with kv_append and taken in with csm_index_append: the device index equals
    the oracle's lazy updates, every bound still holds, and the blocks kept contain those a fresh
    build keeps."""
    B, d, H_q, H_kv = 32, 128, 8, 2
    lens = [1000, 1020, 700, 31]
    cap = 1300
    K, V, N, L, q = _setup(dev, "bf16", d, B, 0.2, seed=5, lens=lens, cap=cap)
    S = len(lens)
    index = lib.new_index(K, B)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    lib.index_build(K, N, L, index, err, B)
    K64, N64 = parity.to_f64(K.cpu()), N.cpu().numpy().astype(np.int64)
    refs = [oix.build(K64[z], N64[z], lens[z], B, cap=cap) for z in range(S)]
    gen = torch.Generator(device=dev).manual_seed(3)
    for step in range(150):
        kn = (torch.randn((S, d), generator=gen, device=dev) * 1.5).to(torch.bfloat16)
        vn = torch.randn((S, d), generator=gen, device=dev).to(torch.bfloat16)
        lib.kv_append(K, V, N, L, kn, vn, err)
        lib.index_append(K, N, L, index, err, B)
        knh = parity.to_f64(kn.cpu())
        for z in range(S):
            oix.append_lazy(refs[z], knh[z], 1, lens[z] + step + 1)
    assert lib.read_error(err) == lib.OK
    lens_now = L.cpu().tolist()
    assert lens_now == [x + 150 for x in lens]
    P = lib.index_leaf_slots(cap, B)
    mu, rho, lmax, wt = _node_arrays(lib, index, S, P, d)
    K64, N64 = parity.to_f64(K.cpu()), N.cpu().numpy().astype(np.int64)
    qh = parity.to_f64(q.cpu())
    for z in range(S):
        ref = refs[z]
        used = ref["wt"] > 0
        assert np.array_equal(wt[z][1:], ref["wt"][1:].astype(np.int32))
        np.testing.assert_allclose(mu[z][1:][used[1:]], ref["mu"][1:][used[1:]], rtol=1e-5, atol=1e-5)
        np.testing.assert_allclose(rho[z][1:][used[1:]], ref["rho"][1:][used[1:]], rtol=2e-4, atol=1e-5)
        dev_idx = {"mu": mu[z].astype(np.float64), "rho": rho[z].astype(np.float64),
                   "lmax": lmax[z].astype(np.float64), "P": P}
        s = lens_now[z]
        for qq in qh[z // 2, (z % 2) * 4:(z % 2) * 4 + 4]:
            zr = oix.logits(qq, K64[z, :s], N64[z, :s])
            for r in range(s):
                u = P + r // B
                while u >= 1:
                    assert zr[r] <= oix.bound(dev_idx, u, qq) + 1e-6
                    u //= 2
    fresh = lib.new_index(K, B)
    lib.index_build(K, N, L, fresh, err, B)
    for tau in (1.0, 4.0):
        _, k_lazy, _ = lib.decode_attn_logn_pruned(q, K, V, N, L, H_q, H_kv, index, tau, 16, 64, B,
                                                   kept=True)
        _, k_fresh, _ = lib.decode_attn_logn_pruned(q, K, V, N, L, H_q, H_kv, fresh, tau, 16, 64, B,
                                                    kept=True)
        assert torch.all(k_lazy >= k_fresh), tau


def test_pruned_decode_bad_length_and_ar1_keys(lib, dev):
    """A length above the bound sets the error word and gives zeros; on AR(1) keys with random
    queries (the benchmark's data) the ball bounds drop nothing, and the result is full log-N
    attention."""
    from tests.gpu.conftest import host_cache
    B, H_q, H_kv = 64, 8, 2
    lens = [3000, 2900, 2000, 1500]
    K, V, N, L = (t.to(dev) for t in host_cache(4, 3000, lens, seed=17, degrees=True))
    q = torch.randn((2, H_q, 128), generator=torch.Generator(device=dev).manual_seed(1),
                    device=dev).to(torch.bfloat16)
    index = lib.new_index(K, B)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    lib.index_build(K, N, L, index, err, B)
    assert lib.read_error(err) == lib.OK
    O, kept, ws = lib.decode_attn_logn_pruned(q, K, V, N, L, H_q, H_kv, index, 8.0, kept=True)
    assert lib.read_error(ws) == lib.OK
    ref = lib.decode_attn_logn(q, K, V, N, L, H_q, H_kv)
    nleaf = [-(-s // B) for s in lens]
    assert all(int(kept[z, :nleaf[z]].sum()) == nleaf[z] for z in range(4))
    assert float((O - ref).abs().max()) < 1e-5
    L2 = L.clone()
    L2[1] = 3001
    O2, _, ws2 = lib.decode_attn_logn_pruned(q, K, V, N, L2, H_q, H_kv, index, 8.0, max_len=3000)
    assert lib.read_error(ws2) == lib.EDEVICE
    assert torch.all(O2[0, 4:] == 0)


def test_pruned_decode_deep_trees_walk_level_by_level(lib, dev):
    """Trees of more than 4096 nodes are walked level by level, evaluating only the nodes whose
    parent passed (smaller ones evaluate every node at once and walk the bits): 16-row blocks
    over 40000-row slices (4096 leaf slots), kept blocks and outputs against the oracle."""
    B, H_kv, G = 16, 2, 4
    lens = [40000, 2500, 0, 33333]
    K, V, N, L, q = _setup(dev, "bf16", 128, B, 0.05, seed=77, lens=lens, cap=40000,
                           H_q=G * H_kv, H_kv=H_kv)
    index = lib.new_index(K, B)
    assert lib.index_leaf_slots(40000, B) == 4096
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    lib.index_build(K, N, L, index, err, B)
    assert lib.read_error(err) == lib.OK
    total_dropped = 0
    for tau in (2.0, float("inf")):
        dropped, near, differ, wf, wfull, ok = _compare_pruned(lib, K, V, N, L, q, index, tau, B,
                                                               16, 64, G * H_kv, H_kv)
        print("deep tree, tau", tau, "dropped rows", dropped, "near-threshold differences", near,
              "vs oracle (device's rows)", wf, "vs full", wfull)
        assert wf < 2e-4 and ok
        if tau == float("inf"):
            assert dropped == 0 and wfull < 2e-4
        total_dropped += dropped
    assert total_dropped > 0


def test_index_and_pruned_decode_full_size_sampled(lib, dev):
    """The launch configuration the benchmark times: the 64K workload's serving geometry (246
    slices of 13,081 rows and 10 outlier slices of 65,536, capacity for the decode appends,
    64-row blocks, 2048 leaf slots), its queries, tau = 8.  Sampled slices (two compressed, one
    outlier): the built tree node by node against the oracle's build, the kept blocks against
    the oracle's walk over the same bounds, and the output against the oracle's attention over
    the kept rows; every slice's output against the plain call."""
    w = kvsynth.workload(4)
    c = kvsynth.make_cache(w, dev, with_appends=False)
    K, V, N, mask = c["K"], c["V"], c["N"], c["mask"]
    maskh = mask.cpu().numpy()
    L = torch.tensor(np.where(maskh != 0, w.ctx, 13081).astype(np.int32), device=dev)
    q = kvsynth.make_queries(w, dev, steps=1)[0]
    B, tau = 64, 8.0
    S, cap, d = K.shape
    P = lib.index_leaf_slots(cap, B)
    index = lib.new_index(K, B)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    lib.index_build(K, N, L, index, err, B)
    assert lib.read_error(err) == lib.OK
    O, kept, ws = lib.decode_attn_logn_pruned(q, K, V, N, L, w.H_q, w.H_kv, index, tau, w.n1, w.n2,
                                              B, kept=True)
    assert lib.read_error(ws) == lib.OK
    plain = lib.decode_attn_logn(q, K, V, N, L, w.H_q, w.H_kv)
    print("full size: max |pruned - plain|", float((O - plain).abs().max()))
    assert float((O - plain).abs().max()) < 1e-5
    G = w.H_q // w.H_kv
    nodes = 2 * P
    out = [int(np.argmin(maskh)), 137, int(np.argmax(maskh))]
    ib = index.view(torch.uint8)
    al = lambda x: (x + 255) // 256 * 256
    o_rho = al(S * nodes * d * 4)
    o_lmax = o_rho + al(S * nodes * 4)
    o_wt = o_lmax + al(S * nodes * 4)
    for z in out:
        s = int(L[z])
        mu = ib[z * nodes * d * 4:(z + 1) * nodes * d * 4].cpu().numpy().view(np.float32).reshape(nodes, d)
        rho = ib[o_rho + z * nodes * 4:o_rho + (z + 1) * nodes * 4].cpu().numpy().view(np.float32)
        lmax = ib[o_lmax + z * nodes * 4:o_lmax + (z + 1) * nodes * 4].cpu().numpy().view(np.float32)
        wt = ib[o_wt + z * nodes * 4:o_wt + (z + 1) * nodes * 4].cpu().numpy().view(np.int32)
        K64 = parity.to_f64(K[z, :s].cpu())
        V64 = parity.to_f64(V[z, :s].cpu())
        N64 = N[z, :s].cpu().numpy().astype(np.int64)
        ref = oix.build(K64, N64, s, B, cap=cap)
        assert ref["P"] == P
        used = ref["wt"] > 0
        assert np.array_equal(wt[1:], ref["wt"][1:].astype(np.int32)), z
        np.testing.assert_allclose(mu[1:][used[1:]], ref["mu"][1:][used[1:]], rtol=1e-5, atol=1e-5)
        r_dev, r_ref = rho[1:][used[1:]], ref["rho"][1:][used[1:]]
        assert np.all(r_dev >= r_ref * (1 - 1e-6) - 1e-6) and np.all(r_dev <= r_ref * (1 + 1e-4) + 1e-5)
        np.testing.assert_allclose(lmax[1:][used[1:]], ref["lmax"][1:][used[1:]], atol=1e-5)
        g, kvh = divmod(z, w.H_kv)
        qs = parity.to_f64(q[g, kvh * G:(kvh + 1) * G].cpu())
        T = oix.thresholds(qs, K64, N64, s, w.n1, w.n2, tau, B)
        ref_keep = oix.kept_tree(ref, qs, T, oix.protected_blocks(s, w.n1, w.n2, B))
        dev_keep = kept[z, :ref["nleaf"]].cpu().numpy().astype(bool)
        assert not kept[z, ref["nleaf"]:].cpu().numpy().any()
        for b in np.nonzero(dev_keep != ref_keep)[0]:
            margin = max(oix.bound(ref, P + b, qq) - t for qq, t in zip(qs, T))
            assert abs(margin) < NEAR, ("kept block differs", z, b, margin)
        rows = oix.kept_rows(dev_keep, s, B)
        for h in range(G):
            want = oatt.logn_attention_one(qs[h], K64[rows], V64[rows], N64[rows])
            assert float(np.abs(O[g, kvh * G + h].cpu().double().numpy() - want).max()) < 2e-4
        print("slice", z, "rows", s, "kept blocks", int(dev_keep.sum()), "of", ref["nleaf"])


def test_seeded_sweep_pruned_decode(lib, dev):
    """36 seeded random geometries: storage format, head dim, block rows 16..256, heads per group
    (1..8), KV heads, ragged lengths (empty, one row, full, random), protected-row counts (none
    included), key spreads and thresholds from 0.5 to +inf.  Every build and pruned call against
    the oracle as in the tests above."""
    rng = np.random.default_rng(2024)
    dts = ["bf16", "f16", "f32"]
    total_dropped = total_near = 0
    worst = 0.0
    for case in range(36):
        dt = dts[case % 3]
        d = 64 if (case // 3) % 2 else 128
        B = int(rng.choice([16, 32, 64, 128, 256]))
        G = int(rng.choice([1, 2, 4, 8]))
        H_kv = int(rng.choice([1, 2, 4]))
        groups = int(rng.choice([1, 2]))
        S = groups * H_kv
        cap = int(rng.integers(1, 3000))
        lens = [int(rng.choice([0, 1, cap, int(rng.integers(0, cap + 1))])) for _ in range(S)]
        n1, n2 = int(rng.choice([0, 1, 16])), int(rng.choice([0, 7, 64]))
        spread = float(rng.choice([0.05, 0.3, 1.0]))
        tau = float(rng.choice([0.5, 2.0, 6.0, np.inf]))
        K, V, N, L, q = _setup(dev, dt, d, B, spread, seed=3000 + case, lens=lens, cap=cap,
                               H_q=G * H_kv, H_kv=H_kv)
        index = lib.new_index(K, B)
        err = torch.zeros(1, dtype=torch.int32, device=dev)
        lib.index_build(K, N, L, index, err, B)
        assert lib.read_error(err) == lib.OK, case
        dropped, near, differ, wf, wfull, ok = _compare_pruned(lib, K, V, N, L, q, index, tau, B,
                                                               n1, n2, G * H_kv, H_kv)
        assert wf < 2e-4 and ok, (case, dt, d, B, G, H_kv, lens, n1, n2, tau, wf)
        if tau == float("inf"):
            assert dropped == 0 and wfull < 2e-4, case
        total_dropped += dropped
        total_near += near
        worst = max(worst, wf)
    print("dropped rows", total_dropped, "near-threshold differences", total_near,
          "worst vs oracle (device's rows)", worst)
    assert total_dropped > 0
