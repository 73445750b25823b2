"""The Algorithm 1 loop on the GPU: prefill rounds to the budget, then decode steps
(append, log-N attention, re-clustering on trigger), checked in lockstep with the oracle."""
import numpy as np
import pytest
import torch

import kvsynth
from oracle import attention as oatt
from tests import parity

pytestmark = pytest.mark.gpu


class Lockstep:
    """Compares every round on a few sampled slices with the oracle, on the GPU's own state."""

    def __init__(self, sample):
        self.sample = sample
        self.rep = parity.Report()
        self.rounds = 0

    def before_round(self, cache, r):
        self.state = {z: (cache.K[z].cpu(), cache.V[z].cpu(), cache.N[z].cpu(), int(cache.lens[z]))
                      for z in self.sample}

    def after_round(self, cache, r, best, sel, src):
        self.rounds += 1
        for z, (K, V, N, s) in self.state.items():
            parity.compare_slice(self.rep, parity.to_f64(K), parity.to_f64(V),
                                 N.numpy().astype(np.int64), s, cache.n1, cache.n2, cache.c, r, "bf16",
                                 best[z].cpu().numpy(), sel[z].cpu().numpy(), src[z].cpu().numpy(),
                                 parity.to_f64(cache.K[z].cpu()), parity.to_f64(cache.V[z].cpu()),
                                 cache.N[z].cpu().numpy().astype(np.int64), int(cache.lens[z]))


def test_algorithm1_loop_32k_batch4(lib, dev):
    from kv_cache_clustering_amd.pipeline import ClusteredKVCache
    w = kvsynth.workload(3)
    c = kvsynth.make_cache(w, dev)
    q_all = kvsynth.make_queries(w, dev)
    obs = Lockstep(sample=[0, 517, 1023])
    cache = ClusteredKVCache(c["K"], c["V"], c["N"], c["lens"], H_q=w.H_q, H_kv=w.H_kv, n=w.ctx,
                             R=w.R, Gamma=w.steps, g=w.g, observer=obs)
    rs = cache.prefill()
    assert len(rs) == 12 and cache.sched.s == 6573
    check_steps = {1, 200, 500, w.steps - 1}
    triggers = []
    worst = 0.0
    for i in range(1, w.steps):             # Algorithm 1 runs decode steps 1 .. Gamma-1
        O, r = cache.decode_step(q_all[i], c["app_k"][i - 1], c["app_v"][i - 1])
        if r is not None:
            triggers.append(i)
        if i in check_steps:
            Oh = O.cpu().double().numpy()
            for z in obs.sample:
                g, kvh = divmod(z, w.H_kv)
                s = int(cache.lens[z])
                Kz = parity.to_f64(cache.K[z, :s].cpu())
                Vz = parity.to_f64(cache.V[z, :s].cpu())
                Nz = cache.N[z, :s].cpu().numpy().astype(np.int64)
                for h in range(w.G):
                    hq = kvh * w.G + h
                    # the attention of step i ran before a trigger round of the same step
                    if r is not None:
                        continue
                    ref = oatt.logn_attention_one(parity.to_f64(q_all[i, g, hq].cpu()), Kz, Vz, Nz)
                    worst = max(worst, float(np.abs(Oh[g, hq] - ref).max()))
    cache.check_errors()
    print(obs.rep, "decode max abs", worst, "triggers", triggers)
    assert triggers == [213, 527, 841]
    assert obs.rounds == 15
    L = cache.lens.cpu().numpy()
    assert np.all(L == 6630)                  # the hand-derived final length
    live = torch.arange(cache.N.shape[1], device=dev)[None, :] < cache.lens[:, None]
    Nsum = torch.where(live, cache.N, 0).sum(dim=1, dtype=torch.int64).cpu().numpy()
    assert np.all(Nsum == w.ctx + w.steps - 1)
    parity.check_report(obs.rep)
    assert worst < 2e-4


def test_mha_32k_batch8_full_size(lib, dev):
    """Llama-2-7B-32K MHA shape at batch 8: 8192 slices, ~137 GB of bf16 K/V resident in HBM.
    Prefill rounds to the 25% budget in lockstep on sampled slices, then two decode steps."""
    from kv_cache_clustering_amd.pipeline import ClusteredKVCache
    w = kvsynth.workload(5, steps=3, cap_extra=3)
    c = kvsynth.make_cache(w, dev, batch_slices=256)
    assert c["K"].numel() * 2 * 2 > 130e9
    q_all = kvsynth.make_queries(w, dev)
    obs = Lockstep(sample=[0, 4097, w.slices - 1])
    cache = ClusteredKVCache(c["K"], c["V"], c["N"], c["lens"], H_q=w.H_q, H_kv=w.H_kv, n=w.ctx,
                             R=w.R, Gamma=128, g=w.g, observer=obs)
    rs = cache.prefill()
    assert len(rs) == 8 and cache.sched.s == 7947        # the hand-derived prefill trajectory
    worst = 0.0
    for i in range(1, 3):
        O, r = cache.decode_step(q_all[i], c["app_k"][i - 1], c["app_v"][i - 1])
        assert r is None
        Oh = O.cpu().double().numpy()
        for z in obs.sample:
            g, kvh = divmod(z, w.H_kv)
            s = int(cache.lens[z])
            ref = oatt.logn_attention_one(parity.to_f64(q_all[i, g, kvh].cpu()),
                                          parity.to_f64(cache.K[z, :s].cpu()),
                                          parity.to_f64(cache.V[z, :s].cpu()),
                                          cache.N[z, :s].cpu().numpy().astype(np.int64))
            worst = max(worst, float(np.abs(Oh[g, kvh] - ref).max()))
    cache.check_errors()
    print(obs.rep, "decode max abs", worst)
    assert np.all(cache.lens.cpu().numpy() == 7949)
    parity.check_report(obs.rep)
    assert worst < 2e-4
    del cache, c, q_all
    torch.cuda.empty_cache()
