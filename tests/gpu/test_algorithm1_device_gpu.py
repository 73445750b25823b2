"""Algorithm 1 with the trigger and the annealed r decided on the device, end to end on the 64K
workload, against the oracle.

Chelsea review, section 三, Algorithm 1: after prefill the cache is clustered while s >= B + g
(B = R (n + Gamma)); each decode step i = 1 .. Gamma - 1 appends a token, attends, and
clusters when s >= B + g.  CentroidKV page, 渐进式调度: r = r_init - j * delta_r over rounds j.

The trigger steps, the lengths after every round and the round counters are checked against
oracle.schedule.run_algorithm1 (the oracle's own loop, not the library's host bookkeeping).
Every round the device runs on a sampled slice is checked in lockstep: the same slices' input
state is run through csm_compress_debug at the oracle's r, whose output must equal the
triggered round's bit for bit (so the device took that r), and whose decisions and output are
compared with the oracle round (tests/parity.py).  Decode outputs are compared with the
oracle's log-N attention at several steps, including the step whose round fires.  The same
run captured as whole-step HIP graphs (capture_loop / run_loop) must reproduce every output and
the final cache bit for bit.
"""
import numpy as np
import pytest
import torch

import kvsynth
from oracle import attention as oatt
from oracle import schedule as oschedule
from tests import parity

pytestmark = pytest.mark.gpu


class DeviceLockstep:
    """Observer of csm_compress_triggered calls on a few sampled slices."""

    def __init__(self, lib, sample, maskh, osched, w):
        self.lib, self.sample, self.maskh, self.osched, self.w = lib, sample, maskh, osched, w
        self.rep = parity.Report()
        self.prefill_calls = 0
        self.fired = []          # (step, slice) of every device round seen on a sampled slice
        self.trigger = {i: (s, s2, r) for (i, s, s2, r) in osched["triggers"]}

    def expected(self, cache):
        """(runs, s_in, s_out, r) the oracle expects of this call for a compressed slice."""
        if cache.step_index == 0:
            k = self.prefill_calls
            pre = self.osched["prefill"]
            if k + 1 < len(pre):
                return True, pre[k], pre[k + 1], oschedule.annealed_r(k)
            return False, pre[-1], pre[-1], None
        if cache.step_index in self.trigger:
            s, s2, r = self.trigger[cache.step_index]
            return True, s, s2, r
        return False, None, None, None

    def before_device_round(self, cache):
        torch.cuda.synchronize()
        zs = self.sample
        self.pre = (cache.K[zs].clone(), cache.V[zs].clone(), cache.N[zs].clone(),
                    cache.lens[zs].clone(), cache.round_idx[zs].clone())

    def after_device_round(self, cache):
        lib, w = self.lib, self.w
        runs, s_in, s_out, r = self.expected(cache)
        if cache.step_index == 0:
            self.prefill_calls += 1
        Kp, Vp, Np, Lp, Ip = self.pre
        zs = self.sample
        L_now, I_now = cache.lens[zs].cpu().numpy(), cache.round_idx[zs].cpu().numpy()
        Lp, Ip = Lp.cpu().numpy(), Ip.cpu().numpy()
        comp = [i for i, z in enumerate(zs) if not self.maskh[z]]
        for i, z in enumerate(zs):
            if self.maskh[z] or not runs:         # not run: nothing changes
                assert L_now[i] == Lp[i] and I_now[i] == Ip[i], (cache.step_index, z)
                continue
            assert Lp[i] == s_in and L_now[i] == s_out, (cache.step_index, z, Lp[i], L_now[i])
            assert I_now[i] == Ip[i] + 1
            self.fired.append((cache.step_index, z))
        if not runs:
            return
        # the same input state through the debug round at the oracle's r
        Kc, Vc, Nc, Lc = Kp[comp].clone(), Vp[comp].clone(), Np[comp].clone(), torch.from_numpy(
            Lp[comp].astype(np.int32)).to(Kp.device)
        best, sel, src, ws = lib.csm_compress_debug(Kc, Vc, Nc, Lc, w.n1, w.n2, w.c, r,
                                                    max_len=s_in)
        assert lib.read_error(ws) == lib.OK
        for j, i in enumerate(comp):
            z = zs[i]
            assert torch.equal(cache.K[z, :s_out], Kc[j, :s_out]), ("device r differs", z)
            assert torch.equal(cache.V[z, :s_out], Vc[j, :s_out]) and torch.equal(
                cache.N[z, :s_out], Nc[j, :s_out]), z
            parity.compare_slice(self.rep, parity.to_f64(Kp[i].cpu()), parity.to_f64(Vp[i].cpu()),
                                 Np[i].cpu().numpy().astype(np.int64), int(Lp[i]), w.n1, w.n2,
                                 w.c, r, "bf16", best[j].cpu().numpy(), sel[j].cpu().numpy(),
                                 src[j].cpu().numpy(), parity.to_f64(Kc[j].cpu()),
                                 parity.to_f64(Vc[j].cpu()), Nc[j].cpu().numpy().astype(np.int64),
                                 int(Lc[j]))


def test_algorithm1_device_trigger_64k_end_to_end(lib, dev):
    from kv_cache_clustering_amd.pipeline import ClusteredKVCache
    w = kvsynth.workload(4)
    osched = oschedule.run_algorithm1(w.ctx, w.R, w.steps, w.g, w.n1, w.n2, w.c, w.r_init,
                                      w.delta, w.r_min)
    assert len(osched["prefill"]) == 13 and [t[0] for t in osched["triggers"]] == [110]
    c = kvsynth.make_cache(w, dev)
    q_all = kvsynth.make_queries(w, dev)
    mask = c["mask"]
    maskh = mask.cpu().numpy()
    twin = [t.clone() for t in (c["K"], c["V"], c["N"], c["lens"])]
    sample = [z for z in range(3, 256, 41) if not maskh[z]][:6] + [int(np.argmax(maskh))]
    obs = DeviceLockstep(lib, sample, maskh, osched, w)
    kw = dict(H_q=w.H_q, H_kv=w.H_kv, n=w.ctx, R=w.R, Gamma=w.steps, g=w.g, n1=w.n1, n2=w.n2,
              c=w.c, r_init=w.r_init, delta=w.delta, r_min=w.r_min, outlier_mask=mask)
    A = ClusteredKVCache(c["K"], c["V"], c["N"], c["lens"], observer=obs, **kw)
    rs = A.prefill_device()
    assert obs.prefill_calls == 12 and len(rs) == 12
    L = A.lens.cpu().numpy()
    assert np.all(L[maskh == 0] == osched["prefill"][-1]) and np.all(L[maskh == 1] == w.ctx)
    assert np.all(A.round_idx.cpu().numpy() == np.where(maskh == 1, 0, 12))
    check = {1, 2, 109, 110, 111, 200, w.steps - 1}
    outs, fired_host, worst = [], [], 0.0
    for i in range(1, w.steps):
        O, r = A.decode_step_device(q_all[i], c["app_k"][i - 1], c["app_v"][i - 1])
        outs.append(O.clone())
        if r is not None:
            fired_host.append((i, r))
        s_want = osched["prefill"][-1] + i - sum(t[1] - t[2] for t in osched["triggers"] if t[0] <= i)
        assert int(A.lens[sample[0]]) == s_want, i
        if i in check:                              # attention saw the state before the round
            Kp, Vp, Np, Lp, _ = obs.pre
            Oh = O.cpu().double().numpy()
            for j, z in enumerate(sample):
                g, kvh = divmod(z, w.H_kv)
                s = int(Lp[j])
                Kz, Vz = parity.to_f64(Kp[j, :s].cpu()), parity.to_f64(Vp[j, :s].cpu())
                Nz = Np[j, :s].cpu().numpy().astype(np.int64)
                for h in range(w.G):
                    hq = kvh * w.G + h
                    ref = oatt.logn_attention_one(parity.to_f64(q_all[i, g, hq].cpu()), Kz, Vz, Nz)
                    worst = max(worst, float(np.abs(Oh[g, hq] - ref).max()))
    A.check_errors()
    comp = [z for z in sample if not maskh[z]]
    assert sorted(set(s for s, _ in obs.fired)) == [0, 110]
    assert [z for s, z in obs.fired if s == 110] == comp
    assert fired_host == [(t[0], t[3]) for t in osched["triggers"]]
    L = A.lens.cpu().numpy()
    assert np.all(L[maskh == 0] == osched["final"]) and np.all(L[maskh == 1] == w.ctx + w.steps - 1)
    assert np.all(A.round_idx.cpu().numpy() == np.where(maskh == 1, 0, osched["rounds"]))
    live = torch.arange(A.N.shape[1], device=dev)[None, :] < A.lens[:, None]
    Nsum = torch.where(live, A.N, 0).sum(dim=1, dtype=torch.int64).cpu().numpy()
    assert np.all(Nsum == w.ctx + w.steps - 1)
    print("device rounds in lockstep:", obs.rep, "decode max abs", worst)
    parity.check_report(obs.rep)
    assert obs.rep.slices == 6 * 13
    assert worst < 2e-4

    # the same run as whole-step graphs (51 steps per replay) on a twin cache
    del c["K"], c["V"], c["N"]
    B = ClusteredKVCache(*twin, **kw)
    assert B.prefill_device() == rs
    per = 51
    B.capture_loop(per)
    rounds_b = []
    for rep in range((w.steps - 1) // per):
        lo = rep * per
        Ob, rb = B.run_loop(q_all[lo + 1:lo + 1 + per], c["app_k"][lo:lo + per],
                            c["app_v"][lo:lo + per])
        torch.cuda.synchronize()
        rounds_b += rb
        for j in range(per):
            assert torch.equal(Ob[j], outs[lo + j]), (rep, j)
    B.check_errors()
    assert rounds_b == fired_host
    for x, y in ((A.K, B.K), (A.V, B.V), (A.N, B.N), (A.lens, B.lens), (A.round_idx, B.round_idx)):
        assert torch.equal(x, y)
