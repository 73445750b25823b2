"""Synthetic generator checks (statistics and the blocked AR(1) scan)."""
import numpy as np
import torch

import kvsynth
from kvsynth import gen


def test_blocked_scan_equals_plain_recursion():
    g = torch.Generator().manual_seed(0)
    x = torch.randn((3, 1000, 5), generator=g)
    rho = torch.tensor([0.5, 0.95, 0.99])
    y = gen._ar1_scan_torch(x, rho)
    ref = torch.empty_like(x)
    ref[:, 0] = x[:, 0]
    for t in range(1, 1000):
        ref[:, t] = rho.view(3, 1) * ref[:, t - 1] + x[:, t]
    torch.testing.assert_close(y, ref, atol=1e-4, rtol=1e-4)


def test_cache_statistics_small():
    w = kvsynth.workload(2, layers=2, ctx=4096, steps=4, cap_extra=4)
    c = kvsynth.make_cache(w, "cpu")
    K = c["K"].float()
    assert K.shape == (w.slices, w.cap, w.d) and c["K"].dtype == torch.bfloat16
    k = K[0, :4096].double().numpy()
    mu = k.mean(0)
    kc = k - mu
    lag1 = (kc[1:] * kc[:-1]).sum() / (kc * kc).sum()
    assert abs(lag1 - 0.95) < 0.02
    assert abs(kc.var() - 1.0) < 0.3
    v = c["V"][0, :4096].float().numpy()
    assert abs(v.mean()) < 0.02 and abs(v.var() - 1.0) < 0.03
    assert c["app_k"].shape == (4, w.slices, w.d)
    assert int(c["N"][0, :4096].sum()) == 4096 and int(c["N"][0, 4096:].sum()) == 0
    # the appended keys continue the AR(1) sequence
    last = K[0, 4095].double()
    nxt = c["app_k"][0, 0].double()
    assert torch.nn.functional.cosine_similarity(last, nxt, dim=0) > 0.6


def test_outlier_mask_count_and_broadcast():
    w = kvsynth.workload(4)
    m = kvsynth.outlier_mask(w)
    assert m.sum() == 10 and m.shape == (256,)
    w3 = kvsynth.workload(4, batch=3)
    m3 = kvsynth.outlier_mask(w3)
    assert m3.sum() == 30
    assert np.array_equal(m3[:256], m3[256:512])


def test_seeds_are_per_slice():
    w = kvsynth.workload(2, layers=1, ctx=300, steps=1, cap_extra=1)
    a = kvsynth.make_cache(w, "cpu", batch_slices=8)["K"]
    b = kvsynth.make_cache(w, "cpu", batch_slices=3)["K"]
    assert torch.equal(a, b)
