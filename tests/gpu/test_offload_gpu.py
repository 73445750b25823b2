"""CPU-offloaded clustering end to end: a host mirror of the device cache clustered on the host
(csm_compress_host), the compacted rows sent back with csm_upload_rows, then decode attention on
the device over the result.

CentroidKV page, 它做不到的事（局限性） → 仍留在 GPU 上: grouping on the CPU, only the result sent to
the GPU.  Checked: the device cache after the upload equals the host result bit for bit (rows
[0, lens), lengths; outlier slices and rows before row_begin untouched); the host round and the
device round (csm_compress_debug on a copy) both pass the oracle protocol, and their decisions
are identical in every slice where neither met a near-tie; decode attention over the uploaded
cache matches the oracle.
"""
import numpy as np
import pytest
import torch

import kvsynth
from oracle import attention as oatt
from tests import parity

pytestmark = pytest.mark.gpu


def _pinned_like(t):
    return torch.empty(t.shape, dtype=t.dtype, pin_memory=True)


def test_offload_round_trip_64k_slices(lib, dev):
    w = kvsynth.workload(4)
    c = kvsynth.make_cache(w, dev, with_appends=False)
    maskh = c["mask"].cpu().numpy()
    zs = sorted(set(range(0, 256, 16)) | {int(np.argmax(maskh))})   # 16 slices + one outlier
    K, V, N, L = (c[k][zs].contiguous() for k in ("K", "V", "N", "lens"))
    mask = torch.as_tensor(maskh[zs], dtype=torch.uint8)
    del c
    S = len(zs)
    Kg, Vg, Ng, Lg = K.clone(), V.clone(), N.clone(), L.clone()       # the device round's copy
    # host mirror (pinned), clustered on the host's cores
    Kh, Vh, Nh, Lh = (_pinned_like(t) for t in (K, V, N, L))
    for h, d in ((Kh, K), (Vh, V), (Nh, N), (Lh, L)):
        h.copy_(d)
    Kin, Vin, Nin, lin = Kh.clone(), Vh.clone(), Nh.clone(), Lh.clone()
    best_h, sel_h, src_h = lib.csm_compress_host(Kh, Vh, Nh, Lh, w.n1, w.n2, w.c, w.r_init, mask,
                                                 taps=True, max_len=w.ctx)
    lib.csm_upload_rows(Kh, Vh, Nh, Lh, K, V, N, L, row_begin=w.n1, outlier_mask=mask)
    torch.cuda.synchronize()
    assert torch.equal(L.cpu(), Lh)
    for z in range(S):
        s = int(Lh[z])
        assert torch.equal(K[z, :s].cpu(), Kh[z, :s]) and torch.equal(V[z, :s].cpu(), Vh[z, :s]), z
        assert torch.equal(N[z, :s].cpu(), Nh[z, :s]), z
        if mask[z]:
            assert torch.equal(K[z].cpu(), Kin[z]) and int(L[z]) == w.ctx
    # the device round on the same input, and both against the oracle
    best_g, sel_g, src_g, ws = lib.csm_compress_debug(Kg, Vg, Ng, Lg, w.n1, w.n2, w.c, w.r_init,
                                                      mask.to(dev), max_len=w.ctx)
    assert lib.read_error(ws) == lib.OK
    rep_h, rep_g = parity.Report(), parity.Report()
    same_slices = tie_slices = 0
    for z in range(S):
        if mask[z]:
            continue
        args = (parity.to_f64(Kin[z]), parity.to_f64(Vin[z]), Nin[z].numpy().astype(np.int64),
                int(lin[z]), w.n1, w.n2, w.c, w.r_init, "bf16")
        zh, zg = parity.Report(), parity.Report()
        parity.compare_slice(zh, *args, best_h[z].numpy(), sel_h[z].numpy(), src_h[z].numpy(),
                             parity.to_f64(Kh[z]), parity.to_f64(Vh[z]),
                             Nh[z].numpy().astype(np.int64), int(Lh[z]))
        parity.compare_slice(zg, *args, best_g[z].cpu().numpy(), sel_g[z].cpu().numpy(),
                             src_g[z].cpu().numpy(), parity.to_f64(Kg[z].cpu()),
                             parity.to_f64(Vg[z].cpu()), Ng[z].cpu().numpy().astype(np.int64),
                             int(Lg[z]))
        rep_h.add(zh)
        rep_g.add(zg)
        s = int(Lh[z])
        same = torch.equal(best_h[z], best_g[z].cpu()) and torch.equal(sel_h[z], sel_g[z].cpu())
        if zh.match_near + zh.sel_near + zg.match_near + zg.sel_near == 0:
            # neither round met a near-tie in this slice: both took the definition's decisions
            assert same, z
        else:
            tie_slices += 1
        if same:
            same_slices += 1
            assert torch.equal(Nh[z, :s], Ng[z, :s].cpu())
            # merged values: host divides, the device multiplies by a reciprocal; both within
            # one bf16 step of the oracle, so of each other by at most two
            hk = parity.to_f64(Kh[z, :s]).ravel()
            gk = parity.to_f64(Kg[z, :s].cpu()).ravel()
            assert parity.max_ulp_bf16(hk, gk) <= 2
    print("host round:", rep_h, "\ndevice round:", rep_g, "\nslices with identical decisions:",
          same_slices, "slices with a near-tie on either side:", tie_slices)
    parity.check_report(rep_h)
    parity.check_report(rep_g)
    # decode attention on the device over the uploaded cache
    H_kv, G = 1, 4
    q = torch.randn((S, G, 128), generator=torch.Generator(device=dev).manual_seed(5),
                    device=dev).to(torch.bfloat16)
    O = lib.decode_attn_logn(q, K, V, N, L, G, H_kv).cpu().double().numpy()
    worst = 0.0
    for z in (0, S // 2, S - 1):
        s = int(Lh[z])
        for h in range(G):
            ref = oatt.logn_attention_one(parity.to_f64(q[z, h].cpu()), parity.to_f64(Kh[z, :s]),
                                          parity.to_f64(Vh[z, :s]), Nh[z, :s].numpy().astype(np.int64))
            worst = max(worst, float(np.abs(O[z, h] - ref).max()))
    print("decode over the uploaded cache, max abs", worst)
    assert worst < 2e-4


def test_upload_validates_and_copies_only_unmasked_slices(lib, dev):
    from tests.gpu.conftest import host_cache
    K, V, N, L = host_cache(4, 900, [900, 500, 0, 700], seed=8, degrees=True)
    Kd, Vd, Nd, Ld = (torch.zeros_like(t).to(dev) for t in (K, V, N, L))
    mask = torch.tensor([0, 1, 0, 0], dtype=torch.uint8)
    lib.csm_upload_rows(K, V, N, L, Kd, Vd, Nd, Ld, row_begin=10, outlier_mask=mask)
    torch.cuda.synchronize()
    assert Ld.cpu().tolist() == [900, 0, 0, 700]
    assert torch.equal(Kd[0, 10:900].cpu(), K[0, 10:900]) and torch.all(Kd[0, :10] == 0)
    assert torch.equal(Vd[3, 10:700].cpu(), V[3, 10:700]) and torch.equal(Nd[3, 10:700].cpu(), N[3, 10:700])
    assert torch.all(Kd[1] == 0) and torch.all(Nd[1] == 0)
    bad = L.clone()
    bad[3] = 901
    with pytest.raises(lib.CsmkvError) as e:
        lib.csm_upload_rows(K, V, N, bad, Kd, Vd, Nd, Ld, row_begin=0)
    assert e.value.status == lib.EINVAL
