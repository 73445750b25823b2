"""decode_attn_logn_noalloc (the entry point for callers that cannot allocate) against
decode_attn_logn: bit-identical outputs and error words on consecutive calls, the second over
a smaller input, with nothing allocated by the call itself."""
import os
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

pytestmark = pytest.mark.gpu


def _cache(dev, S, cap, seed, dtype=torch.bfloat16):
    gen = torch.Generator(device=dev).manual_seed(seed)
    K = torch.randn((S, cap, 128), generator=gen, device=dev).to(dtype)
    V = torch.randn((S, cap, 128), generator=gen, device=dev).to(dtype)
    N = torch.randint(1, 9, (S, cap), generator=gen, device=dev, dtype=torch.int32)
    L = torch.randint(0, cap + 1, (S,), generator=gen, device=dev, dtype=torch.int32)
    return K, V, N, L, gen


def test_noalloc_decode_matches_workspace_decode():
    from kv_cache_clustering_amd import _lib as lib
    from oracle import attention as oatt
    from tests import parity
    dev = torch.device("cuda:0")
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    calls = [(64, 5000, 16, 4, torch.bfloat16), (8, 900, 8, 2, torch.float16)]
    for i, (S, cap, H_q, H_kv, dt) in enumerate(calls):
        K, V, N, L, gen = _cache(dev, S, cap, seed=70 + i, dtype=dt)
        L[1] = 0
        q = torch.randn((S // H_kv, H_q, 128), generator=gen, device=dev).to(dt)
        ref = lib.decode_attn_logn(q, K, V, N, L, H_q, H_kv, max_len=cap)
        out = torch.full_like(ref, float("nan"))
        torch.cuda.synchronize()
        before = torch.cuda.memory_stats(dev)["allocation.all.allocated"]
        lib.decode_attn_logn_noalloc(q, K, V, N, L, H_q, H_kv, out, err, max_len=cap)
        after = torch.cuda.memory_stats(dev)["allocation.all.allocated"]
        assert after == before, "the call allocated through torch"
        assert lib.read_error(err) == lib.OK, i
        assert torch.equal(out, ref), i
        G = H_q // H_kv
        for z in (0, 1, S - 1):
            s = int(L[z])
            g, kvh = divmod(z, H_kv)
            want = oatt.logn_attention_one(parity.to_f64(q[g, kvh * G].cpu()),
                                           parity.to_f64(K[z, :s].cpu()),
                                           parity.to_f64(V[z, :s].cpu()),
                                           N[z, :s].cpu().numpy().astype(np.int64))
            assert np.abs(out[g, kvh * G].cpu().double().numpy() - want).max() < 2e-4
    # a bad length: both variants give zeros for that slice and set their error words
    K, V, N, L, gen = _cache(dev, 8, 900, seed=99)
    L[3] = 901
    q = torch.randn((4, 8, 128), generator=gen, device=dev).to(torch.bfloat16)
    ws = lib.new_workspace(lib.decode_workspace_bytes(K, 8, 2, max_len=900), dev)
    ref = lib.decode_attn_logn(q, K, V, N, L, 8, 2, max_len=900, workspace=ws)
    out = torch.empty_like(ref)
    lib.decode_attn_logn_noalloc(q, K, V, N, L, 8, 2, out, err, max_len=900)
    assert lib.read_error(ws) == lib.EDEVICE and lib.read_error(err) == lib.EDEVICE
    assert torch.equal(out, ref) and torch.all(out[1, 4:8] == 0)
    lib.clear_error(err)
    assert lib.read_error(err) == lib.OK


def test_noalloc_rejects_geometries_beyond_its_scratch():
    from kv_cache_clustering_amd import _lib as lib
    dev = torch.device("cuda:0")
    S, cap = 8192, 32896
    K = torch.empty((S, 1, 128), dtype=torch.bfloat16, device=dev)   # shape checks only
    desc_need = lib.raw.decode_attn_logn_workspace_bytes(
        lib.ctypes.byref(lib.CacheDesc(S, cap, 128, lib.BF16, cap)), 32, 32)
    assert desc_need > lib.NOALLOC_SCRATCH_BYTES
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    O = torch.empty((S // 32, 32, 128), dtype=torch.float32, device=dev)
    rc = lib.raw.decode_attn_logn_noalloc(
        lib._ptr(K), lib._ptr(K), lib._ptr(K), lib._ptr(err), lib._ptr(err),
        lib.ctypes.byref(lib.CacheDesc(S, cap, 128, lib.BF16, cap)), 32, 32, lib._ptr(O),
        lib._ptr(err), None)
    assert rc == lib.EWORKSPACE
    assert lib.read_error(err) == lib.OK
