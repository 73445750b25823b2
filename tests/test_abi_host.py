"""Host-only checks of the C ABI: the library loads, exports every declared entry point,
and rejects bad arguments before enqueuing anything (no GPU work is started here)."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "kv_cache_clustering_amd", "libcsmkv.so")
HDR = os.path.join(ROOT, "include", "csmkv.h")


def _declared():
    text = open(HDR).read()
    return re.findall(r"^CSMKV_API\s+[\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libcsmkv.so is not built: run __graft_entry__.build()")
    from kv_cache_clustering_amd import _lib
    return _lib


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert len(names) == 23
    raw = ctypes.CDLL(LIB)
    for n in names:
        assert hasattr(raw, n), n
    assert set(names) == set(lib.EXPORTED)


def test_status_strings_and_version(lib):
    assert lib.version() == 106
    for code in range(-6, 1):
        assert lib.status_string(code).startswith("CSMKV_")
    assert "unknown" in lib.status_string(-99)


def _desc(lib, S=4, cap=1000, d=128, dtype=0, max_len=1000):
    return lib.CacheDesc(S, cap, d, dtype, max_len)


def test_workspace_sizes(lib):
    d = _desc(lib)
    units = lib.raw.csm_compress_units(ctypes.byref(d), 16, 64, 256)
    assert units == math.ceil((1000 - 80) / 256) + 1
    ws = lib.raw.csm_compress_workspace_bytes(ctypes.byref(d), 16, 64, 256)
    assert ws >= 4 * (4 * units) + 2 * 4 * 4 and ws % 256 == 0
    assert lib.raw.csm_compress_workspace_bytes(ctypes.byref(d), 16, 64, 1) == 0
    assert lib.raw.csm_compress_workspace_bytes(ctypes.byref(_desc(lib, d=96)), 16, 64, 256) == 0
    dws = lib.raw.decode_attn_logn_workspace_bytes(ctypes.byref(d), 8, 2)
    assert dws >= 4 * 2 * (2 + 128) * 4 * 2
    assert lib.raw.decode_attn_logn_workspace_bytes(ctypes.byref(d), 6, 4) == 0
    assert lib.raw.decode_attn_logn_workspace_bytes(ctypes.byref(d), 32, 2) == 0  # G = 16


FAKE = ctypes.c_void_p(1 << 20)  # never dereferenced: every call below fails validation


def _compress(lib, desc, n1=16, n2=64, c=256, r=0.5, K=FAKE, ws=FAKE, ws_bytes=1 << 30):
    return lib.raw.csm_compress(K, FAKE, FAKE, FAKE, ctypes.byref(desc), n1, n2, c, r, None, ws,
                                ws_bytes, None)


def test_compress_argument_validation(lib):
    d = _desc(lib)
    assert _compress(lib, d, r=1.5) == lib.EINVAL
    assert _compress(lib, d, r=-0.1) == lib.EINVAL
    assert _compress(lib, d, r=float("nan")) == lib.EINVAL
    assert _compress(lib, d, c=1) == lib.EINVAL
    assert _compress(lib, d, c=513) == lib.EUNSUPPORTED
    assert _compress(lib, _desc(lib, dtype=1), c=257) == lib.EUNSUPPORTED  # fp32: c <= 256
    assert _compress(lib, d, n1=-1) == lib.EINVAL
    assert _compress(lib, d, n2=-3) == lib.EINVAL
    assert _compress(lib, d, K=None) == lib.EINVAL
    assert _compress(lib, d, K=ctypes.c_void_p((1 << 20) + 8)) == lib.EINVAL  # misaligned
    assert _compress(lib, d, ws=None) == lib.EWORKSPACE
    assert _compress(lib, d, ws_bytes=16) == lib.EWORKSPACE
    assert _compress(lib, d, ws=ctypes.c_void_p((1 << 20) + 64)) == lib.EWORKSPACE
    assert _compress(lib, _desc(lib, dtype=7)) == lib.EDTYPE
    assert _compress(lib, _desc(lib, d=96)) == lib.EUNSUPPORTED
    assert _compress(lib, _desc(lib, max_len=1001)) == lib.EINVAL
    assert _compress(lib, _desc(lib, cap=0, max_len=0)) == lib.EINVAL
    assert _compress(lib, _desc(lib, cap=(1 << 24) + 1, max_len=10)) == lib.EUNSUPPORTED
    assert lib.raw.csm_compress(FAKE, FAKE, FAKE, FAKE, None, 16, 64, 256, 0.5, None, FAKE,
                                1 << 30, None) == lib.EINVAL


def test_compress_into_rejects_aliasing_and_mismatch(lib):
    d = _desc(lib)
    args = (FAKE, FAKE, FAKE, FAKE, ctypes.byref(d), FAKE, ctypes.c_void_p(2 << 20),
            ctypes.c_void_p(3 << 20), ctypes.c_void_p(4 << 20), ctypes.byref(d), 16, 64, 256,
            0.5, None, FAKE, 1 << 30, None)
    assert lib.raw.csm_compress_into(*args) == lib.EINVAL          # K_in == K_out
    d2 = _desc(lib, S=5)
    args2 = (FAKE, FAKE, FAKE, FAKE, ctypes.byref(d), ctypes.c_void_p(5 << 20),
             ctypes.c_void_p(2 << 20), ctypes.c_void_p(3 << 20), ctypes.c_void_p(4 << 20),
             ctypes.byref(d2), 16, 64, 256, 0.5, None, FAKE, 1 << 30, None)
    assert lib.raw.csm_compress_into(*args2) == lib.EINVAL         # slice counts differ


def test_triggered_argument_validation(lib):
    d = _desc(lib)

    def trig(thr=FAKE, idx=FAKE, r_init=0.5, r_delta=0.05, r_min=0.1, c=256, ws_bytes=1 << 30):
        return lib.raw.csm_compress_triggered(FAKE, FAKE, FAKE, FAKE, ctypes.byref(d), 16, 64, c,
                                              thr, idx, r_init, r_delta, r_min, None, FAKE,
                                              ws_bytes, None)

    assert trig(thr=None) == lib.EINVAL
    assert trig(idx=None) == lib.EINVAL
    assert trig(r_init=1.5) == lib.EINVAL
    assert trig(r_init=0.05) == lib.EINVAL          # below r_min
    assert trig(r_min=-0.1) == lib.EINVAL
    assert trig(r_delta=-0.01) == lib.EINVAL
    assert trig(r_delta=float("nan")) == lib.EINVAL
    assert trig(r_min=float("nan")) == lib.EINVAL
    assert trig(c=600) == lib.EUNSUPPORTED
    assert trig(ws_bytes=8) == lib.EWORKSPACE


def test_debug_taps_must_come_together(lib):
    d = _desc(lib)
    rc = lib.raw.csm_compress_debug(FAKE, FAKE, FAKE, FAKE, ctypes.byref(d), 16, 64, 256, 0.5,
                                    None, FAKE, 1 << 30, None, FAKE, None, None)
    assert rc == lib.EINVAL


def test_decode_and_append_validation(lib):
    d = _desc(lib, S=8)
    dec = lib.raw.decode_attn_logn
    assert dec(FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(d), 6, 4, FAKE, FAKE, 1 << 30, None) == lib.EINVAL
    assert dec(FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(d), 48, 3, FAKE, FAKE, 1 << 30, None) == lib.EINVAL
    assert dec(FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(d), 64, 4, FAKE, FAKE, 1 << 30, None) == lib.EUNSUPPORTED
    assert dec(None, FAKE, FAKE, FAKE, FAKE, ctypes.byref(d), 16, 4, FAKE, FAKE, 1 << 30, None) == lib.EINVAL
    assert dec(FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(d), 16, 4, FAKE, FAKE, 8, None) == lib.EWORKSPACE
    app = lib.raw.kv_append
    assert app(FAKE, FAKE, FAKE, None, ctypes.byref(d), FAKE, FAKE, None, None) == lib.EINVAL
    assert app(FAKE, FAKE, FAKE, FAKE, ctypes.byref(_desc(lib, dtype=3)), FAKE, FAKE, None, None) == lib.EDTYPE
    assert lib.raw.csmkv_read_error(None, None) == lib.EINVAL
    assert lib.raw.csmkv_clear_error(None, None) == lib.EINVAL


def test_upload_validation(lib):
    """csm_upload_rows checks its pointers, row_begin and every host length before enqueuing."""
    import numpy as np
    up = lib.raw.csm_upload_rows
    d = _desc(lib, S=3, cap=100, max_len=100)
    lens = np.array([100, 50, 101], np.int32)
    lp = ctypes.c_void_p(lens.ctypes.data)
    assert up(FAKE, FAKE, FAKE, lp, FAKE, FAKE, FAKE, FAKE, ctypes.byref(d), 0, None, None) == lib.EINVAL
    lens[2] = 7
    assert up(FAKE, FAKE, FAKE, lp, FAKE, FAKE, FAKE, FAKE, ctypes.byref(d), -1, None, None) == lib.EINVAL
    assert up(None, FAKE, FAKE, lp, FAKE, FAKE, FAKE, FAKE, ctypes.byref(d), 0, None, None) == lib.EINVAL
    assert up(FAKE, FAKE, FAKE, lp, FAKE, FAKE, FAKE, FAKE, ctypes.byref(_desc(lib, d=96)), 0, None,
              None) == lib.EUNSUPPORTED


def test_noalloc_decode_validation(lib):
    """The allocation-free decode rejects a missing error word and any geometry whose partials
    would not fit its fixed scratch array, before touching the GPU."""
    noa = lib.raw.decode_attn_logn_noalloc
    d = _desc(lib, S=256, cap=65792, max_len=65792)            # 64K workload, G = 4: fits
    assert lib.raw.decode_attn_logn_workspace_bytes(ctypes.byref(d), 32, 8) <= lib.NOALLOC_SCRATCH_BYTES
    assert noa(FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(d), 32, 8, FAKE, None, None) == lib.EINVAL
    assert noa(FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(d), 6, 4, FAKE, FAKE, None) == lib.EINVAL
    big = _desc(lib, S=8192, cap=32896, max_len=32896)          # 8192 slices of 32K, G = 1
    assert lib.raw.decode_attn_logn_workspace_bytes(ctypes.byref(big), 32, 32) > lib.NOALLOC_SCRATCH_BYTES
    assert noa(FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(big), 32, 32, FAKE, FAKE, None) == lib.EWORKSPACE
    assert lib.raw.csmkv_clear_error(ctypes.c_void_p(FAKE.value + 2), None) == lib.EINVAL


def _items_for_lengths(S, max_len, lens):
    """Work items a decode call lays out for these lengths, by the rule the decode kernel
    states: calls over at most 1024 slices take an item size of the total length over 256
    items, rounded up to 16 tokens, within [256, 2048]; larger calls take the smallest of 512,
    1024 and 2048 tokens that is at least S * max_len / 2048 (else 2048).  A slice of s tokens
    has ceil(s / item size) items; lengths above the bound count none."""
    ok = [s for s in lens if 0 <= s <= max_len]
    if S <= 1024:
        T = sum(ok)
        ts = min(max(-(-(-(-T // 256)) // 16) * 16, 256), 2048)
    else:
        want, ts = S * max_len // 2048, 512
        while ts < 2048 and ts < want:
            ts *= 2
    return sum(-(-s // ts) for s in ok)


def test_decode_workspace_holds_every_item_plan(lib):
    """The decode workspace must hold one (max, sum, pad, o[d]) fp32 partial per item and head
    for any lengths within the bound: random geometries (both planning rules), random and
    extreme length mixes, against the size the library asks for."""
    rng = np.random.default_rng(5)
    cases = [(8, 65792), (256, 65792), (1024, 6200), (1025, 6200), (3, 1), (1, 300000),
             (1000, 2049), (1100, 513)]
    cases += [(int(rng.integers(1, 1500)), int(rng.integers(1, 70000))) for _ in range(40)]
    for S, max_len in cases:
        for d, G in ((128, 4), (64, 8), (128, 1)):
            H_kv = 1
            desc = lib.CacheDesc(S, max_len, d, 0, max_len)
            ws = lib.raw.decode_attn_logn_workspace_bytes(ctypes.byref(desc), G * H_kv, H_kv)
            assert ws > 0
            part = G * (4 + d) * 4
            mixes = [[max_len] * S, [1] * S, [0] * (S - 1) + [max_len],
                     list(rng.integers(0, max_len + 1, size=S)),
                     list(rng.choice([1, max_len, max_len // 2 + 1, 2049, 257], size=S))]
            for lens in mixes:
                items = _items_for_lengths(S, max_len, [int(x) for x in lens])
                assert items * part + (S + 1) * 4 <= ws, (S, max_len, d, G, items, ws)


def test_binding_checks_the_host_cache_first(lib):
    """csm_upload_rows' binding rejects a host cache whose V, N or lens do not match K (the
    library would read past them) before it looks at the device tensors."""
    import torch
    K = torch.zeros((2, 8, 64), dtype=torch.bfloat16)
    V = torch.zeros((2, 8, 64), dtype=torch.bfloat16)
    N = torch.zeros((2, 8), dtype=torch.int32)
    L = torch.zeros(2, dtype=torch.int32)
    bad = [(K, torch.zeros((2, 4, 64), dtype=torch.bfloat16), N, L), (K, V, N.to(torch.int64), L), (K, V, N, L[:1]),
           (K, V.to(torch.float16), N, L)]
    for kh, vh, nh, lh in bad:
        with pytest.raises(ValueError, match="host cache"):
            lib.csm_upload_rows(kh, vh, nh, lh, K, V, N, L)
    with pytest.raises(ValueError, match="outlier_mask"):
        lib.csm_upload_rows(K, V, N, L, K, V, N, L, outlier_mask=torch.zeros(3, dtype=torch.uint8))
