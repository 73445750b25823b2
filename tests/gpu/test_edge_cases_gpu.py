"""The method's tie, zero-key and identical-group cases through the kernels, against the oracle.

Sources: CentroidKV page, 分块软匹配 (CSM) (each A token takes its most similar B token; the
matches are ranked and the top fraction merged) and Chelsea review, section 三, 分块软匹配算法
step 3; the tie readings (lowest B index for a match, lower A index at the selection cut) and
the zero-key reading (norms floored at 1e-12).  Chelsea review, section 三, 核心公式: when the
members of every cluster are identical, attention over the centroids with log N added equals
attention over the original cache.

Exact ties get no near-tie exemption: the parity protocol counts a decision that differs
where the fp64 scores are exactly equal as a hard error.  Each test also checks that the
case it plants was actually exercised (the report's exact-tie counters).
"""
import numpy as np
import pytest
import torch

from tests import parity
from tests.gpu.conftest import host_cache
from tests.gpu.test_csm_gpu import run_and_compare

pytestmark = pytest.mark.gpu

DT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}
# (storage, head dim, chunk) combinations: every storage format, both head dims, chunks up to
# 256 rows (one B part) and up to 512 rows (the 256 x 256 tile, two B parts merged in LDS)
COMBOS = [("bf16", 128, 256), ("bf16", 64, 256), ("f16", 128, 256), ("f32", 128, 256),
          ("f32", 64, 256), ("bf16", 128, 512), ("f16", 64, 512), ("bf16", 64, 100),
          ("f16", 128, 300)]


def _np_cache(S, cap, lens, d, seed, degrees=True):
    K, V, N, L = host_cache(S, cap, lens, d=d, dtype=torch.float32, seed=seed, degrees=degrees)
    return K.numpy().copy(), V.numpy().copy(), N.numpy().copy(), L


def _to(dt, K, V, N, L):
    return (torch.from_numpy(K).to(DT[dt]), torch.from_numpy(V).to(DT[dt]), torch.from_numpy(N), L)


def _chunks(s, n1, n2, c):
    M = s - n1 - n2
    return [(a, min(a + c, n1 + M)) for a in range(n1, n1 + M, c)] if M >= 2 else []


@pytest.mark.parametrize("dt,d,c", COMBOS)
def test_duplicate_b_rows_match_the_lowest_b(lib, dev, dt, d, c):
    """B rows copied onto other B rows of the same chunk (lower and higher indices, inside
    and across the 32-row MFMA tiles and, for c > 256, across the two B parts): every A row
    whose best match was copied ties between the copies and must take the lowest."""
    lens = [3000, 2100, 3000]
    K, V, N, L = _np_cache(3, 3000, lens, d, seed=c + d + len(dt))
    rng = np.random.default_rng(c * 3 + d)
    for z, s in enumerate(lens):
        for (a, b) in _chunks(s, 16, 64, c):
            nB = (b - a) // 2
            if nB < 2:
                continue
            for _ in range(max(2, nB // 6)):
                j, j2 = rng.choice(nB, 2, replace=False)
                K[z, a + 2 * j2 + 1] = K[z, a + 2 * j + 1]
    for r in (0.5, 1.0):
        rep = run_and_compare(lib, dev, *_to(dt, K, V, N, L), 16, 64, c, r)
        print(dt, d, c, r, rep)
        parity.check_report(rep)
        assert rep.exact_match_ties > 20


@pytest.mark.parametrize("dt,d,c", COMBOS)
def test_equal_scores_straddling_the_cut_select_the_lower_a(lib, dev, dt, d, c):
    """In every chunk a group of A rows (more than m of them, spread over the chunk) is one
    repeated vector u, and one B row is u as well, so the group shares the top score exactly
    and the selection cut falls inside it: the lowest-indexed members must be the ones merged.
    Other chunks get a smaller group (all selected) or random duplicate A rows."""
    lens = [3000, 2500]
    K, V, N, L = _np_cache(2, 3000, lens, d, seed=7 * c + d)
    rng = np.random.default_rng(11 * c + d)
    for z, s in enumerate(lens):
        for ci, (a, b) in enumerate(_chunks(s, 16, 64, c)):
            nA, nB = (b - a + 1) // 2, (b - a) // 2
            if nB < 2:
                continue
            u = rng.standard_normal(d)
            m_top = max(1, nA // 4) if ci % 3 else nA       # r = 0.5 merges about nA / 2
            grp = rng.choice(nA, size=min(nA, m_top + nA // 4 + 1), replace=False)
            if ci % 3 == 1:
                grp = grp[:max(1, nA // 8)]                # smaller than m: all merged
            K[z, a + 2 * grp] = u
            K[z, a + 2 * int(rng.integers(nB)) + 1] = u
    rep = run_and_compare(lib, dev, *_to(dt, K, V, N, L), 16, 64, c, 0.5)
    print(dt, d, c, rep)
    parity.check_report(rep)
    assert rep.exact_cut_ties >= 2


@pytest.mark.parametrize("dt,d,c", [("bf16", 128, 256), ("f16", 128, 256), ("f32", 128, 256),
                                    ("bf16", 64, 512), ("f32", 64, 64)])
def test_zero_and_tiny_norm_keys(lib, dev, dt, d, c):
    """Zero keys score 0 against everything (ties to the lowest B, and equal scores at the cut);
    keys whose norm is below the 1e-12 floor score as if their norm were 1e-12; keys just above
    it score as plain cosines.  fp16 cannot hold a norm near the floor (nor the elements of such
    a key, which would be subnormal), so there zero keys and keys scaled by 2^-4 and 2^-2 are
    planted.  A merge of a zero or tiny key into a target can leave a mean far below the terms it
    came from, where fp32 accumulation error exceeds one ulp of the result: the absolute floor of
    the value check is allowed here (and counted in the report)."""
    lens = [2600, 2600]
    K, V, N, L = _np_cache(2, 2600, lens, d, seed=17 + d + c)
    rng = np.random.default_rng(23 + d)
    tiny, small = (1e-14, 1e-11) if dt != "f16" else (2.0 ** -4, 2.0 ** -2)
    for z, s in enumerate(lens):
        for ci, (a, b) in enumerate(_chunks(s, 16, 64, c)):
            L_ = b - a
            rows = rng.choice(L_, size=max(2, L_ // 5), replace=False) + a
            kinds = rng.integers(0, 3, size=rows.size)
            for row, kind in zip(rows, kinds):
                K[z, row] = 0.0 if kind == 0 else K[z, row] * (tiny if kind == 1 else small)
            if ci == 0:                                  # a chunk of zero keys only
                K[z, a:b] = 0.0
    total = parity.Report()
    for r in (0.5, 1.0):
        rep = run_and_compare(lib, dev, *_to(dt, K, V, N, L), 16, 64, c, r)
        print(dt, d, c, r, rep)
        parity.check_report(rep, floor_allowed=True)
        total.add(rep)
    assert total.exact_match_ties > 0 and total.exact_cut_ties > 0


def _grouped_cache(S, s, d, group, seed):
    """Every group of `group` consecutive rows of the middle [16, s - 64) holds one vector (K
    and V), all groups distinct; sinks and recent rows distinct; degrees 1."""
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((S, s, d))
    V = rng.standard_normal((S, s, d))
    for z in range(S):
        for g0 in range(16, s - 64, group):
            K[z, g0:g0 + group] = K[z, g0]
            V[z, g0:g0 + group] = V[z, g0]
    return K.astype(np.float32), V.astype(np.float32), np.ones((S, s), np.int32)


@pytest.mark.parametrize("dt,d,c", [("bf16", 128, 256), ("f16", 128, 256), ("f32", 128, 256),
                                    ("bf16", 64, 512), ("f16", 64, 128), ("f32", 64, 256)])
@pytest.mark.parametrize("group", [2, 4])
def test_identical_groups_give_exact_attention(lib, dev, dt, d, c, group):
    """Pairs (one round at r = 1) or quads (two rounds at r = 1) of identical rows: every merge
    joins a group's members, so the compressed cache holds each group once with N = group,
    and log-N decode attention over it equals plain softmax attention over the original
    cache.  The rounds are also compared with the oracle as usual."""
    from oracle import attention as oatt
    S, H_kv, H_q = 4, 2, 8
    s = 16 + 4 * 256 * 2 + 64 + (0 if c != 128 else 128)    # middle: whole chunks, multiple of 4
    Kf, Vf, Nf = _grouped_cache(S, s, d, group, seed=31 + group + d + c)
    K, V, N = torch.from_numpy(Kf).to(DT[dt]), torch.from_numpy(Vf).to(DT[dt]), torch.from_numpy(Nf)
    L = torch.full((S,), s, dtype=torch.int32)
    Korig, Vorig = parity.to_f64(K), parity.to_f64(V)
    Kd, Vd, Nd, Ld = K.to(dev), V.to(dev), N.to(dev), L.to(dev)
    rep = parity.Report()
    for rnd in range(group // 2):
        Kc, Vc, Nc, Lc = Kd.cpu(), Vd.cpu(), Nd.cpu(), Ld.cpu()
        best, sel, src, ws = lib.csm_compress_debug(Kd, Vd, Nd, Ld, 16, 64, c, 1.0)
        assert lib.read_error(ws) == lib.OK
        for z in range(S):
            parity.compare_slice(rep, parity.to_f64(Kc[z]), parity.to_f64(Vc[z]),
                                 Nc[z].numpy().astype(np.int64), int(Lc[z]), 16, 64, c, 1.0, dt,
                                 best[z].cpu().numpy(), sel[z].cpu().numpy(), src[z].cpu().numpy(),
                                 parity.to_f64(Kd[z].cpu()), parity.to_f64(Vd[z].cpu()),
                                 Nd[z].cpu().numpy().astype(np.int64), int(Ld[z]))
    print(dt, d, c, group, rep)
    parity.check_report(rep)
    assert rep.followed_chunks == 0
    M = s - 80
    s_new = 16 + M // group + 64
    assert Ld.cpu().tolist() == [s_new] * S
    Nh = Nd.cpu().numpy()
    assert np.all(Nh[:, 16:s_new - 64] == group) and np.all(Nh[:, :16] == 1)
    q = torch.randn((S // H_kv, H_q, d), generator=torch.Generator().manual_seed(group + d)).to(DT[dt])
    O = lib.decode_attn_logn(q.to(dev), Kd, Vd, Nd, Ld, H_q, H_kv).cpu().double().numpy()
    qh = parity.to_f64(q)
    worst = 0.0
    for z in range(S):
        g, kvh = divmod(z, H_kv)
        for h in range(H_q // H_kv):
            hq = kvh * (H_q // H_kv) + h
            full = oatt.softmax_attention_one(qh[g, hq], Korig[z], Vorig[z])
            worst = max(worst, float(np.abs(O[g, hq] - full).max()))
    print("compressed log-N attention vs full attention over the original cache:", worst)
    assert worst < 1e-4
