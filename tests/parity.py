"""GPU-vs-oracle comparison helpers (test infrastructure).

Protocol (near-tie aware, per chunk), on the same stored input bits:
  * the reference decisions are the oracle's, taken on the definition in fp64;
  * a differing match index is a near-tie if the GPU's B scores within 1e-5 of the best B's
    fp64 similarity and strictly below it: an exact tie in the definition has one answer
    (the lowest B index), so a different choice there is a hard error;
  * a differing selection is a near-tie if the edge's fp64 score lies within 1e-5 of the
    selection cut [s_(m+1), s_(m)], unless an edge the GPU took and one it left have
    exactly equal fp64 scores (an exact tie at the cut resolves to the lower A index);
  * chunks with a near-tie are re-run in the oracle with the GPU's decisions ("follow"),
    so merging, degrees and compaction are still compared everywhere;
  * then lens, src_pos and N must match exactly and K, V within one ulp of the storage
    format;
  * the bar: no hard mismatch, and near-tie mismatches under 0.1% of the A edges.
"""
import numpy as np
import torch

from oracle import bf16 as obf16
from oracle import csm as ocsm
from oracle import fp16 as of16

NEAR = 1e-5


def to_f64(t):
    """Stored cache values (bf16, fp16 or fp32 tensor) -> exact fp64 numpy array."""
    if t.dtype == torch.bfloat16:
        return obf16.bits_to_f64(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
    return t.cpu().double().numpy()


def ordered_bf16(bits):
    b = bits.astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)


def max_ulp_bf16(gpu_vals, oracle_vals):
    """Largest distance in bf16 steps between two arrays of bf16-representable values."""
    g = ordered_bf16(obf16.f64_to_bits(gpu_vals))
    o = ordered_bf16(obf16.f64_to_bits(oracle_vals))
    return int(np.max(np.abs(g - o))) if g.size else 0


ABS_FLOOR = 2.0 ** -20


def ordered_f16(bits):
    b = bits.astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)


def check_values(rep, gpu_vals, oracle_vals, storage):
    """Merged values agree within one ulp of the storage format (bf16 steps for bf16 and
    fp32 storage, fp16 steps for fp16) of the oracle's value.  Where a weighted mean
    cancels to a value far below its terms, fp32 accumulation error (about 2**-24 of the
    terms) can exceed one ulp of the tiny result; such elements pass when the absolute
    difference is below 2**-20 and are counted in rep.abs_floor_used (rep.abs_floor_used_f32 for
    fp32 storage)."""
    g = np.asarray(gpu_vals, np.float64)
    o = np.asarray(oracle_vals, np.float64)
    if g.size == 0:
        return
    diff = np.abs(g - o)
    rep.max_abs = max(rep.max_abs, float(diff.max()))
    if storage == "bf16":
        ulp = np.abs(ordered_bf16(obf16.f64_to_bits(g)) - ordered_bf16(obf16.f64_to_bits(o)))
        rep.max_ulp = max(rep.max_ulp, int(ulp.max()))
        bad = ulp > 1
    elif storage == "f16":
        ulp = np.abs(ordered_f16(of16.f64_to_bits(g)) - ordered_f16(of16.f64_to_bits(o)))
        rep.max_ulp = max(rep.max_ulp, int(ulp.max()))
        bad = ulp > 1
    else:
        _, e = np.frexp(o)
        ulp_bf16 = np.ldexp(1.0, np.maximum(e, -125) - 8)
        bad = diff > ulp_bf16
    floor_ok = bad & (diff <= ABS_FLOOR)
    if storage == "f32":
        rep.abs_floor_used_f32 += int(floor_ok.sum())
    else:
        rep.abs_floor_used += int(floor_ok.sum())
    hard = bad & ~floor_ok
    assert not hard.any(), ("K/V differ by more than one ulp", storage, float(diff[hard].max()))


def max_ulp_f32(gpu_vals, oracle_vals):
    g = np.asarray(gpu_vals, np.float32).view(np.int32).astype(np.int64)
    o = np.asarray(oracle_vals, np.float32).view(np.int32).astype(np.int64)
    g = np.where(g < 0, -(g & 0x7FFFFFFF), g)
    o = np.where(o < 0, -(o & 0x7FFFFFFF), o)
    return int(np.max(np.abs(g - o))) if g.size else 0


class Report:
    def __init__(self):
        self.edges = 0
        self.match_near = 0
        self.match_hard = 0
        self.sel_near = 0
        self.sel_hard = 0
        self.followed_chunks = 0
        self.max_ulp = 0
        self.max_abs = 0.0
        self.abs_floor_used = 0      # 16-bit storage
        self.abs_floor_used_f32 = 0  # fp32 storage (compared against one bf16 step: see check_values)
        self.slices = 0
        self.exact_match_ties = 0   # A rows whose best fp64 score is attained by >= 2 B rows
        self.exact_cut_ties = 0     # chunks whose selection cut falls inside a run of equal scores

    def near_fraction(self):
        return (self.match_near + self.sel_near) / max(1, self.edges)

    def __repr__(self):
        return (f"Report(slices={self.slices}, edges={self.edges}, match_near={self.match_near}, "
                f"match_hard={self.match_hard}, sel_near={self.sel_near}, sel_hard={self.sel_hard}, "
                f"followed={self.followed_chunks}, max_ulp={self.max_ulp}, "
                f"max_abs={self.max_abs:.3g}, abs_floor_used={self.abs_floor_used}, "
                f"abs_floor_used_f32={self.abs_floor_used_f32}, "
                f"near_frac={self.near_fraction():.2e}, exact_match_ties={self.exact_match_ties}, "
                f"exact_cut_ties={self.exact_cut_ties})")

    def add(self, other):
        """Accumulate another report's counts into this one."""
        for f in ("edges", "match_near", "match_hard", "sel_near", "sel_hard", "followed_chunks",
                  "abs_floor_used", "abs_floor_used_f32", "slices", "exact_match_ties",
                  "exact_cut_ties"):
            setattr(self, f, getattr(self, f) + getattr(other, f))
        self.max_ulp = max(self.max_ulp, other.max_ulp)
        self.max_abs = max(self.max_abs, other.max_abs)


def compare_slice(rep, Kin, Vin, Nin, s, n1, n2, c, r, storage, gpu_best, gpu_sel, gpu_src,
                  gpu_K, gpu_V, gpu_N, gpu_len):
    """Compare one slice's GPU round against the oracle; raises AssertionError on failure."""
    rep.slices += 1
    first = ocsm.csm_round_slice(Kin, Vin, Nin, s, n1, n2, c, r, storage)
    taps = first[4]
    forced = {}
    for j, t in enumerate(taps["chunks"]):
        if "best_b" not in t:
            continue
        nA = len(t["best_b"])
        rep.edges += nA
        gb = gpu_best[j, :nA].astype(np.int64)
        gs = gpu_sel[j, :nA].astype(bool)
        assert np.all(gpu_best[j, nA:] == -1) and not gpu_sel[j, nA:].any()
        S64 = t["S"]
        nB = S64.shape[1]
        best = S64.max(axis=1)
        rep.exact_match_ties += int(np.sum(np.sum(S64 == best[:, None], axis=1) > 1))
        m = t["m"]
        sc = np.sort(best)[::-1]
        if 0 < m < nA and sc[m - 1] == sc[m]:
            rep.exact_cut_ties += 1
        bad_b = np.nonzero(gb != t["best_b"])[0]
        bad_s = np.nonzero(gs != t["selected"])[0]
        if bad_b.size == 0 and bad_s.size == 0:
            continue
        for i in bad_b:
            assert 0 <= gb[i] < nB, ("GPU match index out of range", t["start"], i, gb[i])
            if best[i] - NEAR <= S64[i, gb[i]] < best[i]:
                rep.match_near += 1
            else:
                rep.match_hard += 1
        if bad_s.size:
            hi = sc[m - 1] if m >= 1 else np.inf
            lo = sc[m] if m < nA else -np.inf
            taken = set(best[i] for i in bad_s if gs[i])
            left = set(best[i] for i in bad_s if not gs[i])
            exact_wrong = bool(taken & left)
            for i in bad_s:
                v = best[i]
                if lo - NEAR <= v <= hi + NEAR and not exact_wrong:
                    rep.sel_near += 1
                else:
                    rep.sel_hard += 1
        assert int(gs.sum()) == t["m"], ("GPU merged a different number of edges", t["start"])
        forced[t["start"]] = (gb, gs)
    rep.followed_chunks += len(forced)
    if forced:
        K2, V2, N2, s2, taps2 = ocsm.csm_round_slice(Kin, Vin, Nin, s, n1, n2, c, r, storage,
                                                     forced=forced)
    else:
        K2, V2, N2, s2, taps2 = first
    assert gpu_len == s2, ("length", gpu_len, s2)
    assert np.array_equal(gpu_src[:s2], taps2["src_pos"]), "src_pos differs"
    assert np.array_equal(gpu_N[:s2], N2[:s2]), "N differs"
    for g, o in ((gpu_K[:s2], K2[:s2]), (gpu_V[:s2], V2[:s2])):
        check_values(rep, g, o, storage)


def check_report(rep, near_bar=1e-3, floor_allowed=False):
    """No hard mismatch, near-ties below near_bar of the A edges, and (unless the inputs are built
    to make weighted means cancel) no 16-bit merged value that needed the absolute floor.  fp32
    storage is held to one bf16 step of the oracle's value; where a mean of terms of order one
    cancels to ~1e-6 or below, fp32 accumulation error alone exceeds that step, so its floor uses
    are counted and reported (about three per million merged edges on random data), not refused."""
    assert rep.match_hard == 0 and rep.sel_hard == 0, rep
    assert rep.near_fraction() < near_bar, rep
    if not floor_allowed:
        assert rep.abs_floor_used == 0, rep
