"""One round of Chunked Soft Matching (CSM) over a K/V cache, plain and step by step.

TEST INFRASTRUCTURE ONLY (see the package header).  Written from:
  * Chelsea review, section 三, 分块软匹配算法: step 1 (chunk the sequence, keep the first
    n1 sink tokens and the last n2 recent tokens), step 2 (alternating partition into A
    and B inside each chunk), step 3 (soft matching of the most similar A/B pairs),
    step 4 (merge each cluster's keys and values into one centre; the degree n_t counts
    the tokens a centre stands for); Algorithm 1 (K, V, N, s are rewritten by a round).
  * CentroidKV page, 技术摘要 / 方法论 / 分块软匹配 (CSM): cosine similarity of keys,
    bipartite soft matching in which each A token takes its most similar B token,
    candidate matches ranked by similarity and only the top fraction set by r merged;
    聚合: degree-weighted averaging of keys and values into one centroid, the degree
    accumulating over rounds.

Readings taken where the pages are silent:
  * A = chunk offsets 0, 2, 4, ... (the theorem's 1-indexed odd positions), B = offsets
    1, 3, 5, ...; A tokens are the sources that disappear, B tokens the targets that stay.
  * Chunks tile the middle [n1, s - n2) from n1; the last chunk may be shorter (length
    L < c) and is processed with its own length.  A chunk with no B token is untouched.
  * Similarity = cosine of the current keys; norms are floored at 1e-12.
  * Match: lowest B index among equal maxima.  Rank: descending score, equal scores
    take the lower A index first.  m = floor(r*L/2 + 1e-9) evaluated in fp64.
  * Merge: all sources of one target fold in with one weighted mean, summed in
    ascending A order; new degree = sum of degrees; stored back with RNE rounding.
  * Compaction keeps the original order; a centroid occupies its target's slot.
  * Outlier (masked) slices are left untouched.

Decisions are taken on the definition in fp64: every dot product is summed in one fixed
order for every pair of rows (so two identical rows score identically and exact ties
stay exact ties), norms likewise, and the cosine is the dot product over the product of
the two floored norms.

Pins (tests/oracle/): Theorem 6.1 brute force for the partition; argmax / ranking
properties on every chunk; r = 0 identity; sum of N conserved; first moments
sum(N*k), sum(N*v) conserved per chunk in fp64 storage; every centroid equals the plain
mean of the original tokens it stands for over several rounds; compaction order and
length closed form; identical-pair data give exact full attention (with attention.py);
hand-built 4-token chunks with known answers (tests/golden/csm_tiny_cases.json).
Merged values at generic inputs beyond these invariants: parity unpinned (the pages
print no worked example).
"""

import numpy as np

from .bf16 import round_to_storage

NORM_FLOOR = 1e-12
M_GUARD = 1e-9


def merge_count(r, L):
    """Number of A->B edges merged in a chunk of length L: floor(r*L/2), fp64, guarded."""
    if L < 2:
        return 0
    m = int(np.floor(float(r) * L / 2.0 + M_GUARD))
    return max(0, min(m, (L + 1) // 2))


def chunk_bounds(s, n1, n2, c):
    """[start, end) of every chunk of the middle [n1, s - n2), in order."""
    M = s - n1 - n2
    if M < 2:
        return []
    return [(a, min(a + c, n1 + M)) for a in range(n1, n1 + M, c)]


def partition(L):
    """Alternating partition of chunk offsets 0..L-1: A = even offsets, B = odd offsets."""
    return np.arange(0, L, 2), np.arange(1, L, 2)


def cosine_matrix(Ka, Kb):
    """Cosine similarity S[i, j] = <a_i, b_j> / (max(|a_i|, eps) * max(|b_j|, eps)), fp64.

    The dot products are evaluated element by element in the same summation order for every
    (i, j) (einsum's own loop, not a blocked matrix product whose order can depend on where
    a row sits in the block), so rows with equal values give bit-identical scores.
    """
    a = np.asarray(Ka, dtype=np.float64)
    b = np.asarray(Kb, dtype=np.float64)
    dots = np.einsum("ik,jk->ij", a, b)
    na = np.sqrt(np.einsum("ik,ik->i", a, a))
    nb = np.sqrt(np.einsum("jk,jk->j", b, b))
    den = np.maximum(na, NORM_FLOOR)[:, None] * np.maximum(nb, NORM_FLOOR)[None, :]
    return dots / den


def match(S):
    """Each A row takes its most similar B column; the lowest column wins a tie."""
    best = np.argmax(S, axis=1)          # numpy returns the first maximum
    score = S[np.arange(S.shape[0]), best]
    return best, score


def select_top(score, m):
    """Boolean mask of the m highest-ranked A rows: descending score, ties -> lower index."""
    order = np.argsort(-score, kind="stable")
    sel = np.zeros(score.shape[0], dtype=bool)
    sel[order[:m]] = True
    return sel


def csm_round_slice(K, V, N, s, n1, n2, c, r, storage="bf16", forced=None):
    """One CSM round over one slice.

    K, V : [cap, d] fp64 arrays holding the stored values; N : [cap] integer degrees;
    s : current length.  Rows at and beyond s are ignored and returned unchanged.
    storage : format the merged centroids are rounded to ('bf16', 'f16', 'f32' or 'f64').
    forced : optional {chunk start: (best_b, selected)} replacing the match and selection
    decisions of those chunks (used to follow another implementation's decisions where
    they differ only at a near-tie, so that merging and compaction can still be compared).
    Returns (K', V', N', s', taps) where taps['chunks'] holds one dict per chunk
    (start, L, m, best_b, score, selected, and S, the chunk's similarity matrix) and
    taps['src_pos'] maps every output row < s' to the input row it came from.
    """
    K = np.array(K, dtype=np.float64)
    V = np.array(V, dtype=np.float64)
    N = np.array(N, dtype=np.int64)
    cap = K.shape[0]
    Kout, Vout, Nout = K.copy(), V.copy(), N.copy()
    chunks = chunk_bounds(s, n1, n2, c)
    keep_rows = list(range(0, min(n1, s)))
    taps = []
    for (start, end) in chunks:
        L = end - start
        A, B = partition(L)
        rows_a, rows_b = start + A, start + B
        tap = {"start": start, "L": L, "m": 0}
        if B.size == 0:
            keep_rows.extend(range(start, end))
            taps.append(tap)
            continue
        S = cosine_matrix(K[rows_a], K[rows_b])
        best_b, score = match(S)
        m = merge_count(r, L)
        sel = select_top(score, m)
        if forced is not None and start in forced:
            best_b = np.asarray(forced[start][0], dtype=np.int64)
            sel = np.asarray(forced[start][1], dtype=bool)
        tap.update(m=m, best_b=best_b, score=score, selected=sel, S=S)
        taps.append(tap)
        # Degree-weighted merge: every selected A row folds into its matched B row.
        numk = {}
        numv = {}
        deg = {}
        for i in np.nonzero(sel)[0]:            # ascending A order
            b = int(best_b[i])
            tb = rows_b[b]
            if b not in deg:
                deg[b] = int(N[tb])
                numk[b] = N[tb] * K[tb]
                numv[b] = N[tb] * V[tb]
            ta = rows_a[i]
            deg[b] += int(N[ta])
            numk[b] = numk[b] + N[ta] * K[ta]
            numv[b] = numv[b] + N[ta] * V[ta]
        for b, W in deg.items():
            tb = rows_b[b]
            Kout[tb] = round_to_storage(numk[b] / W, storage)
            Vout[tb] = round_to_storage(numv[b] / W, storage)
            Nout[tb] = W
        removed = set(int(x) for x in rows_a[sel])
        keep_rows.extend(x for x in range(start, end) if x not in removed)
    if chunks:
        keep_rows.extend(range(chunks[-1][1], s))
    else:
        keep_rows = list(range(s))
    src_pos = np.array(keep_rows, dtype=np.int64)
    s_new = len(keep_rows)
    K2, V2, N2 = K.copy(), V.copy(), N.copy()
    K2[:s_new] = Kout[src_pos]
    V2[:s_new] = Vout[src_pos]
    N2[:s_new] = Nout[src_pos]
    assert s_new <= cap
    return K2, V2, N2, s_new, {"chunks": taps, "src_pos": src_pos}


def csm_compress(K, V, N, lens, n1, n2, c, r, outlier_mask=None, storage="bf16"):
    """One CSM round over every slice of a cache.

    K, V : [S, cap, d]; N : [S, cap]; lens : [S]; outlier_mask : [S] (nonzero = skip).
    Returns (K', V', N', lens', taps) with taps[slice] = None for skipped slices.
    """
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    N = np.asarray(N, dtype=np.int64)
    S_ = K.shape[0]
    K2, V2, N2 = K.copy(), V.copy(), N.copy()
    lens2 = np.array(lens, dtype=np.int64).copy()
    taps = []
    for z in range(S_):
        if outlier_mask is not None and outlier_mask[z]:
            taps.append(None)
            continue
        k, v, n, s2, t = csm_round_slice(K[z], V[z], N[z], int(lens[z]), n1, n2, c, r,
                                         storage)
        K2[z], V2[z], N2[z], lens2[z] = k, v, n, s2
        taps.append(t)
    return K2, V2, N2, lens2, taps
