"""Hierarchical centroid index over a clustered cache and attention over the rows it keeps.

TEST INFRASTRUCTURE ONLY (see the package header).  Written from the LycheeCluster page,
方法论 §2 层次 KV 索引 (each block's KV vectors summarised by a compact centroid; the centroids
organised as a binary tree whose node distances obey the triangle inequality; at inference the
query walks the tree and drops whole subtrees whose centroid is too far, so the candidate set
shrinks from O(N) to O(log N)) and §3 流式懒更新 (a new token updates only the leaf of the most
recent block; the upper centroids are recomputed lazily), applied to the cache that Chunked Soft
Matching leaves (rows k, v with degrees N; Chelsea review, section 三, 核心公式 for log-N
attention).

Readings (the page gives only this outline):
  * Blocks are fixed runs of B consecutive rows of a slice (the page's boundary detector needs
    a model and is not built).  Block b holds rows [bB, min((b+1)B, s)).
  * A node is a ball: centre mu = degree-weighted mean of its keys (a leaf) or of its children's
    centres weighted by their degree totals (an inner node); radius rho = the largest distance
    from mu to a member key (a leaf) or max over children of |mu_c - mu| + rho_c (an inner node,
    so every child ball lies inside its parent's: the triangle inequality); lmax = the largest
    log2 N of its rows.  The tree is the complete binary tree over P = 2^ceil(log2(leaves))
    leaf slots in heap order (root 1, children 2u and 2u+1, leaf b at P + b); nodes over no
    rows are empty.
  * "Too far" is read as a bound on the attention logit: for every key k in a ball,
    q.k <= q.mu + |q| rho (Cauchy-Schwarz and the triangle inequality), so in base 2 every
    logit z = log2(e) (q.k / sqrt(d)) + log2 N of the node's rows is at most
    U = log2(e) (q.mu + |q| rho) / sqrt(d) + lmax.
  * The rows of the blocks that hold a protected row (the first n1 and the last n2 of the slice)
    are always kept; m_low = the largest exact logit among the protected rows and the first row
    of every block (real rows, so a lower bound on the maximum logit); a block is kept when
    U >= m_low - tau * log2(e) (tau in natural-log units)
    for at least one of the G query heads that share the slice (so K and V are read once per KV
    head).  The walk descends into a node only if the node passes; since a child's ball lies in
    its parent's, this keeps exactly the blocks that pass the test themselves.
  * Attention over the kept rows is the log-N attention of attention.py; tau = inf keeps every
    block, i.e. full log-N attention.  A dropped row weighs at most 2^(-tau log2 e) = e^-tau of
    the maximum row (which is always kept), so the output moves by at most
    2 e^-tau (dropped rows) max|v| (with degrees counted in the row weights).
  * Lazy update on append: the new row joins the last leaf, or opens a new leaf whose centre is
    the row and radius 0; the leaf's centre does not move, its radius grows to cover the row;
    each ancestor's radius grows to cover its updated child ball (an empty ancestor takes the
    child's ball); centres are recomputed only when the index is rebuilt.  Bounds stay valid and
    can only loosen, so the kept set can only grow relative to a rebuild.

Pins (tests/oracle/test_index.py): every row's logit is below its leaf's and every ancestor's
bound (brute force); the tree walk keeps exactly the leaves the direct test keeps; tau = inf
gives full log-N attention; the dropped-mass error bound holds; after lazy appends the bounds
stay valid and the kept set contains a fresh rebuild's; a four-row tree with unequal degrees,
worked by hand from the definitions above (tests/golden/index_tiny_case.json), fixes its centres,
radii, largest log-degrees, two bounds and two lazy appends.  Values at generic inputs beyond
these pins: parity unpinned (the page prints no worked example).
"""

import numpy as np

LOG2E = 1.4426950408889634


def build(K, N, s, B, cap=None):
    """Index of the first s rows of one slice: dict of heap arrays (index 1..2P-1), with leaf
    slots for `cap` rows (default s) so that appended rows find their leaf."""
    K = np.asarray(K, dtype=np.float64)
    N = np.asarray(N, dtype=np.int64)
    d = K.shape[1]
    nleaf = -(-s // B)
    P = 1
    while P < max(nleaf, -(-(cap or s) // B)):
        P *= 2
    mu = np.zeros((2 * P, d))
    rho = np.zeros(2 * P)
    lmax = np.full(2 * P, -np.inf)
    wt = np.zeros(2 * P, dtype=np.int64)
    for b in range(nleaf):
        rows = slice(b * B, min((b + 1) * B, s))
        w = N[rows]
        u = P + b
        wt[u] = int(w.sum())
        mu[u] = (w[:, None] * K[rows]).sum(axis=0) / wt[u]
        rho[u] = np.sqrt(((K[rows] - mu[u]) ** 2).sum(axis=1)).max()
        lmax[u] = np.log2(w.astype(np.float64)).max()
    for u in range(P - 1, 0, -1):
        kids = [c for c in (2 * u, 2 * u + 1) if wt[c] > 0]
        if not kids:
            continue
        wt[u] = sum(int(wt[c]) for c in kids)
        mu[u] = sum(wt[c] * mu[c] for c in kids) / wt[u]
        rho[u] = max(np.sqrt(((mu[c] - mu[u]) ** 2).sum()) + rho[c] for c in kids)
        lmax[u] = max(lmax[c] for c in kids)
    return {"P": P, "B": B, "nleaf": nleaf, "mu": mu, "rho": rho, "lmax": lmax, "wt": wt}


def bound(idx, u, q):
    """Base-2 upper bound on the logit of every row under node u for query q."""
    q = np.asarray(q, dtype=np.float64)
    d = q.shape[0]
    return LOG2E * (q @ idx["mu"][u] + np.linalg.norm(q) * idx["rho"][u]) / np.sqrt(d) + idx["lmax"][u]


def logits(q, K, N):
    q = np.asarray(q, dtype=np.float64)
    return LOG2E * (np.asarray(K, np.float64) @ q) / np.sqrt(q.shape[0]) + np.log2(np.asarray(N, np.float64))


def protected_blocks(s, n1, n2, B):
    """Blocks that hold one of the first n1 or the last n2 rows."""
    rows = [r for r in range(min(n1, s))] + [r for r in range(max(s - n2, 0), s)]
    return sorted(set(r // B for r in rows))


def reference_rows(s, n1, n2, B):
    """Rows whose exact logits give the lower bound m_low: the protected rows and the first row
    of every block."""
    return sorted(set(list(range(min(n1, s))) + list(range(max(s - n2, 0), s)) +
                      list(range(0, s, B))))


def thresholds(qs, K, N, s, n1, n2, tau, B):
    """Per query head: m_low - tau log2(e), m_low the best exact logit of a reference row."""
    ref = reference_rows(s, n1, n2, B)
    out = []
    for q in qs:
        m_low = logits(q, K[ref], N[ref]).max() if ref else -np.inf
        out.append(m_low - tau * LOG2E)
    return np.array(out)


def kept_direct(idx, qs, T, forced):
    """Leaves kept by testing every leaf: a protected block, or a bound at or above the
    threshold for some head."""
    keep = np.zeros(idx["nleaf"], dtype=bool)
    keep[forced] = True
    for b in range(idx["nleaf"]):
        u = idx["P"] + b
        if any(bound(idx, u, q) >= t for q, t in zip(qs, T)):
            keep[b] = True
    return keep


def kept_tree(idx, qs, T, forced):
    """Leaves kept by walking the tree from the root, dropping a subtree whose node fails."""
    keep = np.zeros(idx["nleaf"], dtype=bool)
    keep[forced] = True
    stack = [1] if idx["wt"][1] > 0 else []
    while stack:
        u = stack.pop()
        if not any(bound(idx, u, q) >= t for q, t in zip(qs, T)):
            continue
        if u >= idx["P"]:
            keep[u - idx["P"]] = True
        else:
            stack.extend(c for c in (2 * u, 2 * u + 1) if idx["wt"][c] > 0)
    return keep


def kept_rows(keep, s, B):
    return np.array([r for r in range(s) if keep[r // B]], dtype=np.int64)


def pruned_attention(qs, K, V, N, s, n1, n2, B, tau, idx=None, keep=None):
    """Log-N attention of every query head over the rows the index keeps.  Returns (O [G, d],
    keep [leaves])."""
    from .attention import logn_attention_one
    if idx is None:
        idx = build(K, N, s, B)
    if keep is None:
        T = thresholds(qs, K, N, s, n1, n2, tau, B)
        keep = kept_tree(idx, qs, T, protected_blocks(s, n1, n2, B))
    rows = kept_rows(keep, s, B)
    O = np.stack([logn_attention_one(q, K[rows], V[rows], N[rows]) for q in qs])
    return O, keep


def append_lazy(idx, k, n_new, s_new):
    """Update the index for the row s_new - 1 (key k, degree n_new) just appended."""
    P, B = idx["P"], idx["B"]
    r = s_new - 1
    b = r // B
    if b >= P:
        raise ValueError("the tree has no leaf slot for this row")
    k = np.asarray(k, dtype=np.float64)
    u = P + b
    if r % B == 0:                    # a new leaf
        idx["mu"][u] = k
        idx["rho"][u] = 0.0
        idx["lmax"][u] = np.log2(n_new)
        idx["wt"][u] = n_new
        idx["nleaf"] = b + 1
    else:
        idx["rho"][u] = max(idx["rho"][u], np.sqrt(((k - idx["mu"][u]) ** 2).sum()))
        idx["lmax"][u] = max(idx["lmax"][u], np.log2(n_new))
        idx["wt"][u] += n_new
    c = u
    while c > 1:
        p = c // 2
        if idx["wt"][p] == 0:
            idx["mu"][p] = idx["mu"][c]
            idx["rho"][p] = idx["rho"][c]
            idx["lmax"][p] = idx["lmax"][c]
        else:
            idx["rho"][p] = max(idx["rho"][p],
                                np.sqrt(((idx["mu"][c] - idx["mu"][p]) ** 2).sum()) + idx["rho"][c])
            idx["lmax"][p] = max(idx["lmax"][p], idx["lmax"][c])
        idx["wt"][p] += n_new
        c = p
    return idx
