"""Log-degree decode attention and cache append (test infrastructure only).

Written from the Chelsea review, section 三, 核心公式:
  * original attention  Attn(q, K, V) = sum_i exp(q.k_i/sqrt(d)) v_i / sum_i exp(q.k_i/sqrt(d));
  * clustered approximation with centres k^_t, v^_t and degrees n_t, in which each
    exponential is weighted by n_t;
  * the same written as O = Softmax(q K^T / sqrt(d) + log N) V (natural log),
and Algorithm 1's decode update (append k, v to K, V, append 1 to N, s = s + 1, then
attend).  Grouped-query reading: query head h reads kv head floor(h / (H_q / H_kv)).

Pins (tests/oracle/test_attention.py): with N = 1 it equals torch's CPU fp64
scaled_dot_product_attention; for any (K^, V^, N) it equals plain softmax attention over
the cache with row t repeated n_t times; the weighted-sum form and the log-N form agree.
"""

import numpy as np


def logn_attention_one(q, K, V, N):
    """O = softmax(q K^T / sqrt(d) + ln N) V for one query vector, in fp64."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    if K.shape[0] == 0:
        return np.zeros(V.shape[1], dtype=np.float64)
    d = q.shape[0]
    z = K @ q / np.sqrt(d) + np.log(np.asarray(N, dtype=np.float64))
    w = np.exp(z - z.max())
    return (w @ V) / w.sum()


def weighted_attention_one(q, K, V, N):
    """The clustered approximation as printed: sum n_t e^{q.k_t/sqrt d} v_t / sum n_t e^{...}."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    d = q.shape[0]
    z = K @ q / np.sqrt(d)
    w = np.asarray(N, dtype=np.float64) * np.exp(z - z.max())
    return (w @ np.asarray(V, dtype=np.float64)) / w.sum()


def softmax_attention_one(q, K, V):
    """Plain softmax attention (the page's original formula)."""
    return logn_attention_one(q, K, V, np.ones(np.asarray(K).shape[0]))


def decode_attn_logn(q, K, V, N, lens, H_q, H_kv):
    """Grouped-query log-N decode attention over a sliced cache.

    q : [groups, H_q, d]; K, V : [groups * H_kv, cap, d]; N : [groups * H_kv, cap];
    lens : [groups * H_kv].  Returns O : [groups, H_q, d] in fp64.  An empty slice
    gives a zero output.
    """
    q = np.asarray(q, dtype=np.float64)
    groups = q.shape[0]
    G = H_q // H_kv
    O = np.zeros(q.shape, dtype=np.float64)
    for g in range(groups):
        for h in range(H_q):
            z = g * H_kv + h // G
            s = int(lens[z])
            O[g, h] = logn_attention_one(q[g, h], K[z, :s], V[z, :s], N[z, :s])
    return O


def kv_append(K, V, N, lens, k_new, v_new):
    """Algorithm 1 decode update: K=[K,k], V=[V,v], N=[N,1], s=s+1, per slice (copies)."""
    K = np.array(K, dtype=np.float64)
    V = np.array(V, dtype=np.float64)
    N = np.array(N, dtype=np.int64)
    lens = np.array(lens, dtype=np.int64)
    for z in range(K.shape[0]):
        s = int(lens[z])
        K[z, s] = k_new[z]
        V[z, s] = v_new[z]
        N[z, s] = 1
        lens[z] = s + 1
    return K, V, N, lens
