"""Pins for oracle.attention (Chelsea review, section 三, 核心公式; Algorithm 1 decode update)."""
import numpy as np
import torch

from oracle import attention, bf16, csm


def _sdpa(q, K, V):
    """torch CPU fp64 scaled_dot_product_attention for one query."""
    qt = torch.from_numpy(np.asarray(q, np.float64)).view(1, 1, 1, -1)
    kt = torch.from_numpy(np.asarray(K, np.float64)).view(1, 1, K.shape[0], -1)
    vt = torch.from_numpy(np.asarray(V, np.float64)).view(1, 1, V.shape[0], -1)
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt).view(-1).numpy()


def test_degree_one_is_textbook_attention():
    rng = np.random.default_rng(0)
    for T in (1, 7, 300):
        q, K, V = rng.standard_normal(64), rng.standard_normal((T, 64)), rng.standard_normal((T, 64))
        np.testing.assert_allclose(attention.logn_attention_one(q, K, V, np.ones(T)), _sdpa(q, K, V),
                                   atol=1e-13)


def test_expansion_identity_any_cache():
    rng = np.random.default_rng(1)
    T, d = 50, 32
    q, K, V = rng.standard_normal(d), rng.standard_normal((T, d)), rng.standard_normal((T, d))
    N = rng.integers(1, 9, size=T)
    Kx, Vx = np.repeat(K, N, axis=0), np.repeat(V, N, axis=0)
    np.testing.assert_allclose(attention.logn_attention_one(q, K, V, N), _sdpa(q, Kx, Vx), atol=1e-13)
    np.testing.assert_allclose(attention.weighted_attention_one(q, K, V, N),
                               attention.logn_attention_one(q, K, V, N), atol=1e-13)


def test_identical_pairs_give_exact_full_attention():
    """Offsets 2i and 2i+1 of every chunk identical, all pairs distinct: r=1 merges every
    A into its twin with N=2, and log-N attention equals full attention over the original."""
    rng = np.random.default_rng(2)
    s, n1, n2, c, d = 16 + 4 * 64 + 64, 16, 64, 64, 32
    base = rng.standard_normal((s, d))
    vb = rng.standard_normal((s, d))
    K = base.copy(); V = vb.copy()
    for t in range(n1, s - n2, 2):
        K[t + 1] = K[t]; V[t + 1] = V[t]
    K, V = bf16.round_to_bf16(K), bf16.round_to_bf16(V)
    N = np.ones(s, np.int64)
    K2, V2, N2, s2, _ = csm.csm_round_slice(K, V, N, s, n1, n2, c, 1.0)
    assert s2 == n1 + (s - n1 - n2) // 2 + n2
    assert sorted(set(N2[:s2].tolist())) == [1, 2]
    for _ in range(5):
        q = rng.standard_normal(d)
        full = _sdpa(q, K, V)
        np.testing.assert_allclose(attention.logn_attention_one(q, K2[:s2], V2[:s2], N2[:s2]), full,
                                   atol=1e-13)
    # quads over two rounds
    K = base.copy(); V = vb.copy()
    for t in range(n1, s - n2, 4):
        K[t + 1:t + 4] = K[t]; V[t + 1:t + 4] = V[t]
    N = np.ones(s, np.int64)
    Ka, Va, Na, sa, _ = csm.csm_round_slice(K, V, N, s, n1, n2, c, 1.0, storage="f64")
    Kb, Vb, Nb, sb, _ = csm.csm_round_slice(Ka, Va, Na, sa, n1, n2, c, 1.0, storage="f64")
    assert sb < sa < s and int(Nb[:sb].sum()) == s
    q = rng.standard_normal(d)
    np.testing.assert_allclose(attention.logn_attention_one(q, Kb[:sb], Vb[:sb], Nb[:sb]), _sdpa(q, K, V),
                               atol=1e-12)


def test_gqa_mapping_matches_torch_enable_gqa():
    rng = np.random.default_rng(3)
    groups, H_q, H_kv, T, d = 2, 8, 2, 40, 16
    q = rng.standard_normal((groups, H_q, d))
    K = rng.standard_normal((groups * H_kv, T + 3, d))
    V = rng.standard_normal((groups * H_kv, T + 3, d))
    N = np.ones((groups * H_kv, T + 3), np.int64)
    lens = np.full(groups * H_kv, T)
    O = attention.decode_attn_logn(q, K, V, N, lens, H_q, H_kv)
    qt = torch.from_numpy(q).view(groups, H_q, 1, d)
    kt = torch.from_numpy(K[:, :T]).view(groups, H_kv, T, d)
    vt = torch.from_numpy(V[:, :T]).view(groups, H_kv, T, d)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, enable_gqa=True).view(groups, H_q, d)
    np.testing.assert_allclose(O, ref.numpy(), atol=1e-13)


def test_empty_slice_is_zero_and_append():
    q = np.ones((1, 1, 4))
    K = np.zeros((1, 3, 4)); V = np.zeros((1, 3, 4)); N = np.zeros((1, 3), np.int64)
    O = attention.decode_attn_logn(q, K, V, N, np.array([0]), 1, 1)
    assert np.all(O == 0)
    K2, V2, N2, lens2 = attention.kv_append(K, V, N, np.array([0]), np.full((1, 4), 2.0), np.full((1, 4), 3.0))
    assert lens2[0] == 1 and N2[0, 0] == 1 and np.all(K2[0, 0] == 2.0) and np.all(V2[0, 0] == 3.0)
    O = attention.decode_attn_logn(q, K2, V2, N2, lens2, 1, 1)
    np.testing.assert_allclose(O[0, 0], 3.0)
