"""Pins of the oracle's delta rule (the DeltaNet recurrence of
"linear_sparse_attention.py", function delta_rule_recurrent, and its checks
[d] and [e] in main()).

* the page's check [d]: without the erase term and with beta = 1 the state
  is the additive sum of k v^T;
* the page's check [e]: for orthonormal keys with beta = 1 the erase term
  changes nothing, for random unit keys it does;
* retrieval: with unit keys and beta = 1 the state maps k_t exactly to v_t,
  so reading with q_t = k_t returns v_t; with beta in (0, 1) it returns the
  mix (1 - beta) k_t^T S_{t-1} + beta v_t;
* beta = 0 leaves S0 untouched;
* the explicit product form S_L = prod_t (I - beta_t k_t k_t^T) ... with
  d x d matrices on tiny inputs;
* the chunkwise form with the triangular (UT) transform, written here in
  numpy independently of the oracle, equals the token loop for several chunk
  lengths and a ragged tail (the form the GPU prefill uses);
* two planted mistakes (erase dropped, erase after the write) are caught.
"""
import numpy as np
import pytest

import oracle


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def test_additive_fallback_is_the_plain_sum():
    rng = np.random.default_rng(0)
    L, d = 13, 6
    K = _unit(rng.standard_normal((L, d)))
    V = rng.standard_normal((L, d))
    _, S = oracle.delta_run(K, K, V, np.ones(L), use_delta=False)
    assert np.allclose(S, K.T @ V, rtol=0, atol=1e-12)


def test_erase_term_vanishes_exactly_for_orthonormal_keys():
    rng = np.random.default_rng(1)
    d = 6
    Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    Ko = Qm.T                                   # d orthonormal rows
    Vo = rng.standard_normal((d, d))
    _, S_delta = oracle.delta_run(Ko, Ko, Vo, np.ones(d))
    _, S_add = oracle.delta_run(Ko, Ko, Vo, np.ones(d), use_delta=False)
    assert np.abs(S_delta - S_add).max() < 1e-12
    K = _unit(rng.standard_normal((13, d)))
    V = rng.standard_normal((13, d))
    _, a = oracle.delta_run(K, K, V, np.ones(13))
    _, b = oracle.delta_run(K, K, V, np.ones(13), use_delta=False)
    assert np.linalg.norm(a - b) > 1e-3


def test_unit_key_retrieval():
    rng = np.random.default_rng(2)
    L, dk, dv = 9, 5, 3
    K = _unit(rng.standard_normal((L, dk)))
    V = rng.standard_normal((L, dv))
    S0 = rng.standard_normal((dk, dv))
    out, _ = oracle.delta_run(K, K, V, np.ones(L), S0=S0)
    assert np.allclose(out, V, rtol=0, atol=1e-12)
    beta = rng.uniform(0.1, 0.9, L)
    out_b, _ = oracle.delta_run(K, K, V, beta, S0=S0)
    prev = S0
    for t in range(L):
        want = (1 - beta[t]) * (K[t] @ prev) + beta[t] * V[t]
        assert np.allclose(out_b[t], want, rtol=0, atol=1e-12)
        _, prev = oracle.delta_run(K[:t + 1], K[:t + 1], V[:t + 1], beta[:t + 1], S0=S0)


def test_zero_strength_keeps_the_initial_state():
    rng = np.random.default_rng(3)
    L, dk, dv = 7, 4, 5
    Q, K = rng.standard_normal((2, L, dk))
    V = rng.standard_normal((L, dv))
    S0 = rng.standard_normal((dk, dv))
    out, S = oracle.delta_run(Q, K, V, np.zeros(L), S0=S0)
    assert np.array_equal(S, S0)
    assert np.allclose(out, Q @ S0, rtol=0, atol=1e-12)


def test_explicit_product_form():
    rng = np.random.default_rng(4)
    L, dk, dv = 6, 4, 3
    Q, K = rng.standard_normal((2, L, dk))
    V = rng.standard_normal((L, dv))
    beta = rng.uniform(0, 1, L)
    S0 = rng.standard_normal((dk, dv))
    S = S0.copy()
    outs = []
    for t in range(L):
        E = np.eye(dk) - beta[t] * np.outer(K[t], K[t])
        S = E @ S + beta[t] * np.outer(K[t], V[t])
        outs.append(Q[t] @ S)
    out, Sf = oracle.delta_run(Q, K, V, beta, S0=S0)
    assert np.allclose(out, np.array(outs), rtol=0, atol=1e-12)
    assert np.allclose(Sf, S, rtol=0, atol=1e-12)


def _chunkwise_ut(Q, K, V, beta, S0, C):
    """Chunkwise delta rule: per chunk, T = (I + strict_lower(diag(beta) K
    K^T))^-1 diag(beta), W = T K, U = T V, U' = U - W S, O = Q S +
    (Q K^T * inclusive mask) U', S <- S + K^T U'."""
    L = Q.shape[0]
    S = S0.copy()
    out = np.zeros((L, V.shape[1]))
    for c0 in range(0, L, C):
        q, k, v, b = Q[c0:c0 + C], K[c0:c0 + C], V[c0:c0 + C], beta[c0:c0 + C]
        n = q.shape[0]
        A = np.tril(b[:, None] * (k @ k.T), -1)
        T = np.linalg.solve(np.eye(n) + A, np.diag(b))
        W, U = T @ k, T @ v
        Up = U - W @ S
        out[c0:c0 + n] = q @ S + np.tril(q @ k.T) @ Up
        S = S + k.T @ Up
    return out, S


@pytest.mark.parametrize("C", [1, 4, 7, 16])
def test_chunkwise_ut_form_equals_the_loop(C):
    rng = np.random.default_rng(5 + C)
    L, dk, dv = 23, 8, 5
    Q = rng.standard_normal((L, dk))
    K = _unit(rng.standard_normal((L, dk)))
    V = rng.standard_normal((L, dv))
    beta = rng.uniform(0, 1, L)
    S0 = rng.standard_normal((dk, dv))
    ref, Sr = oracle.delta_run(Q, K, V, beta, S0=S0)
    got, Sg = _chunkwise_ut(Q, K, V, beta, S0, C)
    assert np.allclose(got, ref, rtol=0, atol=1e-10)
    assert np.allclose(Sg, Sr, rtol=0, atol=1e-10)


def test_batched_pairs_are_independent():
    rng = np.random.default_rng(6)
    B, H, L, d = 2, 3, 11, 4
    q, k, v = rng.standard_normal((3, B, H, L, d))
    beta = rng.uniform(0, 1, (B, H, L))
    out, S = oracle.delta_run(q, k, v, beta, nthreads=4)
    for b in range(B):
        for h in range(H):
            o1, S1 = oracle.delta_run(q[b, h], k[b, h], v[b, h], beta[b, h])
            assert np.array_equal(out[b, h], o1) and np.array_equal(S[b, h], S1)


@pytest.mark.parametrize("mutation", ["delta_no_erase", "delta_erase_after"])
def test_planted_delta_mistakes_are_caught(mutation):
    with oracle.mutation(mutation):
        failed = 0
        for fn in (test_unit_key_retrieval, test_explicit_product_form,
                   lambda: test_chunkwise_ut_form_equals_the_loop(4)):
            try:
                fn()
            except AssertionError:
                failed += 1
    assert failed >= 2
