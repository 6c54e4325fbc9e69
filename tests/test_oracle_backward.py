"""Pins of the oracle's backward (the reverse-mode derivative of the token loop).

The pages give no gradients, so the backward is pinned by mathematics alone:

* central finite differences of the forward oracle (itself pinned by the
  pages' worked examples and closed forms) for every input that has a
  gradient, in every gate mode, with and without S0 and dS_final;
* the textbook gradients of the masked matrix product (Q K^T * tril) V for
  the ungated, identity-feature case;
* invariance under the checkpoint spacing;
* two planted mistakes (gradient not decayed, dq read from the previous
  state), each caught by the finite differences.
"""
import numpy as np
import pytest

import oracle

B, H, L, DK, DV = 1, 2, 6, 3, 2


def _inputs(seed, gate_mode, with_s0):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, H, L, DK))
    k = r.standard_normal((B, H, L, DK))
    v = r.standard_normal((B, H, L, DV))
    la = None
    if gate_mode == oracle.GATE_DIAG:
        la = -np.abs(r.standard_normal((B, H, L, DK))) * 0.5
    elif gate_mode == oracle.GATE_SCALAR:
        la = -np.abs(r.standard_normal((B, H, L))) * 0.5
    S0 = r.standard_normal((B, H, DK, DV)) if with_s0 else None
    Wo = r.standard_normal((B, H, L, DV))
    WS = r.standard_normal((B, H, DK, DV))
    return q, k, v, la, S0, Wo, WS


def _loss(q, k, v, la, S0, Wo, WS, gate_mode, gamma, phi):
    out, S, _ = oracle.run(q, k, v, gate_mode=gate_mode, gamma=gamma, log_alpha=la,
                           phi=phi, S0=S0)
    loss = float(np.sum(Wo * out))
    if WS is not None:
        loss += float(np.sum(WS * S))
    return loss


def _fd(fn, x, h=1e-6):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        old = x[idx]
        x[idx] = old + h
        fp = fn()
        x[idx] = old - h
        fm = fn()
        x[idx] = old
        g[idx] = (fp - fm) / (2 * h)
    return g


CASES = [
    # gate mode, gamma, phi, with S0, with dS_final
    (oracle.GATE_NONE, None, oracle.PHI_IDENTITY, False, False),
    (oracle.GATE_NONE, None, oracle.PHI_ELU1, True, True),
    (oracle.GATE_GAMMA, [0.8, 0.5], oracle.PHI_IDENTITY, True, True),
    (oracle.GATE_GAMMA, [0.0, 1.0], oracle.PHI_IDENTITY, True, False),
    (oracle.GATE_DIAG, None, oracle.PHI_IDENTITY, False, True),
    (oracle.GATE_DIAG, None, oracle.PHI_ELU1, True, True),
    (oracle.GATE_SCALAR, None, oracle.PHI_IDENTITY, True, True),
    (oracle.GATE_SCALAR, None, oracle.PHI_ELU1, False, True),
]


def _check_fd(case, seed=0, rtol=1e-6):
    gate_mode, gamma, phi, with_s0, with_dsf = case
    q, k, v, la, S0, Wo, WS = _inputs(seed, gate_mode, with_s0)
    if not with_dsf:
        WS = None
    g = oracle.backward(q, k, v, Wo, gate_mode=gate_mode, gamma=gamma, log_alpha=la,
                        phi=phi, S0=S0, dS_final=WS)
    f = lambda: _loss(q, k, v, la, S0, Wo, WS, gate_mode, gamma, phi)
    checks = [("dq", q), ("dk", k), ("dv", v)]
    if gate_mode in (oracle.GATE_DIAG, oracle.GATE_SCALAR):
        checks.append(("dlog_alpha", la))
    if with_s0:
        checks.append(("dS0", S0))
    for name, x in checks:
        num = _fd(f, x)
        scale = max(1.0, float(np.max(np.abs(num))))
        err = float(np.max(np.abs(g[name] - num))) / scale
        assert err < rtol, f"{name}: finite-difference mismatch {err:.3e} ({case})"


@pytest.mark.parametrize("case", CASES)
def test_backward_matches_finite_differences(case):
    _check_fd(case)


def test_dS0_of_zero_state_run_is_the_decayed_gradient():
    # with S0 = None the initial state is zero; dS0 is still the gradient of
    # the loss with respect to it, and must equal the finite difference taken
    # around S0 = 0
    gate_mode = oracle.GATE_DIAG
    q, k, v, la, _, Wo, WS = _inputs(3, gate_mode, False)
    g = oracle.backward(q, k, v, Wo, gate_mode=gate_mode, log_alpha=la, dS_final=WS)
    S0 = np.zeros((B, H, DK, DV))
    num = _fd(lambda: _loss(q, k, v, la, S0, Wo, WS, gate_mode, None, oracle.PHI_IDENTITY), S0)
    assert np.max(np.abs(g["dS0"] - num)) < 1e-6 * max(1.0, np.max(np.abs(num)))


def test_ungated_gradients_equal_the_masked_matmul_textbook_form():
    # out = (Q K^T * tril) V + Q S0 and S_final = S0 + K^T V, so for the
    # loss sum(dO * out) + sum(W * S_final):
    #   dV = (Q K^T * tril)^T dO + K W,   dQ = ((dO V^T) * tril) K,
    #   dK = ((dO V^T) * tril)^T Q + V W^T,   dS0 = Q^T dO + W
    r = np.random.default_rng(11)
    Lx, dk, dv = 9, 4, 3
    Q, K, V = r.standard_normal((Lx, dk)), r.standard_normal((Lx, dk)), r.standard_normal((Lx, dv))
    dO, W = r.standard_normal((Lx, dv)), r.standard_normal((dk, dv))
    M = np.tril(np.ones((Lx, Lx)))
    A = (Q @ K.T) * M
    dA = (dO @ V.T) * M
    g = oracle.backward(Q, K, V, dO, dS_final=W)
    np.testing.assert_allclose(g["dv"], A.T @ dO + K @ W, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dq"], dA @ K, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dk"], dA.T @ Q + V @ W.T, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dS0"], Q.T @ dO + W, rtol=1e-12, atol=1e-12)


def test_checkpoint_spacing_does_not_change_the_result():
    r = np.random.default_rng(5)
    Lx = 150
    q, k = r.standard_normal((2, 1, 2, Lx, 4))
    v, do = r.standard_normal((2, 1, 2, Lx, 3))
    la = -np.abs(r.standard_normal((1, 2, Lx, 4))) * 0.1
    S0, W = r.standard_normal((2, 1, 2, 4, 3))
    ref = oracle.backward(q, k, v, do, gate_mode=oracle.GATE_DIAG, log_alpha=la, S0=S0,
                          dS_final=W, checkpoint=1000)
    for ck in (1, 7, 64):
        got = oracle.backward(q, k, v, do, gate_mode=oracle.GATE_DIAG, log_alpha=la, S0=S0,
                              dS_final=W, checkpoint=ck)
        for name in ("dq", "dk", "dv", "dlog_alpha", "dS0"):
            np.testing.assert_array_equal(got[name], ref[name])


@pytest.mark.parametrize("mutation", sorted(m for m in oracle.MUTATIONS if m.startswith("bwd_")))
def test_planted_backward_mistakes_are_caught(mutation):
    case = (oracle.GATE_DIAG, None, oracle.PHI_IDENTITY, True, True)
    with oracle.mutation(mutation):
        with pytest.raises(AssertionError):
            _check_fd(case)
