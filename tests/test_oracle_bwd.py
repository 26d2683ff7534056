"""Pins for the float64 backward oracle (CPU only).

Each check ties the oracle to something other than itself:
  * finite differences of a brute-force forward evaluated at 60 digits
    (mpmath), i.e. the definition of the derivative;
  * torch autograd of torch's own attention routine, in float64;
  * closed forms: identical keys give dQ = 0 and dV_c = mean_r dO_r;
    identical value rows give dQ = dK = 0; dO = 0 gives zero gradients;
  * identities of the chain rule: the gradient of sum(O * dO) summed over
    all keys of dK is 0 (rows of dS sum to 0); adding a constant vector w
    to every key (K + 1 w^T) leaves dQ, dK and dV unchanged;
  * the method's rendering from the forward's O and L ([FS] STAGE 5)
    equals the plain one.
"""
import mpmath
import numpy as np
import pytest
import torch

import oracle


def _inputs(n, m, d, dv=None, seed=0):
    rng = np.random.default_rng(seed)
    dv = d if dv is None else dv
    return (rng.standard_normal((n, d)), rng.standard_normal((m, d)),
            rng.standard_normal((m, dv)), rng.standard_normal((n, dv)))


def _loss_mp(Q, K, V, G, scale):
    """sum_r sum_j O[r,j] G[r,j] with O written out term by term (no max shift)."""
    n, d = len(Q), len(Q[0])
    m = len(K)
    total = mpmath.mpf(0)
    for r in range(n):
        s = [scale * mpmath.fsum(Q[r][t] * K[c][t] for t in range(d)) for c in range(m)]
        e = [mpmath.exp(x) for x in s]
        z = mpmath.fsum(e)
        for j in range(len(V[0])):
            total += mpmath.fsum(e[c] * V[c][j] for c in range(m)) / z * G[r][j]
    return total


@pytest.mark.parametrize("n,m,d,dv", [(3, 4, 2, 2), (2, 5, 3, 1), (1, 1, 2, 2), (4, 2, 1, 3)])
def test_finite_differences_60_digits(n, m, d, dv):
    mpmath.mp.dps = 60
    Q, K, V, G = _inputs(n, m, d, dv, seed=n * 10 + m)
    scale = 0.7
    dQ, dK, dV = oracle.attention_backward(Q, K, V, G, scale)
    h = mpmath.mpf("1e-25")
    mp = lambda A: [[mpmath.mpf(float(x)) for x in row] for row in A]
    base = {"Q": mp(Q), "K": mp(K), "V": mp(V)}
    for name, grad in (("Q", dQ), ("K", dK), ("V", dV)):
        for i in range(grad.shape[0]):
            for j in range(grad.shape[1]):
                plus = {k: [row[:] for row in v] for k, v in base.items()}
                minus = {k: [row[:] for row in v] for k, v in base.items()}
                plus[name][i][j] += h
                minus[name][i][j] -= h
                fd = (_loss_mp(plus["Q"], plus["K"], plus["V"], mp(G), scale)
                      - _loss_mp(minus["Q"], minus["K"], minus["V"], mp(G), scale)) / (2 * h)
                assert abs(float(fd) - grad[i, j]) < 1e-12, (name, i, j, float(fd), grad[i, j])


@pytest.mark.parametrize("n,m,d,dv,scale", [(37, 29, 8, 8, 0.3), (64, 64, 16, 16, 0.25),
                                            (5, 130, 4, 7, 1.0), (1, 1, 3, 3, 0.5)])
def test_torch_autograd_float64(n, m, d, dv, scale):
    Q, K, V, G = _inputs(n, m, d, dv, seed=m)
    dQ, dK, dV = oracle.attention_backward(Q, K, V, G, scale)
    q, k, v = (torch.tensor(x, requires_grad=True) for x in (Q, K, V))
    o = torch.nn.functional.scaled_dot_product_attention(q[None], k[None], v[None], scale=scale)[0]
    o.backward(torch.tensor(G))
    for got, want in ((dQ, q.grad), (dK, k.grad), (dV, v.grad)):
        np.testing.assert_allclose(got, want.numpy(), rtol=0, atol=1e-12)


def test_identical_keys_closed_form():
    Q, K, V, G = _inputs(9, 6, 4, seed=3)
    K[:] = K[0]
    dQ, dK, dV = oracle.attention_backward(Q, K, V, G, 0.5)
    np.testing.assert_allclose(dQ, 0.0, atol=1e-13)
    # uniform weights 1/m: dV_c = sum_r dO_r / m for every key c
    np.testing.assert_allclose(dV, np.broadcast_to(G.sum(axis=0) / K.shape[0], dV.shape), atol=1e-13)


def test_identical_values_closed_form():
    Q, K, V, G = _inputs(7, 11, 5, seed=4)
    V[:] = V[0]
    dQ, dK, dV = oracle.attention_backward(Q, K, V, G, 0.4)
    np.testing.assert_allclose(dQ, 0.0, atol=1e-13)
    np.testing.assert_allclose(dK, 0.0, atol=1e-13)
    O, _ = oracle.attention_naive(Q, K, V, 0.4)
    W = oracle.scores_to_weights(0.4 * Q @ K.T)[0]
    np.testing.assert_allclose(dV, W.T @ G, atol=1e-13)


def test_zero_upstream_gives_zero():
    Q, K, V, G = _inputs(6, 6, 3, seed=5)
    for g in oracle.attention_backward(Q, K, V, np.zeros_like(G), 1.0):
        assert np.all(g == 0.0)


def test_dk_sums_to_zero_over_keys():
    Q, K, V, G = _inputs(33, 47, 6, seed=6)
    _, dK, _ = oracle.attention_backward(Q, K, V, G, 0.8)
    np.testing.assert_allclose(dK.sum(axis=0), 0.0, atol=1e-12)


def test_key_shift_invariance():
    Q, K, V, G = _inputs(21, 17, 5, seed=7)
    w = np.random.default_rng(8).standard_normal(5)
    a = oracle.attention_backward(Q, K, V, G, 0.6)
    b = oracle.attention_backward(Q, K + w[None, :], V, G, 0.6)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, atol=1e-12)


def test_lse_rendering_equals_plain():
    Q, K, V, G = _inputs(1100, 300, 8, seed=9)   # more than one row chunk
    O, L = oracle.attention_naive(Q, K, V, 0.35)
    a = oracle.attention_backward(Q, K, V, G, 0.35)
    b = oracle.attention_backward_lse(Q, K, V, O, G, L, 0.35)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, atol=1e-12)


def test_row_dot_is_rowsum_of_p_times_dp():
    Q, K, V, G = _inputs(12, 10, 4, seed=10)
    O, _ = oracle.attention_naive(Q, K, V, 0.9)
    P = oracle.scores_to_weights(0.9 * Q @ K.T)[0]
    np.testing.assert_allclose(oracle.row_dot(G, O), np.sum(P * (G @ V.T), axis=1), atol=1e-13)


def test_dense_wrapper_matches_heads():
    rng = np.random.default_rng(11)
    q, k, v, g = (rng.standard_normal((2, 3, 19, 4)) for _ in range(4))
    dq, dk, dv = oracle.attention_backward_dense(q, k, v, g, 0.5)
    a = oracle.attention_backward(q[1, 2], k[1, 2], v[1, 2], g[1, 2], 0.5)
    for x, y in zip((dq[1, 2], dk[1, 2], dv[1, 2]), a):
        np.testing.assert_array_equal(x, y)


def test_lse_dense_wrapper_matches_plain_from_exact_forward():
    rng = np.random.default_rng(12)
    q, k, v, g = (rng.standard_normal((2, 2, 23, 8)) for _ in range(4))
    o = np.empty_like(q)
    lse = np.empty(q.shape[:3])
    for b in range(2):
        for h in range(2):
            o[b, h], lse[b, h] = oracle.attention_naive(q[b, h], k[b, h], v[b, h], 0.4)
    a = oracle.attention_backward_lse_dense(q, k, v, o, g, lse, 0.4)
    e = oracle.attention_backward_dense(q, k, v, g, 0.4)
    for x, y in zip(a, e):
        np.testing.assert_allclose(x, y, atol=1e-12)


def test_lse_rendering_uses_the_given_o_and_l():
    # D_r = sum_j dO[r,j] O[r,j] comes from the O it is given: moving O[r,j]
    # by delta moves D_r by delta*dO[r,j], so dS[r,:] = P[r,:](dP[r,:] - D_r)
    # moves by -P[r,:] delta dO[r,j] and dQ[r] by -scale delta dO[r,j] (P K)[r];
    # dV = P^T dO does not move. Raising L_r by eps scales row r of P by
    # exp(-eps), so dV moves by (exp(-eps) - 1) P[r,:]^T dO[r].
    Q, K, V, G = _inputs(9, 13, 6, seed=13)
    scale, r, j, delta, eps = 0.7, 4, 2, 0.01, 0.05
    O, L = oracle.attention_naive(Q, K, V, scale)
    base = oracle.attention_backward_lse(Q, K, V, O, G, L, scale)
    O2 = O.copy()
    O2[r, j] += delta
    moved = oracle.attention_backward_lse(Q, K, V, O2, G, L, scale)
    P = oracle.scores_to_weights(scale * Q @ K.T)[0]
    want_dq = base[0].copy()
    want_dq[r] -= scale * delta * G[r, j] * (P[r] @ K)
    np.testing.assert_allclose(moved[0], want_dq, atol=1e-12)
    np.testing.assert_allclose(moved[2], base[2], atol=1e-13)
    L2 = L.copy()
    L2[r] += eps
    shifted = oracle.attention_backward_lse(Q, K, V, O, G, L2, scale)
    np.testing.assert_allclose(shifted[2] - base[2], np.outer(P[r], G[r]) * (np.exp(-eps) - 1),
                               atol=1e-12)
