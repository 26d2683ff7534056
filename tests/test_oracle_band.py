"""Pins for the float64 banded-attention oracle (CPU only).

Each check ties ``oracle.attention_banded`` to something other than itself:
  * brute force at 60 digits (mpmath) that sums over the in-band keys of
    each row only (no -inf, no max shift);
  * torch's own attention routine in float64 with an explicit boolean mask;
  * special cases: a window covering every key is full attention (the
    already-pinned full oracle); window 0 gives O[r] = V[r] and
    L[r] = scale q_r . k_r; identical keys give the mean of the in-band
    value rows and L = score + ln(band size), which fixes the band's edges;
  * the [FS] DEMO 6 contrast: at n = 512, d = 64 and a window of 64 the
    banded result is a different function from full attention;
  * locality: keys and values outside row r's band do not change row r.
"""
import math

import mpmath
import numpy as np
import pytest
import torch

import oracle


def _inputs(n, d, seed, dv=None):
    rng = np.random.default_rng(seed)
    dv = d if dv is None else dv
    return rng.standard_normal((n, d)), rng.standard_normal((n, d)), rng.standard_normal((n, dv))


def _brute(Q, K, V, scale, w):
    mpmath.mp.dps = 60
    n, d = Q.shape
    O = np.zeros((n, V.shape[1]))
    L = np.zeros(n)
    for r in range(n):
        cs = [c for c in range(K.shape[0]) if abs(r - c) <= w]
        s = {c: mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(Q[r, t]) * mpmath.mpf(K[c, t])
                                                for t in range(d)) for c in cs}
        z = mpmath.fsum(mpmath.exp(s[c]) for c in cs)
        L[r] = float(mpmath.log(z))
        for j in range(V.shape[1]):
            O[r, j] = float(mpmath.fsum(mpmath.exp(s[c]) * mpmath.mpf(V[c, j]) for c in cs) / z)
    return O, L


@pytest.mark.parametrize("n,d,w", [(6, 3, 0), (7, 2, 1), (9, 4, 2), (5, 3, 4), (5, 2, 9), (1, 3, 0)])
def test_brute_force_60_digits(n, d, w):
    Q, K, V = _inputs(n, d, seed=n * 7 + w, dv=d + 1)
    O, L = oracle.attention_banded(Q, K, V, 0.8, w)
    Ob, Lb = _brute(Q, K, V, 0.8, w)
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-13)
    np.testing.assert_allclose(L, Lb, rtol=0, atol=1e-13)


@pytest.mark.parametrize("n,d,w,scale", [(100, 16, 7, 0.25), (257, 8, 64, 0.5), (64, 4, 63, 1.0),
                                         (33, 5, 100, 0.3)])
def test_torch_attention_with_mask(n, d, w, scale):
    Q, K, V = _inputs(n, d, seed=n + w)
    O, L = oracle.attention_banded(Q, K, V, scale, w)
    idx = torch.arange(n)
    allowed = (idx[:, None] - idx[None, :]).abs() <= w      # True = attend
    t = lambda a: torch.from_numpy(a)[None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(t(Q), t(K), t(V), attn_mask=allowed,
                                                           scale=scale)[0, 0]
    np.testing.assert_allclose(O, ref.numpy(), rtol=0, atol=1e-12)
    S = scale * torch.from_numpy(Q) @ torch.from_numpy(K).T
    lse = torch.logsumexp(S.masked_fill(~allowed, float("-inf")), dim=1)
    np.testing.assert_allclose(L, lse.numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("w", [99, 100, 1000])
def test_wide_window_is_full_attention(w):
    Q, K, V = _inputs(100, 8, seed=3)
    O, L = oracle.attention_banded(Q, K, V, 0.4, w)
    Of, Lf = oracle.attention_naive(Q, K, V, 0.4)
    np.testing.assert_allclose(O, Of, rtol=0, atol=1e-13)
    np.testing.assert_allclose(L, Lf, rtol=0, atol=1e-13)


def test_window_98_is_not_full_attention():
    Q, K, V = _inputs(100, 8, seed=3)
    O, _ = oracle.attention_banded(Q, K, V, 0.4, 98)
    Of, _ = oracle.attention_naive(Q, K, V, 0.4)
    # only the first and the last row lose a key (each other's)
    diff = np.abs(O - Of).max(axis=1)
    assert diff[0] > 1e-6 and diff[-1] > 1e-6
    assert np.all(diff[1:-1] == 0.0)


def test_window_zero_closed_form():
    Q, K, V = _inputs(50, 6, seed=4)
    O, L = oracle.attention_banded(Q, K, V, 0.9, 0)
    np.testing.assert_array_equal(O, V)
    np.testing.assert_allclose(L, 0.9 * np.sum(Q * K, axis=1), rtol=0, atol=1e-13)


@pytest.mark.parametrize("n,w", [(40, 0), (40, 3), (40, 17), (40, 39), (7, 64)])
def test_identical_keys_band_mean(n, w):
    Q, K, V = _inputs(n, 5, seed=5 + w)
    k = K[0]
    O, L = oracle.attention_banded(Q, np.tile(k, (n, 1)), V, 0.6, w)
    for r in range(n):
        lo, hi = max(0, r - w), min(n - 1, r + w)
        np.testing.assert_allclose(O[r], V[lo:hi + 1].mean(axis=0), rtol=0, atol=1e-13)
        assert abs(L[r] - (0.6 * Q[r] @ k + math.log(hi - lo + 1))) <= 1e-13


def test_demo6_band_is_a_different_function():
    """[FS] DEMO 6: n = 512, d = 64, inputs scaled by 1/sqrt(d), unscaled scores,
    a window of 64: not allclose to full attention at atol 1e-10."""
    rng = np.random.default_rng(5)
    Q = rng.standard_normal((512, 64)) / 8.0
    K = rng.standard_normal((512, 64)) / 8.0
    V = rng.standard_normal((512, 64))
    Ob, _ = oracle.attention_banded(Q, K, V, 1.0, 64)
    Of, _ = oracle.attention_naive(Q, K, V, 1.0)
    assert not np.allclose(Ob, Of, atol=1e-10)
    assert np.abs(Ob - Of).max() > 1e-2


def test_locality():
    Q, K, V = _inputs(80, 6, seed=6)
    w, r = 5, 40
    O, L = oracle.attention_banded_rows(Q, K, V, 0.5, w, [r])
    rng = np.random.default_rng(7)
    K2, V2 = K.copy(), V.copy()
    outside = np.r_[0:r - w, r + w + 1:80]
    K2[outside] = rng.standard_normal((outside.size, 6)) * 10
    V2[outside] = rng.standard_normal((outside.size, 6)) * 10
    O2, L2 = oracle.attention_banded_rows(Q, K2, V2, 0.5, w, [r])
    np.testing.assert_array_equal(O, O2)
    np.testing.assert_array_equal(L, L2)
    K2[r + w] += 1.0   # the band's last key does matter
    O3, _ = oracle.attention_banded_rows(Q, K2, V2, 0.5, w, [r])
    assert np.abs(O3 - O).max() > 1e-6


def test_rows_and_dense_wrappers():
    rng = np.random.default_rng(8)
    q, k, v = (rng.standard_normal((2, 3, 70, 4)) for _ in range(3))
    O, L = oracle.attention_banded_dense(q, k, v, 0.5, 9)
    Or, Lr = oracle.attention_banded_dense_rows(q, k, v, 0.5, 9, 1, 2, [0, 33, 69])
    np.testing.assert_array_equal(O[1, 2, [0, 33, 69]], Or)
    np.testing.assert_array_equal(L[1, 2, [0, 33, 69]], Lr)
    Oh, Lh = oracle.attention_banded(q[1, 2], k[1, 2], v[1, 2], 0.5, 9)
    np.testing.assert_array_equal(O[1, 2], Oh)


def test_large_scores_stay_finite():
    Q, K, V = _inputs(30, 4, seed=9)
    O, L = oracle.attention_banded(Q * 40, K * 40, V, 1.0, 3)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))
    Ob, Lb = _brute(Q[:8] * 40, K[:8] * 40, V[:8], 1.0, 3)
    O8, L8 = oracle.attention_banded(Q[:8] * 40, K[:8] * 40, V[:8], 1.0, 3)
    np.testing.assert_allclose(O8, Ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L8, Lb, rtol=1e-15, atol=1e-10)


def test_negative_window_rejected():
    Q, K, V = _inputs(4, 2, seed=10)
    with pytest.raises(ValueError):
        oracle.attention_banded(Q, K, V, 1.0, -1)
