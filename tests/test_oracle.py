"""Pins for the float64 oracle (CPU only).

Each pin ties the oracle to something other than itself: brute force at
50 significant digits through a different formula (log-sum-exp without a
max shift), a library attention routine, scipy's logsumexp and softmax,
closed forms (constant V, identical keys, a single key, shift
invariance), the pages' worked example and self-checks, and the
equivalence of the tiled online algorithm with the definition.
"""
import math
import os

import mpmath
import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import attention_f64 as of

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
mpmath.mp.dps = 50


# ---------------------------------------------------------------------------
# Brute force: pure-Python loops, mpmath at 50 digits, no max shift.
# O[r] = sum_c exp(s_rc - LSE_r) v_c with LSE_r = ln sum_c exp(s_rc).
# ---------------------------------------------------------------------------
def brute_force(Q, K, V, scale):
    Q, K, V = (np.asarray(x, dtype=np.float64) for x in (Q, K, V))
    n, d = Q.shape
    m, dv = V.shape
    sc = mpmath.mpf(scale)
    O = np.zeros((n, dv))
    L = np.zeros(n)
    for r in range(n):
        s = [sc * mpmath.fsum(mpmath.mpf(Q[r, t]) * mpmath.mpf(K[c, t]) for t in range(d))
             for c in range(m)]
        lse = mpmath.log(mpmath.fsum(mpmath.exp(x) for x in s))
        L[r] = float(lse)
        for j in range(dv):
            O[r, j] = float(mpmath.fsum(mpmath.exp(s[c] - lse) * mpmath.mpf(V[c, j])
                                        for c in range(m)))
    return O, L


@pytest.mark.parametrize("n,m,d", [(1, 1, 1), (1, 3, 2), (2, 2, 1), (3, 5, 4), (5, 8, 2),
                                   (8, 3, 4), (8, 8, 4)])
def test_brute_force_tiny(n, m, d):
    rng = np.random.default_rng(100 + 10 * n + m)
    Q = rng.standard_normal((n, d))
    K = rng.standard_normal((m, d))
    V = rng.standard_normal((m, d + 1))  # dv != d catches a transposed V
    scale = 0.7
    O, L = oracle.attention_naive(Q, K, V, scale)
    Ob, Lb = brute_force(Q, K, V, scale)
    assert np.max(np.abs(O - Ob)) <= 1e-13
    assert np.max(np.abs(L - Lb)) <= 1e-13


def test_brute_force_large_scores():
    # Scores of several hundred: an unshifted float64 exp would still be
    # finite here, but the brute force needs no shift at all.
    rng = np.random.default_rng(7)
    Q = 12.0 * rng.standard_normal((4, 4))
    K = 12.0 * rng.standard_normal((6, 4))
    V = rng.uniform(-1, 1, (6, 3))
    O, L = oracle.attention_naive(Q, K, V, 1.0)
    Ob, Lb = brute_force(Q, K, V, 1.0)
    assert np.max(np.abs(O - Ob)) <= 1e-12
    assert np.max(np.abs(L - Lb)) <= 1e-12 * max(1.0, np.max(np.abs(Lb)))


def test_single_key_closed_form():
    # One key: every weight is 1, O = V[0], L = scale * q.k.
    rng = np.random.default_rng(3)
    Q = rng.standard_normal((5, 6))
    K = rng.standard_normal((1, 6))
    V = rng.standard_normal((1, 6))
    O, L = oracle.attention_naive(Q, K, V, 0.3)
    assert np.array_equal(O, np.repeat(V, 5, axis=0))
    assert np.allclose(L, 0.3 * (Q @ K[0]), atol=1e-14, rtol=0)


# ---------------------------------------------------------------------------
# Library routines computing the same function.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n,m,d,scale", [(16, 16, 8, 0.125), (33, 70, 64, 0.125),
                                         (130, 67, 128, 1 / math.sqrt(128)), (7, 300, 16, 1.0)])
def test_matches_library_attention(n, m, d, scale):
    rng = np.random.default_rng(n * 1000 + m)
    Q = rng.standard_normal((n, d))
    K = rng.standard_normal((m, d))
    V = rng.standard_normal((m, d))
    O, L = oracle.attention_naive(Q, K, V, scale)
    t = lambda a: torch.from_numpy(a)[None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(t(Q), t(K), t(V), scale=scale)
    assert np.max(np.abs(O - ref[0, 0].numpy())) <= 1e-12
    # L against scipy's logsumexp of the explicit score matrix.
    S = scale * np.einsum("rk,ck->rc", Q, K)
    assert np.max(np.abs(L - scipy.special.logsumexp(S, axis=1))) <= 1e-12


def test_weights_are_softmax_rows():
    # V = identity makes O the weight matrix itself: each row must be the
    # library softmax of the scaled scores, non-negative, summing to 1.
    rng = np.random.default_rng(11)
    m = 40
    Q = rng.standard_normal((25, 16))
    K = rng.standard_normal((m, 16))
    O, _ = oracle.attention_naive(Q, K, np.eye(m), 0.4)
    W = scipy.special.softmax(0.4 * np.einsum("rk,ck->rc", Q, K), axis=1)
    assert np.max(np.abs(O - W)) <= 1e-14
    assert np.all(O >= 0)
    assert np.max(np.abs(O.sum(axis=1) - 1.0)) <= 1e-13


# ---------------------------------------------------------------------------
# Closed forms.
# ---------------------------------------------------------------------------
def test_constant_v_gives_that_row():
    rng = np.random.default_rng(5)
    Q = 3 * rng.standard_normal((50, 32))
    K = 3 * rng.standard_normal((77, 32))
    v = rng.standard_normal(32)
    O, _ = oracle.attention_naive(Q, K, np.tile(v, (77, 1)), 0.5)
    assert np.max(np.abs(O - v)) <= 1e-13


def test_identical_keys_give_mean_of_v():
    rng = np.random.default_rng(6)
    m = 37
    Q = rng.standard_normal((20, 16))
    k = rng.standard_normal(16)
    V = rng.standard_normal((m, 16))
    O, L = oracle.attention_naive(Q, np.tile(k, (m, 1)), V, 0.25)
    assert np.max(np.abs(O - V.mean(axis=0))) <= 1e-13
    assert np.max(np.abs(L - (0.25 * Q @ k + math.log(m)))) <= 1e-13


def test_shift_invariance_explicit_scores():
    # [FS] STAGE 1: subtracting (or adding) a constant cancels in the ratio.
    rng = np.random.default_rng(8)
    S = rng.standard_normal((6, 30))
    W0, L0 = oracle.scores_to_weights(S)
    W1, L1 = oracle.scores_to_weights(S + 1000.0)
    assert np.max(np.abs(W0 - W1)) <= 1e-13
    assert np.max(np.abs(L1 - L0 - 1000.0)) <= 1e-10


def test_shift_invariance_through_keys():
    # K' = K + 1 w^T adds scale*(q.w) to every score of row q: O unchanged,
    # L shifted by exactly that amount.
    rng = np.random.default_rng(9)
    Q = rng.standard_normal((12, 8))
    K = rng.standard_normal((20, 8))
    V = rng.standard_normal((20, 8))
    w = 5 * rng.standard_normal(8)
    O0, L0 = oracle.attention_naive(Q, K, V, 0.6)
    O1, L1 = oracle.attention_naive(Q, K + w, V, 0.6)
    assert np.max(np.abs(O0 - O1)) <= 1e-12
    assert np.max(np.abs((L1 - L0) - 0.6 * Q @ w)) <= 1e-11


# ---------------------------------------------------------------------------
# The pages' worked example and self-checks.
# ---------------------------------------------------------------------------
def _golden_scores():
    rows = [ln for ln in open(os.path.join(GOLDEN, "overflow_scores.txt"))
            if ln.strip() and not ln.startswith("#")]
    return np.array([float(x) for x in rows[0].split()])


def test_overflow_worked_example():
    # [FS] DEMO 9: scores 800, 810, 805, 790. Without the max shift exp()
    # overflows; with it the weights are exp(s - 810) / sum, in closed form.
    s = _golden_scores()
    with np.errstate(all="ignore"):
        unshifted = np.exp(s)                  # every term overflows
        ratio = unshifted / unshifted.sum()    # inf / inf
    assert np.isinf(unshifted).all() and np.isnan(ratio).all()
    W, L = oracle.scores_to_weights(s)
    ms = [mpmath.mpf(x) for x in s]
    z = mpmath.fsum(mpmath.exp(x - 810) for x in ms)
    expect = [float(mpmath.exp(x - 810) / z) for x in ms]
    assert np.max(np.abs(W[0] - expect)) <= 1e-15
    assert abs(L[0] - float(810 + mpmath.log(z))) <= 1e-12
    # The same row through the attention oracle: one query q = e0, keys
    # k_c = s_c e0 (scale 1), V = identity, so O's row is the weights.
    Q = np.zeros((1, 4)); Q[0, 0] = 1.0
    K = np.zeros((4, 4)); K[:, 0] = s
    O, La = oracle.attention_naive(Q, K, np.eye(4), 1.0)
    assert np.max(np.abs(O[0] - expect)) <= 1e-15
    assert abs(La[0] - L[0]) <= 1e-12


def test_online_softmax_demo():
    # [FS] DEMO 2: 32 scores ~ N(0, 3) streamed in 4 blocks of 8.
    row = np.random.default_rng(1).normal(0, 3, 32)
    ref = scipy.special.softmax(row)
    good = oracle.streamed_softmax(row, width=8, align=True)
    bad = oracle.streamed_softmax(row, width=8, align=False)
    assert np.max(np.abs(good - ref)) <= 1e-15
    assert np.max(np.abs(oracle.softmax(row) - ref)) <= 1e-15
    assert abs(bad.sum() - 1.0) > 1e-3          # the page: "not 1.0"
    assert np.max(np.abs(bad - ref)) > 1e-3


def _unit_scaled_inputs(n, d, seed):
    # Inputs of the [FS] DEMO 6 kind: queries and keys with entries of
    # variance 1/d (so scores have unit variance), values with unit variance.
    g = np.random.default_rng(seed)
    q = g.standard_normal((n, d)) * d ** -0.5
    k = g.standard_normal((n, d)) * d ** -0.5
    v = g.standard_normal((n, d))
    return q, k, v


def test_exactness_demo():
    # [FS] DEMO 6: the tiled method agrees with the definition to 1e-10
    # (n=512, d=64, tiles of 64); restricting every row to a +-64 window of
    # keys is a different function and must not agree.
    Q, K, V = _unit_scaled_inputs(512, 64, 5)
    ref, _ = oracle.attention_naive(Q, K, V, 1.0)
    flash, _ = oracle.blocked_attention(Q, K, V, 1.0, q_width=64, k_width=64)
    assert np.allclose(ref, flash, atol=1e-10)
    pos = np.arange(512)
    window = np.abs(pos[:, None] - pos[None, :]) <= 64
    S = np.where(window, Q @ K.T, -np.inf)
    local = oracle.softmax(S) @ V
    assert not np.allclose(ref, local, atol=1e-10)


# ---------------------------------------------------------------------------
# O2 (tiled online, independent code) against O1 for any tile sizes.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("Br,Bc", [(1, 1), (3, 7), (7, 3), (16, 64), (64, 16), (100, 100),
                                   (93, 93), (98, 98), (64, 1)])
def test_tiled_equals_definition(Br, Bc):
    rng = np.random.default_rng(Br * 131 + Bc)
    n, m, d = 93, 93, 16
    Q = 2 * rng.standard_normal((n, d))
    K = 2 * rng.standard_normal((m, d))
    V = rng.standard_normal((m, d))
    O1, L1 = oracle.attention_naive(Q, K, V, 0.5)
    O2, L2 = oracle.blocked_attention(Q, K, V, 0.5, q_width=Br, k_width=Bc)
    assert np.max(np.abs(O1 - O2)) <= 1e-12
    assert np.max(np.abs(L1 - L2)) <= 1e-12


def _ascending_problem():
    # Scores that rise along the keys: the row max moves on every tile, so
    # a missing rescale cannot go unnoticed.
    n, m, d = 8, 64, 4
    Q = np.ones((n, d))
    K = np.outer(np.linspace(-3, 3, m), np.ones(d))
    V = np.random.default_rng(2).standard_normal((m, d))
    return Q, K, V


@pytest.mark.parametrize("mutation", [dict(align=False), dict(align_values=False)])
def test_mutation_teeth(mutation):
    Q, K, V = _ascending_problem()
    O1, L1 = oracle.attention_naive(Q, K, V, 1.0)
    O2, L2 = oracle.blocked_attention(Q, K, V, 1.0, q_width=4, k_width=8, **mutation)
    assert np.max(np.abs(O1 - O2)) > 1e-3 or np.max(np.abs(L1 - L2)) > 1e-3


# ---------------------------------------------------------------------------
# Drivers: dense rows and varlen packing.
# ---------------------------------------------------------------------------
def test_dense_rows_match_full():
    rng = np.random.default_rng(12)
    q = rng.standard_normal((2, 3, 40, 8))
    k = rng.standard_normal((2, 3, 40, 8))
    v = rng.standard_normal((2, 3, 40, 8))
    O, L = oracle.attention_dense(q, k, v, 0.35)
    rows = np.array([0, 5, 39])
    Or, Lr = oracle.attention_dense_rows(q, k, v, 0.35, 1, 2, rows)
    assert np.array_equal(Or, O[1, 2, rows]) and np.array_equal(Lr, L[1, 2, rows])
    # each (b, h) is its own problem
    Ob, Lb = brute_force(q[1, 2, :3], k[1, 2], v[1, 2], 0.35)
    assert np.max(np.abs(O[1, 2, :3] - Ob)) <= 1e-13
    assert np.max(np.abs(L[1, 2, :3] - Lb)) <= 1e-13


def test_varlen_brute_force_and_isolation():
    # Three sequences of lengths 1, 2, 5 packed as [T, H, d]: each attends
    # to its own tokens only.
    rng = np.random.default_rng(13)
    lengths = [1, 2, 5]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    T, H, d = int(cu[-1]), 2, 4
    q = rng.standard_normal((T, H, d))
    k = rng.standard_normal((T, H, d))
    v = rng.standard_normal((T, H, d))
    O, L = oracle.attention_varlen(q, k, v, cu, 0.9)
    for s in range(3):
        a, e = cu[s], cu[s + 1]
        for h in range(H):
            Ob, Lb = brute_force(q[a:e, h], k[a:e, h], v[a:e, h], 0.9)
            assert np.max(np.abs(O[a:e, h] - Ob)) <= 1e-13
            assert np.max(np.abs(L[h, a:e] - Lb)) <= 1e-13
    # perturbing sequence 2 leaves sequences 0 and 1 untouched
    k2 = k.copy(); k2[cu[2]:] += 3.0 * rng.standard_normal(k2[cu[2]:].shape)
    O2, L2 = oracle.attention_varlen(q, k2, v, cu, 0.9)
    assert np.array_equal(O2[:cu[2]], O[:cu[2]]) and np.array_equal(L2[:, :cu[2]], L[:, :cu[2]])
    assert not np.allclose(O2[cu[2]:], O[cu[2]:])
    Or, Lr = oracle.attention_varlen_rows(q, k, v, cu, 0.9, 2, 1, [0, 4])
    assert np.array_equal(Or, O[[cu[2], cu[2] + 4], 1])
    assert np.array_equal(Lr, L[1, [cu[2], cu[2] + 4]])


def test_torch_inputs_accepted():
    # bf16 tensors are widened exactly to float64 before any arithmetic.
    rng = np.random.default_rng(14)
    q = torch.from_numpy(rng.standard_normal((9, 8)).astype(np.float32)).to(torch.bfloat16)
    k = torch.from_numpy(rng.standard_normal((9, 8)).astype(np.float32)).to(torch.bfloat16)
    v = torch.from_numpy(rng.standard_normal((9, 8)).astype(np.float32)).to(torch.bfloat16)
    O, L = oracle.attention_naive(q, k, v, 0.125)
    Ob, Lb = brute_force(q.double().numpy(), k.double().numpy(), v.double().numpy(), 0.125)
    assert np.max(np.abs(O - Ob)) <= 1e-13 and np.max(np.abs(L - Lb)) <= 1e-13


# ---------------------------------------------------------------------------
# The partial-state combine behind blocked_attention: exact for any split of
# the keys and any combination order, and an empty summary is neutral.
# ---------------------------------------------------------------------------
def test_merge_states_matches_logsumexp_of_union():
    rng = np.random.default_rng(21)
    x = 5 * rng.standard_normal((3, 40))
    v = rng.standard_normal((40, 6))
    for cut in (1, 13, 39):
        a = oracle.block_states(x[:, :cut], v[:cut], width=cut)[0]
        b = oracle.block_states(x[:, cut:], v[cut:], width=40)[0]
        for first, second in ((a, b), (b, a)):
            ref, mass, wsum = oracle.merge_states(first, second)
            assert np.max(np.abs(ref + np.log(mass) - scipy.special.logsumexp(x, axis=1))) <= 1e-13
            assert np.max(np.abs(wsum / mass[:, None] - scipy.special.softmax(x, axis=1) @ v)) <= 1e-13


def test_merge_states_empty_summary_is_neutral():
    rng = np.random.default_rng(22)
    x = rng.standard_normal((2, 9))
    v = rng.standard_normal((9, 3))
    s = oracle.block_states(x, v, width=9)[0]
    empty = (np.full(2, -np.inf), np.zeros(2), np.zeros((2, 3)))
    for got in (oracle.merge_states(s, empty), oracle.merge_states(empty, s)):
        assert np.array_equal(got[0], s[0])
        assert np.max(np.abs(got[1] - s[1])) == 0.0
        assert np.max(np.abs(got[2] - s[2])) == 0.0


@pytest.mark.parametrize("width", [1, 2, 3, 5, 8, 31])
def test_reduce_states_any_width(width):
    rng = np.random.default_rng(width)
    row = 4 * rng.standard_normal(31)
    assert np.max(np.abs(oracle.streamed_softmax(row, width=width) -
                         scipy.special.softmax(row))) <= 1e-15
