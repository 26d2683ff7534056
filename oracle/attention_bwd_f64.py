"""Plain float64 reference for the attention backward pass (dQ, dK, dV).

TEST INFRASTRUCTURE. Only ``tests/`` and the benchmark's ``cpu_baseline`` leg
may import, call or run anything in this module. The HIP library never
routes through it and shares no code with it.

Pages this follows (cited by title and section):

* [FS]  "FlashAttention -- for programmers, not researchers", STAGE 5 (the
        backward pass trade: the score tiles are recomputed from the stored
        row statistics instead of being kept from the forward) and DEMO 5.
* [DS]  flash-attention documentation search results, "Application in
        Backward Pass (5 MMAs)": S = Q K^T, dP = dO V^T, dV = P^T dO,
        dK = dS^T Q, dQ = dS K.
* [KV]  "Kernel visualization: Flash Attention 2", "Write the data back to
        HBM": L = m + log(l) is the statistic kept for the backward.

What is computed. The forward is O = softmax(scale * Q K^T) V, row by row
(the definition the forward oracle writes out). For an upstream gradient
dO of the same shape as O, the backward returns the gradients of
sum(O * dO) with respect to Q, K and V, which the chain rule of that
definition gives in closed form (P = softmax(S) row-wise):

    S  = scale * Q K^T
    dV = P^T dO                      (O = P V)
    dP = dO V^T
    D_r = sum_c P[r,c] dP[r,c] = sum_k dO[r,k] O[r,k]
    dS = P * (dP - D)                (softmax Jacobian, row by row)
    dQ = scale * dS K
    dK = scale * dS^T Q

``attention_backward`` is that definition, with P from a max-shifted row
softmax. ``attention_backward_lse`` is the method's own rendering ([FS]
STAGE 5): it takes the forward's O and L (natural log-sum-exp per row) and
recomputes P = exp(S - L) instead of normalising; pinned equal to the
first. Rows are processed in chunks (rows are independent; dK and dV are
sums over rows and accumulate over the chunks); every row sees all keys.

Parity pins live in ``tests/test_oracle_bwd.py`` (50-digit finite
differences of a brute-force forward, torch autograd in float64, closed
forms for identical keys and identical value rows, the zero column sum of
dK, shift invariance) and ``tests/test_oracle_mutations.py``.
"""
from __future__ import annotations

import numpy as np

ROW_CHUNK = 512


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        import torch  # only for dtype conversion of torch inputs
        x = x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def attention_backward(Q, K, V, dO, scale: float):
    """Gradients (dQ, dK, dV) of sum(O * dO), O = softmax(scale Q K^T) V.

    Q: (n, d), K: (m, d), V: (m, dv), dO: (n, dv)."""
    Q, K, V, dO = _f64(Q), _f64(K), _f64(V), _f64(dO)
    n = Q.shape[0]
    dQ = np.empty_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    for s in range(0, n, ROW_CHUNK):
        rows = slice(s, min(s + ROW_CHUNK, n))
        S = scale * (Q[rows] @ K.T)                    # scores of these rows, all keys
        E = np.exp(S - S.max(axis=1, keepdims=True))
        P = E / E.sum(axis=1, keepdims=True)           # softmax, row by row
        O = P @ V
        dV += P.T @ dO[rows]
        dP = dO[rows] @ V.T
        D = np.sum(dO[rows] * O, axis=1, keepdims=True)
        dS = P * (dP - D)
        dQ[rows] = scale * (dS @ K)
        dK += scale * (dS.T @ Q[rows])
    return dQ, dK, dV


def attention_backward_lse(Q, K, V, O, dO, L, scale: float):
    """The same gradients from the forward's outputs: P = exp(scale Q K^T - L)
    with L the natural-log row normaliser, D = rowsum(dO * O) ([FS] STAGE 5)."""
    Q, K, V, O, dO, L = _f64(Q), _f64(K), _f64(V), _f64(O), _f64(dO), _f64(L)
    n = Q.shape[0]
    dQ = np.empty_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    D_all = np.sum(dO * O, axis=1)
    for s in range(0, n, ROW_CHUNK):
        rows = slice(s, min(s + ROW_CHUNK, n))
        P = np.exp(scale * (Q[rows] @ K.T) - L[rows, None])   # recomputed, not stored
        dV += P.T @ dO[rows]
        dS = P * ((dO[rows] @ V.T) - D_all[rows, None])
        dQ[rows] = scale * (dS @ K)
        dK += scale * (dS.T @ Q[rows])
    return dQ, dK, dV


def attention_backward_dense(q, k, v, do, scale: float):
    """[B, H, N, d] tensors; returns dQ, dK, dV of the same shapes (float64)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, H = q.shape[:2]
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    for b in range(B):
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h] = attention_backward(q[b, h], k[b, h], v[b, h],
                                                              do[b, h], scale)
    return dq, dk, dv


def attention_backward_lse_dense(q, k, v, o, do, lse, scale: float):
    """[B, H, N, d] tensors and L [B, H, N]; the gradients from the given O
    and L, head by head (attention_backward_lse)."""
    q, k, v, o, do, lse = _f64(q), _f64(k), _f64(v), _f64(o), _f64(do), _f64(lse)
    B, H = q.shape[:2]
    dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    for b in range(B):
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h] = attention_backward_lse(
                q[b, h], k[b, h], v[b, h], o[b, h], do[b, h], lse[b, h], scale)
    return dq, dk, dv


def row_dot(dO, O):
    """D_r = sum_k dO[r,k] O[r,k] (float64), any leading shape."""
    return np.sum(_f64(dO) * _f64(O), axis=-1)
