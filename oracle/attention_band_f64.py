"""Plain float64 reference for banded (local-window) attention.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import, call or run anything in this
module. The HIP library never routes through it and shares no code with it.

Page this follows (cited by title and section):

* [FS]  "FlashAttention -- for programmers, not researchers", DEMO 6. Next
        to the check that the tiled method equals plain attention, the demo
        builds a local variant as a contrast: every query row may only look
        at the keys whose index lies within 64 of its own (the scores of all
        other keys are replaced by -inf before the row softmax), and the
        result differs from full attention.

What is computed, for one head of self-attention (query r and key c index
the same token axis) and a window w >= 0:

    S[r, c] = scale * dot(Q[r], K[c])     if |r - c| <= w
            = -inf                        otherwise
    m_r = max_c S[r, c]
    P   = exp(S - m)                      (exp(-inf) = 0: masked keys drop out)
    l_r = sum_c P[r, c]
    O   = (P / l) V
    L_r = m_r + ln(l_r)                   (natural log, as in the full forward)

Readings. The demo's scores carry no scale (its inputs are pre-scaled); as
in the full forward the scale sits on the dot product. The demo's 64 is the
window w, and "within" includes the boundary (|r - c| = w is kept). Key c
= r is always kept, so every row r below the key count has a finite
maximum, and l_r >= 1 (the arg-max key contributes exp(0)).

The mask is built from the index difference over all keys of the row, then
applied to the full score row; rows are independent and processed in chunks
(columns are not split). Pins live in ``tests/test_oracle_band.py`` and the
mutation teeth in ``tests/test_oracle_mutations.py``.
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


def attention_banded_rows(Q, K, V, scale: float, window: int, rows=None):
    """Banded attention for the selected query rows of one head.

    Q: (n, d), K: (m, d), V: (m, dv); row r attends to keys c with
    |r - c| <= window. Returns O (len(rows), dv) and L (len(rows),)."""
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    if window < 0:
        raise ValueError("window must be >= 0")
    if rows is None:
        rows = np.arange(Q.shape[0])
    rows = np.asarray(rows, dtype=np.int64)
    keys = np.arange(K.shape[0], dtype=np.int64)
    O = np.empty((rows.size, V.shape[1]), dtype=np.float64)
    L = np.empty((rows.size,), dtype=np.float64)
    for s in range(0, rows.size, ROW_CHUNK):
        sel = rows[s:s + ROW_CHUNK]
        band = np.abs(sel[:, None] - keys[None, :]) <= window   # [FS] DEMO 6's mask
        S = np.where(band, scale * (Q[sel] @ K.T), -np.inf)     # masked scores
        m = S.max(axis=1, keepdims=True)                        # row max (finite: c = r kept)
        P = np.exp(S - m)                                       # exp(-inf) = 0
        l = P.sum(axis=1, keepdims=True)
        O[s:s + sel.size] = (P / l) @ V
        L[s:s + sel.size] = m[:, 0] + np.log(l[:, 0])
    return O, L


def attention_banded(Q, K, V, scale: float, window: int):
    """Banded attention over every row of one head: (O, L)."""
    return attention_banded_rows(Q, K, V, scale, window, None)


def attention_banded_dense(q, k, v, scale: float, window: int):
    """q, k, v: [B, H, N, d]. Returns O [B, H, N, d] and L [B, H, N]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, _ = q.shape
    O = np.empty(q.shape[:3] + (v.shape[3],), dtype=np.float64)
    L = np.empty((B, H, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            O[b, h], L[b, h] = attention_banded(q[b, h], k[b, h], v[b, h], scale, window)
    return O, L


def attention_banded_dense_rows(q, k, v, scale: float, window: int, b: int, h: int, rows):
    """Selected rows of one (batch, head) of a dense banded problem."""
    return attention_banded_rows(_f64(q[b, h]), _f64(k[b, h]), _f64(v[b, h]), scale, window,
                                 rows)
