"""Plain float64 reference for the FlashAttention-2 forward.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import, call or run anything in this
package. The HIP library never routes through it, and the two share no
code: no kernels, helpers, tables or constants.

Pages this follows (cited by title and section):

* [KV]  "Kernel visualization: Flash Attention 2" (tinyvolt.com): the FA2
        forward kernel, its sections "Steps", "Visualizing operations in a
        single block", "Iteration j = 0/1", "Write the data back to HBM",
        "Counting trips across HBM".
* [FS]  "FlashAttention -- for programmers, not researchers"
        (flash_attention_from_scratch.py, paperfordummies.in): STAGE 1
        (softmax), STAGE 2 (standard attention), STAGE 3 (online softmax),
        STAGE 4 (FlashAttention), DEMO 2, 3, 6, 9.

What the method computes. The pages state that the tiled method is the
same function as plain attention, not an approximation ([FS] STAGE 4 and
DEMO 6). So the oracle ``attention_naive`` is that plain definition,
written out in float64 on the dtype-rounded inputs:

    S   = scale * Q K^T              (the scale sits on the dot product, as
                                      in the [KV] score step)
    m_r = max_c S[r, c]
    P   = exp(S - m)                 (max shift: [FS] STAGE 1)
    l_r = sum_c P[r, c]
    O   = (P / l) V                  ([FS] STAGE 2)
    L_r = m_r + ln(l_r)              (natural log, [KV] "Write the data back
                                      to HBM": L = m + log(l))

Every row uses ALL keys; rows may be processed in chunks because rows are
independent ([KV] "Same operations in another block"), columns may not
(that would be the online method under test).

``attention_tiled`` is a second, independent float64 rendering of the
tiled online algorithm of [FS] STAGE 4 (plus the scale and L of [KV]); it
exists so the pins can check the oracle against the pages' own
equivalence claim, and so a planted mistake (no rescale) can be shown to
fail. It is not used to judge the GPU path.

Parity pins for every function here live in ``tests/test_oracle.py``
(brute force at 50 digits, a library attention routine, scipy's
logsumexp, closed forms for constant V and identical keys, shift
invariance, the [FS] DEMO 9 worked example, the mutation teeth).
"""
from __future__ import annotations

import numpy as np

ROW_CHUNK = 1024


def _f64(x) -> np.ndarray:
    """Accept numpy arrays or CPU torch tensors; return float64 numpy."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        import torch  # only for dtype conversion of torch inputs
        x = x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
# [FS] STAGE 1: softmax with the max subtracted for overflow safety.
# ---------------------------------------------------------------------------
def softmax(x, axis: int = -1) -> np.ndarray:
    z = _f64(x)
    z = z - z.max(axis=axis, keepdims=True)   # largest entry becomes 0
    w = np.exp(z)
    return w / w.sum(axis=axis, keepdims=True)


def scores_to_weights(S):
    """Softmax weights and natural-log normaliser of an explicit score
    matrix (rows = queries): returns (W, L) with L = max + ln(sum exp(S - max))."""
    S = _f64(S)
    if S.ndim == 1:
        S = S[None, :]
    m = np.max(S, axis=-1, keepdims=True)
    p = np.exp(S - m)
    l = np.sum(p, axis=-1, keepdims=True)
    return p / l, (m + np.log(l))[:, 0]


# ---------------------------------------------------------------------------
# [FS] STAGE 3: online softmax over one row seen a block at a time.
# The running max m and running sum l are carried; when a block raises the
# max, the old sum is brought to the new baseline by exp(m_old - m_new).
# ---------------------------------------------------------------------------
def online_softmax(row, block: int = 8, rescale: bool = True) -> np.ndarray:
    x = _f64(row).reshape(-1)
    ref, total = -np.inf, 0.0          # running max, sum of exp(x - ref)
    for b in range(0, x.size, block):
        part = x[b:b + block]
        top = max(ref, float(part.max()))
        carry = float(np.exp(ref - top)) if (rescale and np.isfinite(ref)) else 1.0
        total = total * carry + float(np.exp(part - top).sum())
        ref = top
    return np.exp(x - ref) / total


# ---------------------------------------------------------------------------
# O1: the definition, one head.
# ---------------------------------------------------------------------------
def attention_naive_rows(Q, K, V, scale: float, rows=None):
    """Plain attention for the selected query rows of one head.

    Q: (n, d), K: (m, d), V: (m, dv). Returns O (len(rows), dv) and
    L (len(rows),). Each row is softmax(scale * q K^T) V over all m keys."""
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    if rows is None:
        rows = np.arange(Q.shape[0])
    rows = np.asarray(rows, dtype=np.int64)
    O = np.empty((rows.size, V.shape[1]), dtype=np.float64)
    L = np.empty((rows.size,), dtype=np.float64)
    for s in range(0, rows.size, ROW_CHUNK):
        sel = rows[s:s + ROW_CHUNK]
        S = scale * (Q[sel] @ K.T)                 # scores, every key
        m = S.max(axis=1, keepdims=True)           # row max
        P = np.exp(S - m)                          # shifted exponentials
        l = P.sum(axis=1, keepdims=True)           # row normaliser
        O[s:s + sel.size] = (P / l) @ V            # softmax(S) V
        L[s:s + sel.size] = m[:, 0] + np.log(l[:, 0])
    return O, L


def attention_naive(Q, K, V, scale: float):
    """Plain attention over every row of one head: (O, L)."""
    return attention_naive_rows(Q, K, V, scale, None)


# ---------------------------------------------------------------------------
# Dense [B, H, N, d] and packed varlen [T, H, d] drivers around O1.
# ---------------------------------------------------------------------------
def attention_dense(q, k, v, scale: float):
    """q, k, v: [B, H, N, d]. Returns O [B, H, N, d] and L [B, H, N]
    (the [KV] kernel's L is one row of N values per (batch, head))."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, _ = q.shape
    O = np.empty(q.shape[:3] + (v.shape[3],), dtype=np.float64)
    L = np.empty((B, H, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            O[b, h], L[b, h] = attention_naive(q[b, h], k[b, h], v[b, h], scale)
    return O, L


def attention_dense_rows(q, k, v, scale: float, b: int, h: int, rows):
    """Selected rows of one (batch, head) of a dense [B, H, N, d] problem."""
    return attention_naive_rows(_f64(q[b, h]), _f64(k[b, h]), _f64(v[b, h]), scale, rows)


def attention_varlen(q, k, v, cu_seqlens, scale: float):
    """Packed self-attention: sequence s owns tokens cu[s]..cu[s+1]-1 of the
    [T, H, d] tensors and attends to its own tokens only (no causal mask).
    Returns O [T, H, d] and L [H, T]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    cu = np.asarray(_f64(cu_seqlens), dtype=np.int64)
    T, H, _ = q.shape
    O = np.zeros((T, H, v.shape[2]), dtype=np.float64)
    L = np.zeros((H, T), dtype=np.float64)
    for s in range(cu.size - 1):
        a, e = int(cu[s]), int(cu[s + 1])
        if e <= a:
            continue
        for h in range(H):
            O[a:e, h], L[h, a:e] = attention_naive(q[a:e, h], k[a:e, h], v[a:e, h], scale)
    return O, L


def attention_varlen_rows(q, k, v, cu_seqlens, scale: float, seq: int, h: int, rows):
    """Selected rows (local to sequence `seq`) of one head of a varlen problem."""
    cu = np.asarray(_f64(cu_seqlens), dtype=np.int64)
    a, e = int(cu[seq]), int(cu[seq + 1])
    return attention_naive_rows(_f64(q[a:e, h]), _f64(k[a:e, h]), _f64(v[a:e, h]), scale, rows)


# ---------------------------------------------------------------------------
# O2: the tiled online algorithm, [FS] STAGE 4 with [KV]'s scale and L.
#
# The query rows are cut into blocks of Br and the keys into blocks of Bc;
# query blocks are the outer loop. For every query row of a block three
# running quantities are kept while the key blocks go by: the largest scaled
# score seen so far (run_max), the sum of exp(score - run_max) (run_sum) and
# the matching unnormalised weighted sum of value rows (acc). A key block
# with a larger score moves run_max; the old run_sum and acc were formed
# against the old maximum, so both are first multiplied by
# exp(old_max - new_max) (0 for a row that has not seen any key). After the
# last key block the row is divided by run_sum once, and its logsumexp is
# run_max + ln(run_sum).
#
# `rescale=False` is [FS]'s planted bug (sums taken against different
# baselines); `rescale_o=False` corrects run_sum but not acc. Both must fail
# the equivalence pins.
# ---------------------------------------------------------------------------
def attention_tiled(Q, K, V, scale: float, Br: int = 64, Bc: int = 64,
                    rescale: bool = True, rescale_o: bool = True):
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    n_q, n_k = Q.shape[0], K.shape[0]
    out = np.empty((n_q, V.shape[1]), dtype=np.float64)
    lse = np.empty((n_q,), dtype=np.float64)
    key_blocks = [(a, min(a + Bc, n_k)) for a in range(0, n_k, Bc)]
    for r0 in range(0, n_q, Br):
        r1 = min(r0 + Br, n_q)
        q_blk = Q[r0:r1]
        run_max = np.full(r1 - r0, -np.inf)
        run_sum = np.zeros(r1 - r0)
        acc = np.zeros((r1 - r0, V.shape[1]))
        for (c0, c1) in key_blocks:
            scores = scale * (q_blk @ K[c0:c1].T)          # (rows, keys) block
            new_max = np.maximum(run_max, scores.max(axis=1))
            w = np.exp(scores - new_max[:, None])           # unnormalised weights
            if rescale:
                fix = np.zeros_like(run_max)
                seen = np.isfinite(run_max)
                fix[seen] = np.exp(run_max[seen] - new_max[seen])
                run_sum = fix * run_sum + w.sum(axis=1)
                acc = (fix[:, None] * acc if rescale_o else acc) + w @ V[c0:c1]
            else:
                run_sum = run_sum + w.sum(axis=1)
                acc = acc + w @ V[c0:c1]
            run_max = new_max
        out[r0:r1] = acc / run_sum[:, None]
        lse[r0:r1] = run_max + np.log(run_sum)
    return out, lse
