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

``blocked_attention`` is a second, independent float64 route to the same
result: per-key-block softmax summaries combined exactly by the rescale
rule of [FS] STAGE 3-4 and [KV]'s online update. It exists so the pins can
check the oracle against the pages' own equivalence claim, and so a planted
mistake (summaries combined without the rescale) can be shown to fail. It
is not used to judge the GPU path.

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
# Partial softmax states ([FS] STAGE 3; [KV] "Iteration j = 0/1").
#
# The scores of a set of keys, seen against a reference value r, are
# summarised by the triple (r, mass, wsum): mass = sum_c exp(x_c - r) and,
# when values come along, wsum = sum_c exp(x_c - r) v_c. Summaries of two
# disjoint key sets combine exactly once both are expressed against a common
# reference; the larger of the two keeps every exponent <= 0. Re-expressing
# a summary against a new reference multiplies mass and wsum by
# exp(r_old - r_new) -- the rescale step the pages apply whenever the
# running max moves. A summary of no keys has r = -inf and contributes
# nothing (factor 0).
#
# The functions below cut the keys into blocks, summarise every block
# against its own maximum (vectorised), and combine the summaries with a
# balanced pairwise reduction. `align=False` drops the re-expression (the
# pages' planted bug: masses taken against different references are added
# as if they shared one); `align_values=False` re-expresses mass but not
# wsum. Both must fail the equivalence pins.
# ---------------------------------------------------------------------------
def _to_common(ref_a, ref_b):
    """Factors that bring summaries at references ref_a and ref_b to
    max(ref_a, ref_b); an empty summary (reference -inf) gets factor 0."""
    top = np.maximum(ref_a, ref_b)
    with np.errstate(invalid="ignore"):
        fa = np.where(np.isneginf(ref_a), 0.0, np.exp(ref_a - top))
        fb = np.where(np.isneginf(ref_b), 0.0, np.exp(ref_b - top))
    return top, fa, fb


def merge_states(a, b, align: bool = True, align_values: bool = True):
    """Combine two summaries (ref, mass, wsum) of disjoint key sets. ref and
    mass have one entry per query row; wsum has one row of values per query
    row, or is None."""
    ra, ma, wa = a
    rb, mb, wb = b
    top, fa, fb = _to_common(ra, rb)
    if not align:
        fa, fb = np.ones_like(fa), np.ones_like(fb)
    mass = fa * ma + fb * mb
    if wa is None:
        return top, mass, None
    ga, gb = (fa, fb) if align_values else (np.ones_like(fa), np.ones_like(fb))
    return top, mass, ga[:, None] * wa + gb[:, None] * wb


def block_states(scores, values=None, width: int = 64):
    """Summaries of consecutive key blocks of `width` columns of a score
    matrix (rows = queries), each against its own block maximum."""
    x = np.atleast_2d(_f64(scores))
    out = []
    for c0 in range(0, x.shape[1], width):
        blk = x[:, c0:c0 + width]
        ref = blk.max(axis=1)
        with np.errstate(invalid="ignore"):
            e = np.where(np.isneginf(ref)[:, None], 0.0, np.exp(blk - ref[:, None]))
        wsum = None if values is None else e @ values[c0:c0 + width]
        out.append((ref, e.sum(axis=1), wsum))
    return out


def reduce_states(states, align: bool = True, align_values: bool = True):
    """Combine a list of summaries by a balanced pairwise reduction."""
    states = list(states)
    while len(states) > 1:
        nxt = [merge_states(states[i], states[i + 1], align, align_values)
               for i in range(0, len(states) - 1, 2)]
        if len(states) % 2:
            nxt.append(states[-1])
        states = nxt
    return states[0]


def streamed_softmax(row, width: int = 8, align: bool = True) -> np.ndarray:
    """Softmax of one row from blockwise summaries: the row's weights are
    exp(x - ref) / mass of the combined summary."""
    x = _f64(row).reshape(-1)
    ref, mass, _ = reduce_states(block_states(x[None, :], None, width), align)
    return np.exp(x - ref[0]) / mass[0]


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
# O2: blocked attention from partial states ([FS] STAGE 4 with [KV]'s scale
# and L). Query rows are cut into blocks of q_width and keys into blocks of
# k_width; every (query block, key block) pair yields a summary of that key
# block for those rows, the summaries of a query block are combined, and
# the row is normalised once at the end: O = wsum / mass and
# L = ref + ln(mass). The pages reach the same result by carrying the
# summary through the key blocks one at a time; combining them in a tree is
# equally exact, and shares no structure with the GPU kernel.
# ---------------------------------------------------------------------------
def blocked_attention(Q, K, V, scale: float, q_width: int = 64, k_width: int = 64,
                      align: bool = True, align_values: bool = True):
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    n_q = Q.shape[0]
    out = np.empty((n_q, V.shape[1]), dtype=np.float64)
    lse = np.empty((n_q,), dtype=np.float64)
    for r0 in range(0, n_q, q_width):
        rows = slice(r0, min(r0 + q_width, n_q))
        S = scale * (Q[rows] @ K.T)
        ref, mass, wsum = reduce_states(block_states(S, V, k_width), align, align_values)
        out[rows] = wsum / mass[:, None]
        lse[rows] = ref + np.log(mass)
    return out, lse
