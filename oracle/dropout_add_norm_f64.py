"""Plain float64 reference for the fused dropout + residual + LayerNorm / RMSNorm op.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import, call or run anything in this
module. The HIP library never routes through it and shares no code with it.

What the pages give. flash-attention's documentation search results (the
paragraph on its fused dropout / residual / LayerNorm CUDA extension) list
capabilities only:

- dropout, the residual add and LayerNorm fused into one op;
- pre-norm and post-norm use;
- RMSNorm as an alternative to LayerNorm;
- parallel residuals (two branches added into one stream, as in GPT-J,
  GPT-NeoX, PaLM);
- hidden sizes up to 8192 that are multiples of 8.

No formula and no random-number generator are given. The readings taken
here, for one row of `hidden` values (all arithmetic in float64 on the
dtype-rounded inputs):

    d0   = dropout(x0)             keep0[e] ? x0[e] / (1 - p) : 0
    d1   = dropout(x1)             (parallel residual; absent -> 0)
    z    = d0 + d1 + residual      (residual absent -> 0); z is the new
                                   residual stream, returned for pre-norm
    LayerNorm:  mu = mean(z), var = mean((z - mu)^2),
                rstd = 1 / sqrt(var + eps), y = (z - mu) * rstd * gamma + beta
    RMSNorm:    rstd = 1 / sqrt(mean(z^2) + eps), y = z * rstd * gamma (+ beta)
    a second weight set (gamma1, beta1) gives y1 from the same z and
    statistics (one normalised stream feeding two parallel branches).

The dropout decisions come from Philox4x32-10, the counter-based generator of
Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3"
(SC'11): 10 rounds of two 32x32->64-bit products by 0xD2511F53 and
0xCD9E8D57, with the key bumped by the Weyl constants 0x9E3779B9 and
0xBB67AE85 between rounds. Element e = row * hidden + col of branch s
(0 for x0, 1 for x1) uses word e % 4 of the block for counter
(q mod 2^32, q div 2^32, offset mod 2^32, (offset div 2^32 + s) mod 2^32),
q = e div 4, key (seed mod 2^32, seed div 2^32). The element is kept when
that word is >= floor(p * 2^32), an integer decision, so both sides agree
bit for bit. The HIP kernel implements the same generator on its own.

Pins live in ``tests/test_oracle_norm.py`` (the generator's published
known-answer vectors, torch's layer_norm / rms_norm in float64, closed forms)
and ``tests/test_oracle_mutations.py``.
"""
from __future__ import annotations

import numpy as np

_M32 = np.uint64(0xFFFFFFFF)


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        import torch  # only for dtype conversion of torch inputs
        x = x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def philox4x32_10(counter, key):
    """Philox4x32-10 on an array of counters: counter (..., 4) and key (2,)
    of 32-bit words (any integer dtype); returns (..., 4) uint64 words."""
    c = [np.asarray(counter, dtype=np.uint64)[..., i] & _M32 for i in range(4)]
    k0 = np.uint64(int(key[0]) & 0xFFFFFFFF)
    k1 = np.uint64(int(key[1]) & 0xFFFFFFFF)
    m0, m1 = np.uint64(0xD2511F53), np.uint64(0xCD9E8D57)
    w0, w1 = np.uint64(0x9E3779B9), np.uint64(0xBB67AE85)
    for r in range(10):
        p0 = m0 * c[0]          # < 2^64: exact in uint64
        p1 = m1 * c[2]
        c = [((p1 >> np.uint64(32)) ^ c[1] ^ k0) & _M32, p1 & _M32,
             ((p0 >> np.uint64(32)) ^ c[3] ^ k1) & _M32, p0 & _M32]
        k0 = (k0 + w0) & _M32
        k1 = (k1 + w1) & _M32
    return np.stack(c, axis=-1)


def keep_threshold(p) -> int:
    """floor(p * 2^32) for the float32 value of p, 0 <= p < 1."""
    p32 = float(np.float32(p))
    if not 0.0 <= p32 < 1.0:
        raise ValueError("dropout probability must be in [0, 1)")
    return int(np.floor(p32 * 4294967296.0))


def dropout_keep(rows: int, hidden: int, p, seed: int, offset: int, stream: int = 0,
                 row_ids=None):
    """Boolean keep mask [rows, hidden] of one branch; row_ids gives the global
    row index of each of the rows (default 0 .. rows-1)."""
    thr = keep_threshold(p)
    ids = np.arange(rows, dtype=np.uint64) if row_ids is None else np.asarray(row_ids, np.uint64)
    e = (ids[:, None] * np.uint64(hidden) + np.arange(hidden, dtype=np.uint64)[None, :]).reshape(-1)
    q = e // np.uint64(4)
    ctr = np.empty(q.shape + (4,), dtype=np.uint64)
    ctr[:, 0] = q & _M32
    ctr[:, 1] = q >> np.uint64(32)
    ctr[:, 2] = np.uint64(offset & 0xFFFFFFFF)
    ctr[:, 3] = np.uint64((((offset >> 32) & 0xFFFFFFFF) + stream) & 0xFFFFFFFF)
    words = philox4x32_10(ctr, (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF))
    word = words[np.arange(e.size), (e % np.uint64(4)).astype(np.int64)]
    return (word >= np.uint64(thr)).reshape(rows, hidden)


def dropout_add_norm(x0, gamma0, beta0=None, residual=None, x1=None, gamma1=None, beta1=None,
                     p: float = 0.0, seed: int = 0, offset: int = 0, eps: float = 1e-5,
                     rms: bool = False, row_ids=None):
    """x0, x1, residual: [rows, hidden]; gamma/beta: [hidden]. Returns a dict
    with y0, y1 (or None), z, mean (None for RMSNorm), rstd, keep0, keep1.
    row_ids: global row indices of the given rows (for the dropout counters)."""
    x0 = _f64(x0)
    rows, hidden = x0.shape
    keep_scale = 1.0 / (1.0 - float(np.float32(p)))
    keep0 = dropout_keep(rows, hidden, p, seed, offset, 0, row_ids)
    z = np.where(keep0, x0 * keep_scale, 0.0)                        # dropout(x0)
    keep1 = None
    if x1 is not None:
        keep1 = dropout_keep(rows, hidden, p, seed, offset, 1, row_ids)
        z = z + np.where(keep1, _f64(x1) * keep_scale, 0.0)          # + dropout(x1)
    if residual is not None:
        z = z + _f64(residual)                                       # + residual
    if rms:
        mean = None
        rstd = 1.0 / np.sqrt(np.mean(z * z, axis=1) + eps)
        zn = z * rstd[:, None]
    else:
        mean = np.mean(z, axis=1)
        var = np.mean((z - mean[:, None]) ** 2, axis=1)
        rstd = 1.0 / np.sqrt(var + eps)
        zn = (z - mean[:, None]) * rstd[:, None]

    def affine(g, b):
        y = zn * _f64(g)[None, :]
        return y if b is None else y + _f64(b)[None, :]

    y0 = affine(gamma0, beta0)
    y1 = affine(gamma1, beta1) if gamma1 is not None else None
    return {"y0": y0, "y1": y1, "z": z, "mean": mean, "rstd": rstd, "keep0": keep0,
            "keep1": keep1}
