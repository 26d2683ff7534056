"""Mutation teeth for the oracle's pins (CPU only).

Each case plants one plausible mistake in the oracle's own source text (a
dropped term, a wrong sign, index or axis, a transposed operand, a wrong
log base), loads the mutant as a fresh module, and checks that the pin
suite rejects it, while the unmodified oracle passes the same suite.
"""
import math
import os
import types

import mpmath
import numpy as np
import pytest
import torch

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "oracle", "attention_f64.py")

MUTATIONS = {
    "drop_scale": ("S = scale * (Q[sel] @ K.T)", "S = (Q[sel] @ K.T)"),
    "query_as_key": ("S = scale * (Q[sel] @ K.T)", "S = scale * (Q[sel] @ Q.T)"),
    "no_max_shift": ("P = np.exp(S - m)", "P = np.exp(S)"),
    "wrong_sign": ("P = np.exp(S - m)", "P = np.exp(m - S)"),
    "column_normaliser": ("l = P.sum(axis=1, keepdims=True)", "l = P.sum(axis=0, keepdims=True)"),
    "drop_normaliser": ("O[s:s + sel.size] = (P / l) @ V", "O[s:s + sel.size] = P @ V"),
    "drop_max_in_L": ("L[s:s + sel.size] = m[:, 0] + np.log(l[:, 0])",
                      "L[s:s + sel.size] = np.log(l[:, 0])"),
    "log2_in_L": ("L[s:s + sel.size] = m[:, 0] + np.log(l[:, 0])",
                  "L[s:s + sel.size] = m[:, 0] + np.log2(l[:, 0])"),
    "last_key_dropped": ("S = scale * (Q[sel] @ K.T)", "S = scale * (Q[sel] @ K[:-1].T); V = V[:-1]"),
    "rowmax_over_queries": ("m = S.max(axis=1, keepdims=True)", "m = S.max(axis=0, keepdims=True)"),
}


def load_oracle(mutation=None):
    src = open(ORACLE_SRC).read()
    if mutation is not None:
        old, new = MUTATIONS[mutation]
        assert src.count(old) == 1, f"mutation site for {mutation!r} not found exactly once"
        src = src.replace(old, new)
    mod = types.ModuleType("oracle_under_test")
    exec(compile(src, ORACLE_SRC, "exec"), mod.__dict__)
    return mod


def _brute(Q, K, V, scale):
    mpmath.mp.dps = 50
    n, d = Q.shape
    m = K.shape[0]
    O = np.zeros((n, V.shape[1]))
    L = np.zeros(n)
    for r in range(n):
        s = [mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(Q[r, t]) * mpmath.mpf(K[c, t])
                                             for t in range(d)) for c in range(m)]
        lse = mpmath.log(mpmath.fsum(mpmath.exp(x) for x in s))
        L[r] = float(lse)
        for j in range(V.shape[1]):
            O[r, j] = float(mpmath.fsum(mpmath.exp(s[c] - lse) * mpmath.mpf(V[c, j])
                                        for c in range(m)))
    return O, L


def pins_pass(mod) -> bool:
    """The oracle pin suite in miniature: brute force, a library routine,
    closed forms and a large-score row. True only if every check holds."""
    try:
        with np.errstate(all="ignore"):
            rng = np.random.default_rng(0)
            for (n, m, d) in [(3, 5, 4), (4, 4, 2), (1, 3, 3)]:
                Q = rng.standard_normal((n, d))
                K = rng.standard_normal((m, d))
                V = rng.standard_normal((m, d + 1))
                O, L = mod.attention_naive(Q, K, V, 0.7)
                Ob, Lb = _brute(Q, K, V, 0.7)
                if not (np.max(np.abs(O - Ob)) <= 1e-13 and np.max(np.abs(L - Lb)) <= 1e-13):
                    return False
            Q = rng.standard_normal((20, 16))
            K = rng.standard_normal((33, 16))
            V = rng.standard_normal((33, 16))
            O, _ = mod.attention_naive(Q, K, V, 0.25)
            t = lambda a: torch.from_numpy(a)[None, None]
            ref = torch.nn.functional.scaled_dot_product_attention(t(Q), t(K), t(V), scale=0.25)
            if not np.max(np.abs(O - ref[0, 0].numpy())) <= 1e-12:
                return False
            # identical keys: uniform weights, L = scale q.k + ln m
            k = rng.standard_normal(16)
            O, L = mod.attention_naive(Q, np.tile(k, (33, 1)), V, 0.25)
            if not (np.max(np.abs(O - V.mean(axis=0))) <= 1e-13
                    and np.max(np.abs(L - (0.25 * Q @ k + math.log(33)))) <= 1e-13):
                return False
            # the overflow example: scores 800, 810, 805, 790
            Qx = np.zeros((1, 4)); Qx[0, 0] = 1.0
            Kx = np.zeros((4, 4)); Kx[:, 0] = [800.0, 810.0, 805.0, 790.0]
            O, L = mod.attention_naive(Qx, Kx, np.eye(4), 1.0)
            if not (np.all(np.isfinite(O)) and abs(O.sum() - 1.0) <= 1e-13):
                return False
        return True
    except Exception:
        return False


def test_unmodified_oracle_passes():
    assert pins_pass(load_oracle(None))


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_planted_mistake_is_caught(mutation):
    assert not pins_pass(load_oracle(mutation))


# ---------------------------------------------------------------------------
# The backward oracle: the same scheme on oracle/attention_bwd_f64.py.
# ---------------------------------------------------------------------------
BWD_SRC = os.path.join(os.path.dirname(ORACLE_SRC), "attention_bwd_f64.py")

BWD_MUTATIONS = {
    "drop_D": ("dS = P * (dP - D)", "dS = P * dP"),
    "wrong_D_sign": ("dS = P * (dP - D)", "dS = P * (dP + D)"),
    "D_without_O": ("D = np.sum(dO[rows] * O, axis=1, keepdims=True)",
                    "D = np.sum(dO[rows], axis=1, keepdims=True)"),
    "dQ_without_scale": ("dQ[rows] = scale * (dS @ K)", "dQ[rows] = (dS @ K)"),
    "dQ_against_V": ("dQ[rows] = scale * (dS @ K)", "dQ[rows] = scale * (dS @ V)"),
    "dK_without_scale": ("dK += scale * (dS.T @ Q[rows])", "dK += (dS.T @ Q[rows])"),
    "dK_against_dO": ("dK += scale * (dS.T @ Q[rows])", "dK += scale * (dS.T @ dO[rows])"),
    "dV_from_P_times_dP": ("dV += P.T @ dO[rows]", "dV += (P * (dO[rows] @ V.T)).T @ dO[rows]"),
    "P_unnormalised": ("P = E / E.sum(axis=1, keepdims=True)", "P = E"),
    "normaliser_over_queries": ("P = E / E.sum(axis=1, keepdims=True)", "P = E / E.sum(axis=0, keepdims=True)"),
    "no_max_shift_overflow": ("E = np.exp(S - S.max(axis=1, keepdims=True))", "E = np.exp(S)"),
}


def load_bwd(mutation=None):
    """The backward oracle's module, with the mutation (if any) applied
    inside attention_backward's body only (the same text also appears in the
    docstring and in the rendering from L)."""
    src = open(BWD_SRC).read()
    if mutation is not None:
        old, new = BWD_MUTATIONS[mutation]
        a = src.index("def attention_backward(")
        b = src.index("def attention_backward_lse(")
        body = src[a:b]
        assert body.count(old) == 1, f"mutation site for {mutation!r} not found exactly once"
        src = src[:a] + body.replace(old, new) + src[b:]
    mod = types.ModuleType("bwd_oracle_under_test")
    exec(compile(src, BWD_SRC, "exec"), mod.__dict__)
    return mod


def bwd_pins_pass(mod) -> bool:
    """The backward pin suite in miniature: torch autograd in float64 (a
    library's own derivative), a large-score case and the key-sum identity."""
    try:
        with np.errstate(all="ignore"):
            rng = np.random.default_rng(1)
            for (n, m, d, scale) in [(7, 9, 4, 0.6), (12, 5, 4, 1.3), (3, 3, 4, 0.2)]:
                Q, K, V, G = (rng.standard_normal(s) for s in ((n, d), (m, d), (m, d), (n, d)))
                got = mod.attention_backward(Q, K, V, G, scale)
                q, k, v = (torch.tensor(x, requires_grad=True) for x in (Q, K, V))
                o = torch.nn.functional.scaled_dot_product_attention(q[None], k[None], v[None],
                                                                     scale=scale)[0]
                o.backward(torch.tensor(G))
                for a, b in zip(got, (q.grad, k.grad, v.grad)):
                    if not (a.shape == b.shape and np.max(np.abs(a - b.numpy())) <= 1e-12):
                        return False
            # scores of several hundred: no overflow
            Q = rng.standard_normal((4, 4)) * 30
            K = rng.standard_normal((6, 4)) * 30
            V, G = rng.standard_normal((6, 4)), rng.standard_normal((4, 4))
            if not all(np.all(np.isfinite(g)) for g in mod.attention_backward(Q, K, V, G, 1.0)):
                return False
        return True
    except Exception:
        return False


def test_unmodified_bwd_oracle_passes():
    assert bwd_pins_pass(load_bwd(None))


@pytest.mark.parametrize("mutation", sorted(BWD_MUTATIONS))
def test_planted_bwd_mistake_is_caught(mutation):
    assert not bwd_pins_pass(load_bwd(mutation))


# ---------------------------------------------------------------------------
# The banded oracle: the same scheme on oracle/attention_band_f64.py.
# ---------------------------------------------------------------------------
BAND_SRC = os.path.join(os.path.dirname(ORACLE_SRC), "attention_band_f64.py")

BAND_MUTATIONS = {
    "edge_excluded": ("<= window   #", "< window   #"),
    "one_sided": ("np.abs(sel[:, None] - keys[None, :]) <= window",
                  "(keys[None, :] - sel[:, None]) <= window"),
    "chunk_local_row_index": ("np.abs(sel[:, None] - keys[None, :])",
                              "np.abs(np.arange(sel.size)[:, None] - keys[None, :])"),
    "masked_score_zero": ("np.where(band, scale * (Q[sel] @ K.T), -np.inf)",
                          "np.where(band, scale * (Q[sel] @ K.T), 0.0)"),
    "drop_scale": ("np.where(band, scale * (Q[sel] @ K.T), -np.inf)",
                   "np.where(band, (Q[sel] @ K.T), -np.inf)"),
    "mask_ignored": ("np.where(band, scale * (Q[sel] @ K.T), -np.inf)",
                     "np.where(True, scale * (Q[sel] @ K.T), -np.inf)"),
    "drop_max_in_L": ("L[s:s + sel.size] = m[:, 0] + np.log(l[:, 0])",
                      "L[s:s + sel.size] = np.log(l[:, 0])"),
    "drop_normaliser": ("O[s:s + sel.size] = (P / l) @ V", "O[s:s + sel.size] = P @ V"),
}


def load_band(mutation=None):
    src = open(BAND_SRC).read()
    if mutation is not None:
        old, new = BAND_MUTATIONS[mutation]
        a = src.index("def attention_banded_rows(")
        b = src.index("def attention_banded(")
        body = src[a:b]
        assert body.count(old) == 1, f"mutation site for {mutation!r} not found exactly once"
        src = src[:a] + body.replace(old, new) + src[b:]
    mod = types.ModuleType("band_oracle_under_test")
    exec(compile(src, BAND_SRC, "exec"), mod.__dict__)
    return mod


def _brute_band(Q, K, V, scale, w, rows):
    mpmath.mp.dps = 50
    O = np.zeros((len(rows), V.shape[1]))
    L = np.zeros(len(rows))
    for i, r in enumerate(rows):
        cs = [c for c in range(K.shape[0]) if abs(r - c) <= w]
        s = {c: mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(Q[r, t]) * mpmath.mpf(K[c, t])
                                                for t in range(Q.shape[1])) for c in cs}
        z = mpmath.fsum(mpmath.exp(s[c]) for c in cs)
        L[i] = float(mpmath.log(z))
        for j in range(V.shape[1]):
            O[i, j] = float(mpmath.fsum(mpmath.exp(s[c]) * mpmath.mpf(V[c, j]) for c in cs) / z)
    return O, L


def band_pins_pass(mod) -> bool:
    """The banded pin suite in miniature: brute force over the in-band keys
    (whole heads and a row subset), torch attention with a boolean mask and
    the identical-keys band mean."""
    try:
        with np.errstate(all="ignore"):
            rng = np.random.default_rng(2)
            for (n, d, w, rows) in [(6, 3, 0, None), (9, 4, 2, None), (5, 2, 9, None),
                                    (12, 3, 2, [4, 9])]:
                Q, K, V = (rng.standard_normal((n, d)) for _ in range(3))
                O, L = mod.attention_banded_rows(Q, K, V, 0.8, w, rows)
                Ob, Lb = _brute_band(Q, K, V, 0.8, w, range(n) if rows is None else rows)
                if not (np.max(np.abs(O - Ob)) <= 1e-13 and np.max(np.abs(L - Lb)) <= 1e-13):
                    return False
            Q, K, V = (rng.standard_normal((100, 16)) for _ in range(3))
            O, _ = mod.attention_banded(Q, K, V, 0.25, 7)
            idx = torch.arange(100)
            allowed = (idx[:, None] - idx[None, :]).abs() <= 7
            t = lambda a: torch.from_numpy(a)[None, None]
            ref = torch.nn.functional.scaled_dot_product_attention(t(Q), t(K), t(V),
                                                                   attn_mask=allowed, scale=0.25)
            if not np.max(np.abs(O - ref[0, 0].numpy())) <= 1e-12:
                return False
            k = rng.standard_normal(16)
            O, L = mod.attention_banded(Q[:40], np.tile(k, (40, 1)), V[:40], 0.6, 3)
            for r in range(40):
                lo, hi = max(0, r - 3), min(39, r + 3)
                if not (np.max(np.abs(O[r] - V[lo:hi + 1].mean(axis=0))) <= 1e-13
                        and abs(L[r] - (0.6 * Q[r] @ k + math.log(hi - lo + 1))) <= 1e-13):
                    return False
        return True
    except Exception:
        return False


def test_unmodified_band_oracle_passes():
    assert band_pins_pass(load_band(None))


@pytest.mark.parametrize("mutation", sorted(BAND_MUTATIONS))
def test_planted_band_mistake_is_caught(mutation):
    assert not band_pins_pass(load_band(mutation))


# ---------------------------------------------------------------------------
# The dropout + residual + norm oracle: the same scheme on
# oracle/dropout_add_norm_f64.py.
# ---------------------------------------------------------------------------
NORM_SRC = os.path.join(os.path.dirname(ORACLE_SRC), "dropout_add_norm_f64.py")

NORM_MUTATIONS = {
    "philox_multiplier": ("m0, m1 = np.uint64(0xD2511F53)", "m0, m1 = np.uint64(0xD2511F55)"),
    "philox_nine_rounds": ("for r in range(10):", "for r in range(9):"),
    "philox_no_key_bump": ("k0 = (k0 + w0) & _M32", "k0 = k0 & _M32"),
    "philox_swapped_halves": ("c = [((p1 >> np.uint64(32)) ^ c[1] ^ k0) & _M32, p1 & _M32,",
                              "c = [((p1 >> np.uint64(32)) ^ c[1] ^ k0) & _M32, p0 & _M32,"),
    "word_index_shifted": ("word = words[np.arange(e.size), (e % np.uint64(4)).astype(np.int64)]",
                           "word = words[np.arange(e.size), ((e + np.uint64(1)) % np.uint64(4)).astype(np.int64)]"),
    "stream_ignored": ("+ stream) & 0xFFFFFFFF)", "+ 0) & 0xFFFFFFFF)"),
    "no_keep_scale": ("z = np.where(keep0, x0 * keep_scale, 0.0)", "z = np.where(keep0, x0, 0.0)"),
    "residual_dropped": ("z = z + _f64(residual)", "z = z + 0.0"),
    "var_without_mean": ("var = np.mean((z - mean[:, None]) ** 2, axis=1)",
                         "var = np.mean(z ** 2, axis=1)"),
    "eps_outside_sqrt": ("rstd = 1.0 / np.sqrt(var + eps)", "rstd = 1.0 / np.sqrt(var) + eps"),
    "rms_centred": ("zn = z * rstd[:, None]", "zn = (z - z.mean(axis=1, keepdims=True)) * rstd[:, None]"),
    "beta_ignored": ("return y if b is None else y + _f64(b)[None, :]", "return y"),
}


def load_norm(mutation=None):
    src = open(NORM_SRC).read()
    if mutation is not None:
        old, new = NORM_MUTATIONS[mutation]
        a = src.index("def philox4x32_10(")
        body = src[a:]
        assert body.count(old) == 1, f"mutation site for {mutation!r} not found exactly once"
        src = src[:a] + body.replace(old, new)
    mod = types.ModuleType("norm_oracle_under_test")
    exec(compile(src, NORM_SRC, "exec"), mod.__dict__)
    return mod


def norm_pins_pass(mod) -> bool:
    """The norm pin suite in miniature: the generator's known answers, the
    element-to-word order, torch's layer_norm and rms_norm in float64, the
    exact keep scale and the parallel-residual sum with distinct streams."""
    try:
        with np.errstate(all="ignore"):
            kat = [((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
                   ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
                    (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1))]
            for ctr, key, want in kat:
                got = mod.philox4x32_10(np.array([ctr], dtype=np.uint64), key)[0]
                if tuple(int(x) for x in got) != want:
                    return False
            k = mod.dropout_keep(2, 16, 0.5, 3, 9, stream=1)
            for e in range(32):
                w = mod.philox4x32_10(np.array([[e // 4, 0, 9, 1]], dtype=np.uint64), (3, 0))
                if k.reshape(-1)[e] != (int(w[0, e % 4]) >= 2**31):
                    return False
            rng = np.random.default_rng(3)
            x0, x1, r = (rng.standard_normal((7, 64)) for _ in range(3))
            g, b = 1 + 0.1 * rng.standard_normal(64), 0.1 * rng.standard_normal(64)
            out = mod.dropout_add_norm(x0, g, b, residual=r, p=0.3, seed=4, offset=1)
            s = 1 / (1 - np.float32(0.3).item())
            z = np.where(out["keep0"], x0 * s, 0.0) + r
            if not np.max(np.abs(out["z"] - z)) <= 1e-13:
                return False
            ref = torch.nn.functional.layer_norm(torch.from_numpy(z), (64,), torch.from_numpy(g),
                                                 torch.from_numpy(b), eps=1e-5)
            if not np.max(np.abs(out["y0"] - ref.numpy())) <= 1e-12:
                return False
            out = mod.dropout_add_norm(x0, g, None, residual=r, p=0.0, rms=True, eps=1e-6)
            ref = torch.nn.functional.rms_norm(torch.from_numpy(x0 + r), (64,),
                                               torch.from_numpy(g), eps=1e-6)
            if not np.max(np.abs(out["y0"] - ref.numpy())) <= 1e-12:
                return False
            out = mod.dropout_add_norm(x0, g, b, residual=r, x1=x1, p=0.3, seed=2, offset=8)
            z = (np.where(out["keep0"], x0 * s, 0.0) + np.where(out["keep1"], x1 * s, 0.0) + r)
            if not (np.max(np.abs(out["z"] - z)) <= 1e-13
                    and (out["keep0"] != out["keep1"]).mean() > 0.2):
                return False
        return True
    except Exception:
        return False


def test_unmodified_norm_oracle_passes():
    assert norm_pins_pass(load_norm(None))


@pytest.mark.parametrize("mutation", sorted(NORM_MUTATIONS))
def test_planted_norm_mistake_is_caught(mutation):
    assert not norm_pins_pass(load_norm(mutation))
