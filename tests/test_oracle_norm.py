"""Pins for the float64 dropout + residual + LayerNorm/RMSNorm oracle (CPU only).

  * Philox4x32-10 against the generator's published known-answer vectors
    (Salmon et al., SC'11: zero counter and key; all-ones counter and key;
    counter and key from the digits of pi), against Python's exact integer
    arithmetic for the 32x32->64 products, and for its statistical behaviour
    (uniform words, independent streams, avalanche);
  * the keep mask: integer threshold, expected keep rate, p = 0 keeps all;
  * LayerNorm / RMSNorm against torch's layer_norm / rms_norm in float64;
  * closed forms: constant rows give y = beta; p = 0 without residual is the
    norm of x0 alone; kept values are scaled by exactly 1/(1 - p); the
    parallel residual is the sum of both dropped branches.
"""
import numpy as np
import pytest
import torch

import oracle

KAT = [  # (counter, key, output) of Philox4x32-10
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


@pytest.mark.parametrize("ctr,key,want", KAT)
def test_philox_known_answers(ctr, key, want):
    got = oracle.philox4x32_10(np.array([ctr], dtype=np.uint64), key)[0]
    assert tuple(int(x) for x in got) == want


def test_philox_products_are_exact():
    # the uint64 products of the oracle equal Python's unbounded integers
    rng = np.random.default_rng(0)
    c = rng.integers(0, 2**32, size=(1000, 4), dtype=np.uint64)
    k = (0x12345678, 0x9ABCDEF0)
    got = oracle.philox4x32_10(c, k)
    M0, M1, W0, W1 = 0xD2511F53, 0xCD9E8D57, 0x9E3779B9, 0xBB67AE85
    for row in range(0, 1000, 97):
        x = [int(v) for v in c[row]]
        k0, k1 = k
        for _ in range(10):
            p0, p1 = M0 * x[0], M1 * x[2]
            x = [(p1 >> 32) ^ x[1] ^ k0, p1 % 2**32, (p0 >> 32) ^ x[3] ^ k1, p0 % 2**32]
            k0, k1 = (k0 + W0) % 2**32, (k1 + W1) % 2**32
        assert [int(v) for v in got[row]] == x


def test_philox_statistics():
    n = 1 << 16
    ctr = np.zeros((n, 4), dtype=np.uint64)
    ctr[:, 0] = np.arange(n)
    w = oracle.philox4x32_10(ctr, (7, 9))
    # uniform: 16 equal bins of the top 4 bits, chi-square with 15 dof
    counts = np.bincount((w.reshape(-1) >> np.uint64(28)).astype(np.int64), minlength=16)
    expect = w.size / 16
    chi2 = float(((counts - expect) ** 2 / expect).sum())
    assert chi2 < 40.0
    # avalanche: flipping one counter bit flips about half of the 128 output bits
    ctr2 = ctr.copy()
    ctr2[:, 0] ^= np.uint64(1 << 5)
    w2 = oracle.philox4x32_10(ctr2, (7, 9))
    flips = np.unpackbits((w ^ w2).astype(">u4").view(np.uint8)).mean()
    assert abs(flips - 0.5) < 0.01


def test_keep_mask_threshold_and_rate():
    assert oracle.keep_threshold(0.0) == 0
    assert oracle.keep_threshold(0.5) == 2**31
    assert oracle.keep_threshold(0.25) == 2**30
    k = oracle.dropout_keep(64, 4096, 0.1, seed=3, offset=11)
    assert abs(k.mean() - 0.9) < 0.003
    assert oracle.dropout_keep(8, 64, 0.0, seed=3, offset=11).all()
    # two streams (branches) and two offsets are different masks
    k1 = oracle.dropout_keep(64, 4096, 0.1, seed=3, offset=11, stream=1)
    k2 = oracle.dropout_keep(64, 4096, 0.1, seed=3, offset=12)
    assert (k != k1).mean() > 0.1 and (k != k2).mean() > 0.1
    with pytest.raises(ValueError):
        oracle.keep_threshold(1.0)


def test_keep_mask_element_order():
    # element e of the flat [rows, hidden] array uses word e % 4 of block e // 4
    rows, hidden, seed, offset = 3, 40, 0x1234_5678_9ABC, (5 << 32) | 77
    k = oracle.dropout_keep(rows, hidden, 0.5, seed, offset, stream=1)
    for e in [0, 1, 2, 3, 4, 39, 40, 41, 119]:
        q = e // 4
        w = oracle.philox4x32_10(np.array([[q, 0, 77, 6]], dtype=np.uint64),
                                 (seed & 0xFFFFFFFF, seed >> 32))[0, e % 4]
        assert k.reshape(-1)[e] == (int(w) >= 2**31)


def _inputs(rows, hidden, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((rows, hidden)), rng.standard_normal((rows, hidden)),
            rng.standard_normal((rows, hidden)), 1 + 0.1 * rng.standard_normal(hidden),
            0.1 * rng.standard_normal(hidden))


@pytest.mark.parametrize("p", [0.0, 0.1, 0.5])
def test_layernorm_against_torch(p):
    x0, x1, r, g, b = _inputs(17, 64, 1)
    out = oracle.dropout_add_norm(x0, g, b, residual=r, p=p, seed=5, offset=2, eps=1e-5)
    z = np.where(out["keep0"], x0 / (1 - np.float32(p).item()), 0.0) + r
    np.testing.assert_allclose(out["z"], z, rtol=0, atol=1e-14)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(z), (64,), torch.from_numpy(g),
                                         torch.from_numpy(b), eps=1e-5)
    np.testing.assert_allclose(out["y0"], ref.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(out["mean"], z.mean(axis=1), rtol=0, atol=1e-14)
    np.testing.assert_allclose(out["rstd"], 1 / np.sqrt(z.var(axis=1) + 1e-5), rtol=1e-13)


def test_rmsnorm_against_torch():
    x0, x1, r, g, b = _inputs(9, 128, 2)
    out = oracle.dropout_add_norm(x0, g, None, residual=r, p=0.2, seed=1, offset=0, eps=1e-6,
                                  rms=True)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(out["z"]), (128,), torch.from_numpy(g),
                                       eps=1e-6)
    np.testing.assert_allclose(out["y0"], ref.numpy(), rtol=0, atol=1e-12)
    assert out["mean"] is None


def test_constant_rows_give_beta():
    rows, hidden = 4, 32
    g = np.linspace(0.5, 2, hidden)
    b = np.linspace(-1, 1, hidden)
    x0 = np.full((rows, hidden), 3.0)
    out = oracle.dropout_add_norm(x0, g, b, p=0.0)
    np.testing.assert_allclose(out["y0"], np.broadcast_to(b, (rows, hidden)), atol=1e-12)


def test_no_dropout_no_residual_is_plain_norm():
    x0, _, _, g, b = _inputs(5, 48, 3)
    out = oracle.dropout_add_norm(x0, g, b, p=0.0)
    mu = x0.mean(axis=1, keepdims=True)
    y = (x0 - mu) / np.sqrt(((x0 - mu) ** 2).mean(axis=1, keepdims=True) + 1e-5) * g + b
    np.testing.assert_allclose(out["y0"], y, atol=1e-12)
    assert out["keep0"].all()


def test_kept_values_scaled_exactly():
    x0 = np.ones((4, 64))
    out = oracle.dropout_add_norm(x0, np.ones(64), p=0.25, seed=9, offset=4)
    kept = out["z"][out["keep0"]]
    assert np.all(kept == 1.0 / (1.0 - 0.25)) and np.all(out["z"][~out["keep0"]] == 0.0)


def test_parallel_residual_and_second_output():
    x0, x1, r, g, b = _inputs(6, 64, 4)
    g1, b1 = g[::-1].copy(), -b
    out = oracle.dropout_add_norm(x0, g, b, residual=r, x1=x1, gamma1=g1, beta1=b1, p=0.3,
                                  seed=2, offset=8)
    s = 1 / (1 - np.float32(0.3).item())
    z = np.where(out["keep0"], x0 * s, 0) + np.where(out["keep1"], x1 * s, 0) + r
    np.testing.assert_allclose(out["z"], z, atol=1e-14)
    zn = (z - z.mean(1, keepdims=True)) / np.sqrt(z.var(1, keepdims=True) + 1e-5)
    np.testing.assert_allclose(out["y1"], zn * g1 + b1, atol=1e-12)
    assert (out["keep0"] != out["keep1"]).mean() > 0.2


def test_row_ids_select_rows_of_the_full_mask():
    full = oracle.dropout_keep(50, 24, 0.4, seed=8, offset=3, stream=1)
    sub = oracle.dropout_keep(3, 24, 0.4, seed=8, offset=3, stream=1, row_ids=[0, 17, 49])
    np.testing.assert_array_equal(sub, full[[0, 17, 49]])
