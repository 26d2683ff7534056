"""GPU parity of the banded forward (fa_fwd_banded) against the float64
banded oracle, element by element on the same dtype-rounded inputs.

Bounds are those of the full forward (bf16/fp16: O <= 2e-2, L <= 5e-3):
the in-band work is the same arithmetic, and masked keys contribute exact
zeros. Small problems are compared in full, over windows that cut the
64-key tiles and 256-row workgroups at every kind of boundary (0, 1, tile
width +- 1, wider than a workgroup, the whole sequence and beyond). The
full-size head (B=2 H=32 N=8192 d=128) is compared on sampled rows, plus
properties that hold at any size. A window that keeps every key must give
the full forward's bits; window 0 must return V itself.
"""
import math

import numpy as np
import pytest
import torch

import exact_attention_26_amd as fa
import oracle
import workloads
from gpu_helpers import TOL, announce, assert_close, device, f64

pytestmark = pytest.mark.gpu


def run_banded(q, k, v, window, scale, dev):
    o, lse = fa.forward_banded(q.to(dev), k.to(dev), v.to(dev), window, scale)
    torch.cuda.synchronize()
    return o, lse


SMALL = [(1, 0), (1, 5), (2, 0), (2, 1), (65, 0), (65, 1), (65, 63), (65, 64),
         (257, 0), (257, 1), (257, 31), (257, 63), (257, 64), (257, 65), (257, 100),
         (257, 255), (257, 256), (257, 300), (1000, 0), (1000, 64), (1000, 129), (1000, 300),
         (1000, 700), (1000, 999), (1000, 5000)]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N,window", SMALL)
def test_small_banded(dtype, d, N, window):
    dev = device()
    B, H = (2, 3) if N <= 257 else (1, 2)
    seed = 7000 * d + 13 * N + window + (0 if dtype == "bf16" else 50000)
    announce(f"small banded {dtype} B={B} H={H} N={N} d={d} window={window} seed={seed}")
    q, k, v = workloads.dense_inputs(B, H, N, d, dtype, seed=seed)
    scale = 1.0 / math.sqrt(d)
    o, lse = run_banded(q, k, v, window, scale, dev)
    O_ref, L_ref = oracle.attention_banded_dense(q, k, v, scale, window)
    tol_o, tol_l = TOL[dtype]
    assert_close("O", f64(o), O_ref, tol_o)
    assert_close("L", f64(lse), L_ref, tol_l)


@pytest.mark.parametrize("N", [64, 300, 1000])
def test_window_zero_returns_v(N):
    dev = device()
    announce(f"banded window 0 bf16 N={N}")
    q, k, v = workloads.dense_inputs(1, 2, N, 128, "bf16", seed=N)
    o, lse = run_banded(q, k, v, 0, 0.088, dev)
    assert torch.equal(o.cpu(), v), "window 0: O must be V exactly"
    L_ref = 0.088 * (f64(q) * f64(k)).sum(-1)
    assert_close("L", f64(lse), L_ref, TOL["bf16"][1])


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("N,window", [(300, 299), (300, 300), (1000, 1 << 30), (64, 63)])
def test_full_window_is_bitwise_full_forward(dtype, N, window):
    dev = device()
    announce(f"banded full window {dtype} N={N} window={window}")
    q, k, v = workloads.dense_inputs(2, 2, N, 64, dtype, seed=N + 3)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o, lse = fa.forward_banded(qd, kd, vd, window, 0.125)
    of, lf = fa.forward(qd, kd, vd, 0.125)
    torch.cuda.synchronize()
    assert torch.equal(o, of) and torch.equal(lse, lf)


def _rows(n, w, rng):
    fixed = [0, 1, w - 1, w, w + 1, 63, 64, 255, 256, 257, n // 2, n - w - 2, n - w - 1, n - w,
             n - 257, n - 256, n - 65, n - 64, n - 2, n - 1]
    rows = {r for r in fixed if 0 <= r < n}
    rows.update(int(x) for x in rng.integers(0, n, size=24))
    return np.array(sorted(rows))


@pytest.mark.parametrize("window", [64, 256, 1000, 4096])
def test_full_size_banded_sampled(window):
    dev = device()
    B, H, N, d = 2, 32, 8192, 128
    announce(f"full-size banded bf16 B={B} H={H} N={N} d={d} window={window} (sampled rows)")
    q, k, v = workloads.dense_inputs(B, H, N, d, "bf16", seed=2)
    scale = 1.0 / math.sqrt(d)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o, lse = fa.forward_banded(qd, kd, vd, window, scale)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    tol_o, tol_l = TOL["bf16"]
    rng = np.random.default_rng(window)
    for (b, h) in [(0, 0), (1, 31), (0, 17)]:
        rows = _rows(N, window, rng)
        O_ref, L_ref = oracle.attention_banded_dense_rows(q, k, v, scale, window, b, h, rows)
        assert_close(f"O[b={b},h={h}]", f64(o[b, h, rows]), O_ref, tol_o)
        assert_close(f"L[b={b},h={h}]", f64(lse[b, h, rows]), L_ref, tol_l)


# Windows above the 4-wave limit run the 8-wave kernel. With N = 6000 and
# window 2100 its 256-row workgroups visit 37, 41, 45, ... key tiles, so the
# loop starts in each of its three phases; near the end of the sequence the
# visited range is cut by n and ends in a ragged tile.
@pytest.mark.parametrize("d", [64, 128])
def test_banded_eight_wave_phases(d):
    dev = device()
    B, H, N, window = 1, 2, 6000, 2100
    announce(f"banded 8-wave phases bf16 B={B} H={H} N={N} d={d} window={window} (rows of every workgroup)")
    q, k, v = workloads.dense_inputs(B, H, N, d, "bf16", seed=40 + d)
    scale = 1.0 / math.sqrt(d)
    o, lse = run_banded(q, k, v, window, scale, dev)
    tol_o, tol_l = TOL["bf16"]
    rows = np.unique(np.concatenate([np.arange(0, N, 37), np.arange(N - 300, N)]))
    for h in range(H):
        O_ref, L_ref = oracle.attention_banded_dense_rows(q, k, v, scale, window, 0, h, rows)
        assert_close(f"O[h={h}]", f64(o[0, h, rows]), O_ref, tol_o)
        assert_close(f"L[h={h}]", f64(lse[0, h, rows]), L_ref, tol_l)


def test_banded_is_deterministic():
    dev = device()
    announce("banded determinism bf16 B=1 H=4 N=3000 d=128 window=200")
    q, k, v = workloads.dense_inputs(1, 4, 3000, 128, "bf16", seed=4)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    a = fa.forward_banded(qd, kd, vd, 200, 0.09)
    b = fa.forward_banded(qd, kd, vd, 200, 0.09)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_banded_large_logits_fp16():
    # Scores of several hundred: the running max must move without overflow
    # and rows whose first tiles lie outside the band must not turn to NaN.
    dev = device()
    announce("banded large logits fp16 B=2 H=3 N=700 d=64 window=90 scale=1.0")
    q, k, v = workloads.dense_inputs(2, 3, 700, 64, "fp16", seed=11, qk_std=4.0, v_uniform=True)
    o, lse = run_banded(q, k, v, 90, 1.0, dev)
    O_ref, L_ref = oracle.attention_banded_dense(q, k, v, 1.0, 90)
    assert_close("O", f64(o), O_ref, TOL["fp16"][0])
    assert_close("L", f64(lse), L_ref, TOL["fp16"][1])
