"""Seeded random sweep of the dense, packed and banded forwards and the backward
against the float64 oracles:
random storage dtypes, head sizes, batch and head counts, ragged lengths,
scales and packed-sequence mixes, drawn once from a fixed seed so every run
checks the same cases. It crosses the 4-/8-wave threshold of the dense
16-bit path (N = 2048) and the 64-sequence threshold of the packed unit order.
Full comparison for short problems, sampled rows (exact against all keys)
for long ones. FA_SWEEP_MULT=k draws k times as many cases per kernel (the
default set is the first of them); the default is 1."""
import math
import os

import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import TOL, announce, assert_close, device, f64, run_dense, run_varlen

pytestmark = pytest.mark.gpu
MULT = max(1, int(os.environ.get("FA_SWEEP_MULT", "1")))


def _dense_cases(n=24 * MULT, seed=2026):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dtype = ["fp32", "bf16", "fp16"][rng.integers(3)]
        d = [64, 128][rng.integers(2)]
        long = dtype != "fp32" and rng.random() < 0.45
        N = int(rng.integers(2049, 2400)) if long else int(rng.integers(1, 400))
        cases.append((i, dtype, d, int(rng.integers(1, 3)), int(rng.integers(1, 4)), N,
                      float(rng.uniform(0.05, 0.3))))
    return cases


def _varlen_cases(n=12 * MULT, seed=2027):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dtype = ["fp32", "bf16", "fp16"][rng.integers(3)]
        d = [64, 128][rng.integers(2)]
        nseq = int(rng.choice([1, 3, 17, 63, 64, 65, 90]))
        lengths = [int(x) for x in rng.choice([0, 1, 33, 64, 65, 127, 200, 513], size=nseq)]
        if sum(lengths) == 0:
            lengths[0] = 7
        if dtype != "fp32" and rng.random() < 0.3:
            lengths[-1] = 4200  # past the 4-wave limit: the 8-wave packed kernel
        cases.append((i, dtype, d, int(rng.integers(1, 4)), lengths, float(rng.uniform(0.05, 0.3))))
    return cases


@pytest.mark.parametrize("case", _dense_cases(), ids=lambda c: f"dense{c[0]}-{c[1]}-d{c[2]}-N{c[5]}")
def test_dense_sweep(case):
    i, dtype, d, B, H, N, scale = case
    dev = device()
    announce(f"sweep dense #{i}: {dtype} B={B} H={H} N={N} d={d} scale={scale:.4f}")
    q, k, v = workloads.dense_inputs(B, H, N, d, dtype, seed=1000 + i)
    o, lse = run_dense(q, k, v, scale, dev)
    tol_o, tol_l = TOL[dtype]
    if N <= 400:
        O_ref, L_ref = oracle.attention_dense(q, k, v, scale)
        assert_close("O", f64(o), O_ref, tol_o)
        assert_close("L", f64(lse), L_ref, tol_l)
        return
    rng = np.random.default_rng(i)
    rows = np.unique(np.concatenate([[0, 255, 256, N // 2, N - 257, N - 1],
                                     rng.integers(0, N, size=16)]))
    for b, h in {(0, 0), (B - 1, H - 1)}:
        O_ref, L_ref = oracle.attention_dense_rows(q, k, v, scale, b, h, rows)
        assert_close(f"O[{b},{h}]", f64(o[b, h, rows]), O_ref, tol_o)
        assert_close(f"L[{b},{h}]", f64(lse[b, h, rows]), L_ref, tol_l)


@pytest.mark.parametrize("case", _varlen_cases(), ids=lambda c: f"varlen{c[0]}-{c[1]}-d{c[2]}-n{len(c[4])}")
def test_varlen_sweep(case):
    i, dtype, d, H, lengths, scale = case
    dev = device()
    announce(f"sweep varlen #{i}: {dtype} H={H} d={d} scale={scale:.4f} lengths={lengths}")
    q, k, v, cu = workloads.varlen_inputs(lengths, H, d, dtype, seed=2000 + i)
    o, lse = run_varlen(q, k, v, cu, max(lengths), scale, dev)
    O_ref, L_ref = oracle.attention_varlen(q, k, v, cu, scale)
    tol_o, tol_l = TOL[dtype]
    assert_close("O", f64(o), O_ref, tol_o)
    assert_close("L", f64(lse), L_ref, tol_l)


def _band_cases(n=12 * MULT, seed=2028):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dtype = ["bf16", "fp16"][rng.integers(2)]
        d = [64, 128][rng.integers(2)]
        if rng.random() < 0.3:  # windows past 2048 take the 8-wave kernel
            N, window = int(rng.integers(2100, 2600)), int(rng.integers(2049, 2600))
        else:
            N = int(rng.integers(1, 500))
            window = int(rng.choice([0, 1, 31, 63, 64, 65, int(rng.integers(0, 600))]))
        cases.append((i, dtype, d, int(rng.integers(1, 3)), int(rng.integers(1, 3)), N, window,
                      float(rng.uniform(0.05, 0.3))))
    return cases


@pytest.mark.parametrize("case", _band_cases(), ids=lambda c: f"band{c[0]}-{c[1]}-d{c[2]}-N{c[5]}-w{c[6]}")
def test_banded_sweep(case):
    import exact_attention_26_amd as fa
    i, dtype, d, B, H, N, window, scale = case
    dev = device()
    announce(f"sweep banded #{i}: {dtype} B={B} H={H} N={N} d={d} window={window} scale={scale:.4f}")
    q, k, v = workloads.dense_inputs(B, H, N, d, dtype, seed=3000 + i)
    o, lse = fa.forward_banded(q.to(dev), k.to(dev), v.to(dev), window, scale)
    tol_o, tol_l = TOL[dtype]
    if N <= 500:
        O_ref, L_ref = oracle.attention_banded_dense(q, k, v, scale, window)
        assert_close("O", f64(o), O_ref, tol_o)
        assert_close("L", f64(lse), L_ref, tol_l)
        return
    rng = np.random.default_rng(i)
    rows = np.unique(np.concatenate([[0, 255, 256, N // 2, N - 257, N - 1],
                                     rng.integers(0, N, size=12)]))
    for b, h in {(0, 0), (B - 1, H - 1)}:
        O_ref, L_ref = oracle.attention_banded_dense_rows(q, k, v, scale, window, b, h, rows)
        assert_close(f"O[{b},{h}]", f64(o[b, h, rows]), O_ref, tol_o)
        assert_close(f"L[{b},{h}]", f64(lse[b, h, rows]), L_ref, tol_l)


def _bwd_cases(n=12 * MULT, seed=2029):
    rng = np.random.default_rng(seed)
    return [(i, ["bf16", "fp16"][rng.integers(2)], [64, 128][rng.integers(2)],
             int(rng.integers(1, 3)), int(rng.integers(1, 3)), int(rng.integers(1, 700)),
             float(rng.uniform(0.05, 0.3))) for i in range(n)]


@pytest.mark.parametrize("case", _bwd_cases(), ids=lambda c: f"bwd{c[0]}-{c[1]}-d{c[2]}-N{c[5]}")
def test_backward_sweep(case):
    from test_parity_bwd import TOL_BWD, check_grads, reference_grads, run_bwd
    i, dtype, d, B, H, N, scale = case
    dev = device()
    announce(f"sweep backward #{i}: {dtype} B={B} H={H} N={N} d={d} scale={scale:.4f}")
    q, k, v, do = workloads.dense_bwd_inputs(B, H, N, d, dtype, seed=4000 + i)
    got, fwd = run_bwd(q, k, v, do, scale, dev)
    want = reference_grads(q, k, v, do, fwd, scale)
    check_grads(f"sweep {i}", got, want, TOL_BWD[dtype],
                oracle.attention_backward_dense(q, k, v, do, scale))
