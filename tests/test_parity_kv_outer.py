"""GPU parity of the K/V-outer forward (fa_fwd_kv_outer) against the float64
oracle: it computes the same function as the Q-outer forward, so the same
definition and the same bounds apply (bf16/fp16: O <= 2e-2, L <= 5e-3).

Small problems are compared in full, over query-row group counts that give
one group per head, ragged groups and one 32-row block per group. The
full-size head (B=2 H=32 N=8192 d=128) is compared on sampled rows, and
against the Q-outer kernel's output everywhere.
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


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N,groups", [(1, 1), (2, 5), (63, 1), (64, 2), (65, 1), (65, 3),
                                      (257, 1), (257, 4), (257, 100), (1000, 1), (1000, 7),
                                      (1000, 32)])
def test_small_kv_outer(dtype, d, N, groups):
    dev = device()
    B, H = (2, 3) if N <= 257 else (1, 2)
    seed = 9000 * d + 7 * N + groups + (0 if dtype == "bf16" else 40000)
    announce(f"small kv-outer {dtype} B={B} H={H} N={N} d={d} groups={groups} seed={seed}")
    q, k, v = workloads.dense_inputs(B, H, N, d, dtype, seed=seed)
    scale = 1.0 / math.sqrt(d)
    o, lse = fa.forward_kv_outer(q.to(dev), k.to(dev), v.to(dev), groups, scale)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention_dense(q, k, v, scale)
    tol_o, tol_l = TOL[dtype]
    assert_close("O", f64(o), O_ref, tol_o)
    assert_close("L", f64(lse), L_ref, tol_l)


def test_kv_outer_large_logits_fp16():
    dev = device()
    announce("kv-outer large logits fp16 B=2 H=3 N=500 d=64 scale=1.0 groups=2")
    q, k, v = workloads.dense_inputs(2, 3, 500, 64, "fp16", seed=12, qk_std=4.0, v_uniform=True)
    o, lse = fa.forward_kv_outer(q.to(dev), k.to(dev), v.to(dev), 2, 1.0)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention_dense(q, k, v, 1.0)
    assert_close("O", f64(o), O_ref, TOL["fp16"][0])
    assert_close("L", f64(lse), L_ref, TOL["fp16"][1])


def test_full_size_kv_outer_sampled():
    dev = device()
    B, H, N, d = 2, 32, 8192, 128
    announce(f"full-size kv-outer bf16 B={B} H={H} N={N} d={d} groups=16 (sampled rows)")
    q, k, v = workloads.dense_inputs(B, H, N, d, "bf16", seed=3)
    scale = 1.0 / math.sqrt(d)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o, lse = fa.forward_kv_outer(qd, kd, vd, 16, scale)
    of, lf = fa.forward(qd, kd, vd, scale)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    tol_o, tol_l = TOL["bf16"]
    # both kernels against each other everywhere (each is within tol of the oracle)
    assert float((o.float() - of.float()).abs().max()) <= 2 * tol_o
    assert float((lse - lf).abs().max()) <= 2 * tol_l
    rng = np.random.default_rng(5)
    for (b, h) in [(0, 0), (1, 31)]:
        rows = np.unique(np.r_[0, 31, 32, 511, 512, 4095, 8191, rng.integers(0, N, 30)])
        O_ref, L_ref = oracle.attention_dense_rows(q, k, v, scale, b, h, rows)
        assert_close(f"O[b={b},h={h}]", f64(o[b, h, rows]), O_ref, tol_o)
        assert_close(f"L[b={b},h={h}]", f64(lse[b, h, rows]), L_ref, tol_l)
