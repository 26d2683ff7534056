"""GPU parity of the backward (fa_bwd) against the float64 backward oracle.

The GPU forward (fa_fwd) produces O and L for the same dtype-rounded inputs,
fa_bwd turns them and dO into dQ, dK, dV, and the oracle computes the exact
gradients of the rounded Q, K, V, dO. Bound: max |GPU - oracle| <=
TOL_BWD[dtype] * max |oracle| for each of dQ, dK, dV (the scale is at least
0.1 x the largest of the three, for gradients that vanish). The bound is relative
to the gradient's own scale because gradient magnitudes vary with N, the
scale and the inputs; its value is a few units of the storage dtype's
rounding (2^-9 for bf16, 2^-11 for fp16), which is where P and dS are
rounded and where the forward's O (used for D) was rounded.
"""
import math

import numpy as np
import pytest
import torch

import exact_attention_26_amd as fa
import oracle
import workloads
from gpu_helpers import announce, device, f64

pytestmark = pytest.mark.gpu

TOL_BWD = {"bf16": 1e-2, "fp16": 2.5e-3}


def check_grads(tag, got, want, tol):
    # A gradient can be exactly zero (one key: dQ = dK = 0); its rounding
    # errors still scale with |dO| |V|, which the largest gradient reflects.
    floor = 0.1 * max(float(np.max(np.abs(w))) for w in want)
    for name, g, w in zip(("dQ", "dK", "dV"), got, want):
        g = f64(g)
        assert np.all(np.isfinite(g)), f"{tag} {name}: non-finite values"
        scale = max(float(np.max(np.abs(w))), floor)
        err = np.abs(g - w)
        idx = tuple(int(i) for i in np.unravel_index(int(np.argmax(err)), err.shape))
        print(f"[{tag}] {name}: max|err| {err[idx]:.3e} = {err[idx] / max(scale, 1e-30):.2e} x "
              f"max|ref| {scale:.3e}", flush=True)
        assert err[idx] <= tol * scale, (f"{tag} {name}: max|err| {err[idx]:.3e} > {tol} x "
                                         f"{scale:.3e} at {idx}: got {g[idx]}, oracle {w[idx]}")


def run_bwd(q, k, v, do, scale, dev):
    q, k, v, do = (t.to(dev) for t in (q, k, v, do))
    o, lse = fa.forward(q, k, v, scale)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, scale)
    torch.cuda.synchronize()
    return dq, dk, dv


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 2, 17, 63, 64, 65, 130, 257, 1000])
def test_small_dense_bwd(dtype, d, N):
    dev = device()
    B, H = (2, 2) if N <= 257 else (1, 2)
    seed = 7000 + 1000 * d + N + (50000 if dtype == "fp16" else 0)
    announce(f"bwd small {dtype} B={B} H={H} N={N} d={d} seed={seed}")
    q, k, v, do = workloads.dense_bwd_inputs(B, H, N, d, dtype, seed=seed)
    scale = 1.0 / math.sqrt(d)
    got = run_bwd(q, k, v, do, scale, dev)
    want = oracle.attention_backward_dense(q, k, v, do, scale)
    check_grads(f"{dtype} N={N} d={d}", got, want, TOL_BWD[dtype])


def test_large_logits_fp16_bwd():
    dev = device()
    announce("bwd large-logit fp16 B=1 H=2 N=300 d=64 scale=0.125")
    q, k, v, do = workloads.dense_bwd_inputs(1, 2, 300, 64, "fp16", seed=77, qk_std=4.0,
                                             v_uniform=True)
    got = run_bwd(q, k, v, do, 0.125, dev)
    want = oracle.attention_backward_dense(q, k, v, do, 0.125)
    check_grads("large-logit fp16", got, want, TOL_BWD["fp16"])


def test_bwd_is_deterministic():
    dev = device()
    announce("bwd determinism bf16 B=1 H=4 N=700 d=128")
    q, k, v, do = (t.to(dev) for t in workloads.dense_bwd_inputs(1, 4, 700, 128, "bf16", seed=5))
    o, lse = fa.forward(q, k, v, 0.1)
    a = fa.backward(q, k, v, o, do, lse, 0.1)
    b = fa.backward(q, k, v, o, do, lse, 0.1)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_full_size_head():
    """B=2 H=32 N=8192 d=128 bf16, the forward's long-sequence shape: one head
    against the oracle in full, every head finite, and dK summing to ~0 over
    keys in every head."""
    dev = device()
    announce("bwd full size bf16 B=2 H=32 N=8192 d=128")
    q, k, v, do = workloads.dense_bwd_inputs(2, 32, 8192, 128, "bf16", seed=11)
    scale = 1.0 / math.sqrt(128)
    dq, dk, dv = run_bwd(q, k, v, do, scale, dev)
    for g in (dq, dk, dv):
        assert bool(torch.isfinite(g.float()).all())
    b, h = 1, 29
    want = oracle.attention_backward(q[b, h], k[b, h], v[b, h], do[b, h], scale)
    check_grads("full-size head (1,29)", (dq[b, h], dk[b, h], dv[b, h]), want, TOL_BWD["bf16"])
    ksum = dk.float().sum(dim=2).abs().max().item()
    kmag = dk.float().abs().max().item()
    assert ksum <= 2e-2 * kmag * math.sqrt(8192), (ksum, kmag)
