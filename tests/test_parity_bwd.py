"""GPU parity of the backward (fa_bwd) against the float64 backward oracle.

fa_bwd takes Q, K, V, the forward's O and L, and dO, and returns dQ, dK, dV:
it recomputes P = exp(S - L) with the L it is given and D = rowsum(dO * O)
with the O it is given ("FlashAttention -- for programmers, not
researchers", STAGE 5). The reference is the oracle's rendering of the same
computation on the same inputs (attention_backward_lse, pinned equal to the
chain rule of the plain definition): the GPU forward's O and L, widened to
float64. Bound: max |GPU - oracle| <= TOL_BWD[dtype] * max |oracle| for each of
dQ, dK, dV (the scale is at least 0.1 x the largest of the three, for
gradients that vanish). The bound is relative to the gradient's own scale
because gradient magnitudes vary with N, the scale and the inputs; its value
is a few units of the storage dtype's rounding (2^-9 for bf16, 2^-11 for fp16),
which is where the kernels round P and dS for the matrix products and round
their outputs.

The error against the exact gradient of the rounded Q, K, V, dO (the plain
chain rule, no forward in between) is that plus the forward's own error
carried through D and L; it is printed for every case. D weighs each
element of O by dO, so a bf16 O (itself within the forward's bounds) can move
dQ by a few units more.
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


def check_grads(tag, got, want, tol, exact=None):
    """got: the GPU's (dQ, dK, dV); want: the oracle's from the same O and L;
    exact (optional): the plain chain rule's, whose distance is only reported."""
    # A gradient can be exactly zero (one key: dQ = dK = 0); its rounding
    # errors still scale with |dO| |V|, which the largest gradient reflects.
    floor = 0.1 * max(float(np.max(np.abs(w))) for w in want)
    for j, (name, g, w) in enumerate(zip(("dQ", "dK", "dV"), got, want)):
        g = f64(g)
        assert np.all(np.isfinite(g)), f"{tag} {name}: non-finite values"
        scale = max(float(np.max(np.abs(w))), floor)
        err = np.abs(g - w)
        idx = tuple(int(i) for i in np.unravel_index(int(np.argmax(err)), err.shape))
        end = "" if exact is None else \
            f"; vs the exact gradient {float(np.max(np.abs(g - exact[j]))) / scale:.2e} x"
        print(f"[{tag}] {name}: max|err| {err[idx]:.3e} = {err[idx] / max(scale, 1e-30):.2e} x "
              f"max|ref| {scale:.3e}{end}", flush=True)
        assert err[idx] <= tol * scale, (f"{tag} {name}: max|err| {err[idx]:.3e} > {tol} x "
                                         f"{scale:.3e} at {idx}: got {g[idx]}, oracle {w[idx]}")


def run_bwd(q, k, v, do, scale, dev):
    """The GPU forward, then fa_bwd from its O and L. Returns the gradients
    and that (O, L), fa_bwd's inputs."""
    q, k, v, do = (t.to(dev) for t in (q, k, v, do))
    o, lse = fa.forward(q, k, v, scale)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, scale)
    torch.cuda.synchronize()
    return (dq, dk, dv), (o, lse)


def reference_grads(q, k, v, do, fwd, scale):
    """The oracle's gradients from the same O and L the GPU backward was given."""
    o, lse = fwd
    return oracle.attention_backward_lse_dense(q, k, v, f64(o), do, f64(lse), scale)


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
    got, fwd = run_bwd(q, k, v, do, scale, dev)
    want = reference_grads(q, k, v, do, fwd, scale)
    exact = oracle.attention_backward_dense(q, k, v, do, scale)
    check_grads(f"{dtype} N={N} d={d}", got, want, TOL_BWD[dtype], exact)


def test_large_logits_fp16_bwd():
    dev = device()
    announce("bwd large-logit fp16 B=1 H=2 N=300 d=64 scale=0.125")
    q, k, v, do = workloads.dense_bwd_inputs(1, 2, 300, 64, "fp16", seed=77, qk_std=4.0,
                                             v_uniform=True)
    got, fwd = run_bwd(q, k, v, do, 0.125, dev)
    want = reference_grads(q, k, v, do, fwd, 0.125)
    exact = oracle.attention_backward_dense(q, k, v, do, 0.125)
    check_grads("large-logit fp16", got, want, TOL_BWD["fp16"], exact)


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
    (dq, dk, dv), (o, lse) = run_bwd(q, k, v, do, scale, dev)
    for g in (dq, dk, dv):
        assert bool(torch.isfinite(g.float()).all())
    b, h = 1, 29
    want = oracle.attention_backward_lse(q[b, h], k[b, h], v[b, h], f64(o[b, h]), do[b, h],
                                         f64(lse[b, h]), scale)
    exact = oracle.attention_backward(q[b, h], k[b, h], v[b, h], do[b, h], scale)
    check_grads("full-size head (1,29)", (dq[b, h], dk[b, h], dv[b, h]), want, TOL_BWD["bf16"],
                exact)
    ksum = dk.float().sum(dim=2).abs().max().item()
    kmag = dk.float().abs().max().item()
    assert ksum <= 2e-2 * kmag * math.sqrt(8192), (ksum, kmag)
