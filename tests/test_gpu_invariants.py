"""GPU checks against closed forms and properties of the method, plus the
library's promises (deterministic, writes only its outputs, allocates
nothing)."""
import math

import mpmath
import numpy as np
import pytest
import torch

import exact_attention_26_amd as fa
import workloads
from gpu_helpers import TOL, announce, assert_close, device, f64, run_dense

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["fp32", "bf16", "fp16"])
def test_constant_v(dtype):
    # Every weight row sums to one, so a constant V row comes straight back.
    dev = device()
    announce(f"constant V {dtype}")
    q, k, v = workloads.dense_inputs(1, 2, 300, 128, dtype, seed=21)
    row = v[0, 0, 0].clone()
    v = row.expand_as(v).contiguous()
    o, _ = run_dense(q, k, v, 0.1, dev)
    want = np.broadcast_to(f64(row), o.shape)
    assert_close("O", f64(o), want, TOL[dtype][0])


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_identical_keys(dtype):
    # Identical keys: uniform weights, O = mean of V, L = scale*q.k + ln N.
    dev = device()
    announce(f"identical keys {dtype}")
    N, d = 257, 64
    q, k, v = workloads.dense_inputs(1, 1, N, d, dtype, seed=22)
    k = k[:, :, :1].expand_as(k).contiguous()
    o, lse = run_dense(q, k, v, 0.125, dev)
    assert_close("O", f64(o), np.broadcast_to(f64(v).mean(axis=2, keepdims=True), o.shape),
                 TOL[dtype][0])
    want_l = 0.125 * f64(q)[0, 0] @ f64(k)[0, 0, 0] + math.log(N)
    assert_close("L", f64(lse)[0, 0], want_l, TOL[dtype][1])


def test_overflow_worked_example_fp32():
    # Scores 800, 810, 805, 790 (scale 1): one query direction e0, keys
    # s_c * e0, V = identity rows, so O's first four columns are the weights.
    dev = device()
    announce("overflow worked example fp32")
    s = [800.0, 810.0, 805.0, 790.0]
    N, d = 4, 64
    q = torch.zeros(1, 1, N, d)
    q[..., 0] = 1.0
    k = torch.zeros(1, 1, N, d)
    k[0, 0, :, 0] = torch.tensor(s)
    v = torch.zeros(1, 1, N, d)
    v[0, 0, torch.arange(N), torch.arange(N)] = 1.0
    o, lse = run_dense(q, k, v, 1.0, dev)
    z = mpmath.fsum(mpmath.exp(mpmath.mpf(x) - 810) for x in s)
    wts = np.array([float(mpmath.exp(mpmath.mpf(x) - 810) / z) for x in s])
    assert_close("weights", f64(o)[0, 0, :, :4], np.tile(wts, (N, 1)), TOL["fp32"][0])
    assert_close("L", f64(lse)[0, 0], np.full(N, float(810 + mpmath.log(z))), 1e-4)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_shift_invariance_through_keys(dtype):
    # K' = K + 1 w^T adds scale*(q.w) to every score of row q: O unchanged,
    # L shifted by that amount. Column 0 of K is first snapped to multiples
    # of 1/8 in [-4, 4] and w = 4 e0, so both K and K' are exact in bf16.
    dev = device()
    announce(f"shift invariance {dtype}")
    q, k, v = workloads.dense_inputs(1, 2, 193, 64, dtype, seed=23)
    k[..., 0] = (k[..., 0].float() * 8).round().clamp(-32, 32).div(8).to(k.dtype)
    k2 = k.clone()
    k2[..., 0] += 4.0
    scale = 0.125
    o1, l1 = run_dense(q, k, v, scale, dev)
    o2, l2 = run_dense(q, k2, v, scale, dev)
    assert_close("O", f64(o2), f64(o1), TOL[dtype][0])
    assert_close("L shift", f64(l2) - f64(l1), scale * 4.0 * f64(q)[..., 0], TOL[dtype][1])


def test_deterministic():
    dev = device()
    w = workloads.make("short_bf16")
    announce("determinism short_bf16")
    q, k, v = w["q"].to(dev), w["k"].to(dev), w["v"].to(dev)
    o1, l1 = fa.forward(q, k, v, w["scale"])
    o2, l2 = fa.forward(q, k, v, w["scale"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_writes_only_its_outputs(dtype):
    # NaN canaries before and after O and L stay untouched.
    dev = device()
    announce(f"canaries {dtype}")
    B, H, N, d = 2, 2, 75, 128
    q, k, v = workloads.dense_inputs(B, H, N, d, dtype, seed=24)
    pad = 64
    n_o = B * H * N * d
    o_buf = torch.full((n_o + 2 * pad,), float("nan"), dtype=q.dtype, device=dev)
    l_buf = torch.full((B * H * N + 2 * pad,), float("nan"), dtype=torch.float32, device=dev)
    o = o_buf[pad:pad + n_o].view(B, H, N, d)
    lse = l_buf[pad:pad + B * H * N].view(B, H, N)
    fa.forward(q.to(dev), k.to(dev), v.to(dev), 0.1, out=o, lse=lse)
    torch.cuda.synchronize()
    for buf, n in ((o_buf, n_o), (l_buf, B * H * N)):
        assert torch.isnan(buf[:pad].float()).all() and torch.isnan(buf[pad + n:].float()).all()
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()


def test_allocates_no_device_memory():
    # The library works in the caller's buffers only: no N x N scratch and no
    # allocation of any size (device free memory unchanged across a call).
    dev = device()
    announce("no device allocation")
    w = workloads.make("short_bf16")
    q, k, v = w["q"].to(dev), w["k"].to(dev), w["v"].to(dev)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    fa.forward(q, k, v, w["scale"], out=o, lse=lse)  # warm-up (code object load)
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info(dev)
    for _ in range(3):
        fa.forward(q, k, v, w["scale"], out=o, lse=lse)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info(dev)
    assert free1 == free0


def test_launch_on_a_side_stream():
    # Work is enqueued on the caller's stream: results are ready after that
    # stream is synchronised.
    dev = device()
    announce("side stream")
    q, k, v = workloads.dense_inputs(1, 4, 512, 64, "bf16", seed=25)
    ref_o, ref_l = run_dense(q, k, v, 0.125, dev)
    s = torch.cuda.Stream(device=dev)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        o, lse = fa.forward(qd, kd, vd, 0.125)
    s.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(lse, ref_l)
