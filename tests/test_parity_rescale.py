"""GPU parity on inputs whose running row maximum keeps moving, so that the
forward's rescale paths run: the reference max moves and O, l are rescaled
by exp(m_old - m_new) ("Kernel visualization: Flash Attention 2", the
online update of "Iteration j = 1"; "FlashAttention -- for programmers, not
researchers", STAGE 3: dropping that rescale is silently wrong).

Two input shapes (workloads.moving_max_inputs): scores that rise along the
keys (the max moves in nearly every key tile, as with large logits), and a
few isolated spikes (the max jumps at a few tiles and stays put between, so
the kernel passes back and forth between its settled and unsettled forms).
Dense sizes on both sides of the 4-/8-wave switch (N <= 2048 / > 2048),
d = 64 and 128, both 16-bit dtypes; banded windows; a packed batch. Every
element is compared with the float64 oracle on the same rounded inputs.
"""
import numpy as np
import pytest
import torch

import exact_attention_26_amd as fa
import oracle
import workloads
from gpu_helpers import TOL, announce, assert_close, device, f64, run_dense, run_varlen

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N,spikes", [(300, 0), (1000, 0), (2100, 0), (1000, 6), (2300, 9),
                                      (777, 40)])
def test_dense_moving_max(dtype, d, N, spikes):
    dev = device()
    B, H = 1, 3
    rate = 0.5 if dtype == "bf16" else 0.3  # fp16: first components stay below 2^10
    announce(f"dense moving max {dtype} d={d} N={N} spikes={spikes}")
    q, k, v = workloads.moving_max_inputs(B, H, N, d, dtype, seed=N + d + spikes, rate=rate,
                                          spikes=spikes)
    scale = d ** -0.5
    o, lse = run_dense(q, k, v, scale, dev)
    O_ref, L_ref = oracle.attention_dense(q, k, v, scale)
    tol_o, tol_l = TOL[dtype]
    assert_close("O", f64(o), O_ref, tol_o)
    assert_close("L", f64(lse), L_ref, tol_l)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N,window,spikes", [(700, 100, 0), (1300, 300, 0), (2500, 3000, 0),
                                             (1200, 200, 12), (2400, 2400, 12)])
def test_banded_moving_max(d, N, window, spikes):
    dev = device()
    announce(f"banded moving max d={d} N={N} w={window} spikes={spikes}")
    q, k, v = workloads.moving_max_inputs(1, 2, N, d, "bf16", seed=3 * N + window, rate=0.5,
                                          spikes=spikes)
    scale = d ** -0.5
    o, lse = fa.forward_banded(q.to(dev), k.to(dev), v.to(dev), window, scale)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention_banded_dense(q, k, v, scale, window)
    tol_o, tol_l = TOL["bf16"]
    assert_close("O", f64(o), O_ref, tol_o)
    assert_close("L", f64(lse), L_ref, tol_l)


@pytest.mark.parametrize("d", [64, 128])
def test_varlen_moving_max(d):
    dev = device()
    lengths = [100, 900, 64, 1500, 333]
    announce(f"varlen moving max d={d} lengths={lengths}")
    H = 2
    parts = [workloads.moving_max_inputs(1, H, n, d, "bf16", seed=n, rate=0.5) for n in lengths]
    # [1, H, n, d] per sequence -> packed [T, H, d]
    q, k, v = (torch.cat([p[i][0].transpose(0, 1) for p in parts], dim=0).contiguous()
               for i in range(3))
    cu = workloads.cu_seqlens_of(lengths)
    scale = d ** -0.5
    o, lse = run_varlen(q, k, v, cu, max(lengths), scale, dev)
    O_ref, L_ref = oracle.attention_varlen(q, k, v, cu, scale)
    tol_o, tol_l = TOL["bf16"]
    assert_close("O", f64(o), O_ref, tol_o)
    assert_close("L", f64(lse), L_ref, tol_l)
