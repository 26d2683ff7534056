"""Race check of the LDS pipelines: parity on the debug build
libfa_lds_poison.so, in which every LDS DMA copy's destination is filled
with NaN (and that fill awaited) right before the copy is issued.

The kernels stream K/V (forward) and Q/dO/L/D or K/V (backward) through
multi-stage LDS buffers filled by asynchronous copies; a stage may be read
only after its copy has completed (vmcnt) and a barrier has published it,
and refilled only after every wave has finished reading it. A missing wait
or barrier would let a wave read a stage that is not yet (or no longer)
the tile it expects. In the normal build such a read returns stale data
from an older tile, which might even pass a tolerance; in the poisoned
build it returns NaN, which the outputs carry and the checks below reject.
The pages place a barrier after every phase of their kernel ("Kernel
visualization: Flash Attention 2", "Iteration j = 0"); this checks the
equivalent ordering of the asynchronous pipeline.

Cases: dense forward on both sides of the 4-/8-wave switch with ragged
tails (every peeled phase of the three-stage loop), packed batches on the
4- and 8-wave kernels, banded windows (tile skipping), inputs whose max
keeps moving, and the backward's two LDS pipelines. Each is compared with
the float64 oracle at the parity tolerances, and with the normal build
bit for bit (the fill changes timing only).
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

CODE = {torch.bfloat16: fa.FA_BF16, torch.float16: fa.FA_F16}
_poison = None


def poison_lib():
    global _poison
    if _poison is None:
        _poison = fa.load_library(fa.POISON_LIB_PATH)
    return _poison


def _stream(t):
    return torch.cuda.current_stream(t.device).cuda_stream


def fwd(lib, q, k, v, scale):
    B, H, N, d = q.shape
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=q.device)
    st = lib.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H,
                    N, d, scale, CODE[q.dtype], _stream(q))
    assert st == 0, fa.fa_strerror(st)
    torch.cuda.synchronize()
    return o, lse


def fwd_varlen(lib, q, k, v, cu, max_seqlen, scale):
    T, H, d = q.shape
    o = torch.full_like(q, float("nan"))
    lse = torch.full((H, T), float("nan"), dtype=torch.float32, device=q.device)
    st = lib.fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                           cu.data_ptr(), cu.numel() - 1, T, max_seqlen, H, d, scale,
                           CODE[q.dtype], _stream(q))
    assert st == 0, fa.fa_strerror(st)
    torch.cuda.synchronize()
    return o, lse


def fwd_banded(lib, q, k, v, window, scale):
    B, H, N, d = q.shape
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=q.device)
    st = lib.fa_fwd_banded(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                           B, H, N, d, window, scale, CODE[q.dtype], _stream(q))
    assert st == 0, fa.fa_strerror(st)
    torch.cuda.synchronize()
    return o, lse


def bwd(lib, q, k, v, o, do, lse, scale):
    B, H, N, d = q.shape
    dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
    delta = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=q.device)
    st = lib.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                    lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(),
                    B, H, N, d, scale, CODE[q.dtype], _stream(q))
    assert st == 0, fa.fa_strerror(st)
    torch.cuda.synchronize()
    return dq, dk, dv


def _same(tag, got, want):
    for name, g, w in zip(("O", "L"), got, want):
        assert torch.equal(g, w), f"{tag}: {name} of the poisoned build differs from the normal one"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N,dtype,inputs", [(65, "bf16", "normal"), (1000, "fp16", "normal"),
                                            (2049, "bf16", "normal"), (2200, "fp16", "normal"),
                                            (2300, "bf16", "normal"), (4100, "bf16", "normal"),
                                            (1500, "bf16", "moving_max"),
                                            (2500, "bf16", "moving_max")])
def test_poisoned_dense_forward(d, N, dtype, inputs):
    dev = device()
    lib = poison_lib()
    announce(f"poisoned dense forward d={d} N={N} {dtype} {inputs}")
    B, H = 1, 2
    if inputs == "normal":
        q, k, v = workloads.dense_inputs(B, H, N, d, dtype, seed=N + d)
    else:
        q, k, v = workloads.moving_max_inputs(B, H, N, d, dtype, seed=N + d, rate=0.5)
    scale = d ** -0.5
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o, lse = fwd(lib, qd, kd, vd, scale)
    O_ref, L_ref = oracle.attention_dense(q, k, v, scale)
    tol_o, tol_l = TOL[dtype]
    assert_close("O", f64(o), O_ref, tol_o)
    assert_close("L", f64(lse), L_ref, tol_l)
    _same("dense", (o, lse), fwd(fa.load(), qd, kd, vd, scale))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("lengths", [[1, 63, 64, 65, 130, 4200, 129, 700, 192],
                                     [300, 64, 2048, 1, 999, 128]])
def test_poisoned_packed_forward(d, lengths):
    dev = device()
    lib = poison_lib()
    announce(f"poisoned packed forward d={d} lengths={lengths}")
    H = 2
    q, k, v, cu = workloads.varlen_inputs(lengths, H, d, "bf16", seed=d + len(lengths))
    scale = d ** -0.5
    qd, kd, vd, cud = q.to(dev), k.to(dev), v.to(dev), cu.to(dev)
    o, lse = fwd_varlen(lib, qd, kd, vd, cud, max(lengths), scale)
    O_ref, L_ref = oracle.attention_varlen(q, k, v, cu, scale)
    tol_o, tol_l = TOL["bf16"]
    assert_close("O", f64(o), O_ref, tol_o)
    assert_close("L", f64(lse), L_ref, tol_l)
    _same("packed", (o, lse), fwd_varlen(fa.load(), qd, kd, vd, cud, max(lengths), scale))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N,window", [(1000, 0), (1500, 100), (2600, 700), (3000, 2500),
                                      (2300, 5000)])
def test_poisoned_banded_forward(d, N, window):
    dev = device()
    lib = poison_lib()
    announce(f"poisoned banded forward d={d} N={N} window={window}")
    q, k, v = workloads.dense_inputs(1, 2, N, d, "bf16", seed=N + window)
    scale = d ** -0.5
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o, lse = fwd_banded(lib, qd, kd, vd, window, scale)
    O_ref, L_ref = oracle.attention_banded_dense(q, k, v, scale, window)
    tol_o, tol_l = TOL["bf16"]
    assert_close("O", f64(o), O_ref, tol_o)
    assert_close("L", f64(lse), L_ref, tol_l)
    _same("banded", (o, lse), fwd_banded(fa.load(), qd, kd, vd, window, scale))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [100, 333, 1000])
def test_poisoned_backward(d, N):
    dev = device()
    lib = poison_lib()
    announce(f"poisoned backward d={d} N={N}")
    B, H = 1, 2
    q, k, v, do = workloads.dense_bwd_inputs(B, H, N, d, "bf16", seed=N + d)
    scale = d ** -0.5
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    o, lse = fwd(fa.load(), qd, kd, vd, scale)
    got = bwd(lib, qd, kd, vd, o, dod, lse, scale)
    # The oracle from the same O and L the backward was given.
    want = oracle.attention_backward_lse_dense(q, k, v, f64(o), do, f64(lse), scale)
    floor = 0.1 * max(float(np.max(np.abs(w))) for w in want)
    for name, g, w in zip(("dQ", "dK", "dV"), got, want):
        bound = 1e-2 * max(float(np.max(np.abs(w))), floor)
        assert_close(name, f64(g), w, bound)
    normal = bwd(fa.load(), qd, kd, vd, o, dod, lse, scale)
    for name, g, w in zip(("dQ", "dK", "dV"), got, normal):
        assert torch.equal(g, w), f"backward {name}: poisoned build differs from the normal one"
