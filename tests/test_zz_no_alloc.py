"""fa_bwd_noalloc through the C ABI against fa_bwd: the same kernels with D in
the library's static scratch array instead of a caller buffer, so dQ, dK, dV
must agree bit for bit. Two calls in a row, the second smaller, so the second
reuses the scratch the first left behind; then the free device memory is
checked unchanged across further calls (the entry point allocates nothing)."""
import pytest
import torch

import exact_attention_26_amd as fa
import workloads
from gpu_helpers import announce, device

pytestmark = pytest.mark.gpu


def _problem(B, H, N, d, dtype, seed, dev):
    q, k, v, do = workloads.dense_bwd_inputs(B, H, N, d, dtype, seed=seed)
    q, k, v, do = (t.to(dev) for t in (q, k, v, do))
    o, lse = fa.forward(q, k, v)
    return q, k, v, do, o, lse


def _grads(entry, q, k, v, do, o, lse, delta=None):
    B, H, N, d = q.shape
    dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
    stream = torch.cuda.current_stream(q.device).cuda_stream
    args = [q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr()]
    if delta is not None:
        args.append(delta.data_ptr())
    code = fa.FA_BF16 if q.dtype == torch.bfloat16 else fa.FA_F16
    entry(*args, B, H, N, d, d ** -0.5, code, stream)
    torch.cuda.synchronize()
    return dq, dk, dv


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_bwd_noalloc_matches_bwd(dtype):
    dev = device()
    # (B, H, N, d): the second call is smaller than the first
    for i, (B, H, N, d) in enumerate([(2, 4, 1000, 128), (1, 3, 333, 64)]):
        announce(f"fa_bwd_noalloc vs fa_bwd {dtype} B={B} H={H} N={N} d={d} call {i}")
        q, k, v, do, o, lse = _problem(B, H, N, d, dtype, seed=7 + i, dev=dev)
        delta = torch.empty(B, H, N, dtype=torch.float32, device=dev)
        want = _grads(fa.fa_bwd, q, k, v, do, o, lse, delta)
        got = _grads(fa.fa_bwd_noalloc, q, k, v, do, o, lse)
        for name, g, w in zip(("dQ", "dK", "dV"), got, want):
            assert torch.isfinite(g.float()).all(), f"{name}: non-finite (call {i})"
            assert torch.equal(g, w), (f"{name}: max |noalloc - bwd| = "
                                       f"{(g.float() - w.float()).abs().max().item()} (call {i})")


def test_bwd_noalloc_allocates_nothing():
    dev = device()
    announce("fa_bwd_noalloc allocates no device memory")
    q, k, v, do, o, lse = _problem(1, 2, 500, 64, "bf16", seed=3, dev=dev)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    stream = torch.cuda.current_stream(dev).cuda_stream
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), 1, 2, 500, 64, 0.125, fa.FA_BF16, stream)
    fa.fa_bwd_noalloc(*args)  # first call on this device: code load and scratch lookup
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info(dev)
    for _ in range(3):
        fa.fa_bwd_noalloc(*args)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info(dev)
    assert free1 == free0
