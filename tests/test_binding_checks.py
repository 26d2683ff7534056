"""The binding's checks of caller-supplied tensors: inputs on one GPU, and
output / scratch buffers of exactly the shape, dtype and layout the kernels
write. Every case raises ValueError before anything is enqueued."""
import pytest
import torch

import exact_attention_26_amd as fa
from gpu_helpers import announce, device

pytestmark = pytest.mark.gpu


def _dense(dev, B=1, H=2, N=70, d=64, dtype=torch.bfloat16):
    return [torch.zeros(B, H, N, d, dtype=dtype, device=dev) for _ in range(3)]


@pytest.mark.parametrize("case", ["out_shape", "out_dtype", "out_strided", "lse_shape",
                                  "lse_dtype", "out_on_host", "k_on_host"])
def test_forward_rejects_bad_tensors(case):
    dev = device()
    announce(f"binding check: forward {case}")
    q, k, v = _dense(dev)
    kw = {}
    if case == "out_shape":
        kw["out"] = torch.empty(1, 2, 69, 64, dtype=q.dtype, device=dev)
    elif case == "out_dtype":
        kw["out"] = torch.empty_like(q, dtype=torch.float16)
    elif case == "out_strided":
        kw["out"] = torch.empty(1, 2, 64, 70, dtype=q.dtype, device=dev).transpose(2, 3)
    elif case == "lse_shape":
        kw["lse"] = torch.empty(1, 2, 69, dtype=torch.float32, device=dev)
    elif case == "lse_dtype":
        kw["lse"] = torch.empty(1, 2, 70, dtype=torch.bfloat16, device=dev)
    elif case == "out_on_host":
        kw["out"] = torch.empty(q.shape, dtype=q.dtype)
    elif case == "k_on_host":
        k = k.cpu()
    with pytest.raises(ValueError):
        fa.forward(q, k, v, 0.125, **kw)


@pytest.mark.parametrize("case", ["k_on_host", "v_on_host", "cu_on_host", "out_shape", "lse_shape"])
def test_forward_varlen_rejects_bad_tensors(case):
    dev = device()
    announce(f"binding check: forward_varlen {case}")
    q, k, v = (torch.zeros(100, 2, 64, dtype=torch.bfloat16, device=dev) for _ in range(3))
    cu = torch.tensor([0, 60, 100], dtype=torch.int32, device=dev)
    kw = {}
    if case == "k_on_host":
        k = k.cpu()
    elif case == "v_on_host":
        v = v.cpu()
    elif case == "cu_on_host":
        cu = cu.cpu()
    elif case == "out_shape":
        kw["out"] = torch.empty(99, 2, 64, dtype=q.dtype, device=dev)
    elif case == "lse_shape":
        kw["lse"] = torch.empty(100, 2, dtype=torch.float32, device=dev)
    with pytest.raises(ValueError):
        fa.forward_varlen(q, k, v, cu, 60, 0.125, **kw)


def test_banded_kv_outer_and_backward_reject_bad_buffers():
    dev = device()
    announce("binding check: banded, kv_outer, backward buffers")
    q, k, v = _dense(dev)
    with pytest.raises(ValueError):
        fa.forward_banded(q, k, v, 8, 0.125, out=torch.empty(1, 2, 70, 32, dtype=q.dtype, device=dev))
    with pytest.raises(ValueError):
        fa.forward_kv_outer(q, k, v, 2, 0.125,
                            acc=torch.empty(1 * 2 * 70 * 66 - 1, dtype=torch.float32, device=dev))
    lse = torch.zeros(1, 2, 70, dtype=torch.float32, device=dev)
    for name in ("dq", "dk", "dv"):
        with pytest.raises(ValueError):
            fa.backward(q, k, v, q, q, lse, 0.125,
                        **{name: torch.empty(1, 2, 70, 63, dtype=q.dtype, device=dev)})
    with pytest.raises(ValueError):
        fa.backward(q, k, v, q, q, lse, 0.125,
                    delta=torch.empty(1, 2, 70, dtype=torch.float16, device=dev))


def test_norm_rejects_a_mismatched_out_dict():
    dev = device()
    announce("binding check: dropout_add_norm out dict")
    x = torch.zeros(4, 64, dtype=torch.bfloat16, device=dev)
    g = torch.ones(64, dtype=torch.bfloat16, device=dev)
    out = fa.dropout_add_norm(x, g, stats=True, prenorm=True)
    torch.cuda.synchronize()
    assert fa.dropout_add_norm(x, g, stats=True, prenorm=True, out=out) is out  # same arguments
    with pytest.raises(ValueError):  # asks for a mask the dict does not hold
        fa.dropout_add_norm(x, g, stats=True, prenorm=True, return_mask=True, out=out)
    bad = dict(out, y0=torch.empty(4, 32, dtype=torch.bfloat16, device=dev))
    with pytest.raises(ValueError):
        fa.dropout_add_norm(x, g, stats=True, prenorm=True, out=bad)
