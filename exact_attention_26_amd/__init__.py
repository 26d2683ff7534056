"""MI355X (gfx950) FlashAttention-2 forward (full and banded) and backward, and the fused
dropout + residual + LayerNorm/RMSNorm op: thin Python binding of libfa.so.

The C ABI (include/fa.h) is the product; this module only marshals
arguments. Every step of the forward and backward runs in the library's
HIP kernels.
PyTorch supplies device memory and the current stream.

    fa_fwd(Q, K, V, O, L, B, H, N, d, scale, dtype, stream)        -> None
    fa_fwd_varlen(Q, K, V, O, L, cu_seqlens, nseq, total_tokens,
                  max_seqlen, H, d, scale, dtype, stream)           -> None
    fa_fwd_banded(Q, K, V, O, L, B, H, N, d, window, scale, dtype,
                  stream)                                           -> None
    fa_fwd_kv_outer(Q, K, V, O, L, acc, B, H, N, d, q_groups, scale,
                    dtype, stream)                                  -> None
    fa_bwd(Q, K, V, O, dO, L, dQ, dK, dV, delta, B, H, N, d, scale,
           dtype, stream)                                           -> None
    fa_bwd_noalloc(Q, K, V, O, dO, L, dQ, dK, dV, B, H, N, d, scale,
                   dtype, stream)                                   -> None
    fa_dropout_add_norm(x0, x1, residual, gamma0, beta0, gamma1, beta1,
                        y0, y1, z, mean, rstd, mask, rows, hidden,
                        dropout_p, seed, offset, eps, norm, dtype,
                        stream)                                     -> None
    fa_strerror(status) -> str,  fa_version() -> int

take raw integers (device addresses, sizes, the stream handle) exactly as
the C functions do and raise ``FaError`` on a non-zero status.

    forward(q, k, v, scale=None)                    -> (o, lse)
    forward_varlen(q, k, v, cu_seqlens, max_seqlen, scale=None) -> (o, lse)
    forward_banded(q, k, v, window, scale=None)     -> (o, lse)
    forward_kv_outer(q, k, v, q_groups, scale=None) -> (o, lse)
    backward(q, k, v, o, do, lse, scale=None)       -> (dq, dk, dv)
    dropout_add_norm(x0, gamma0, ...)               -> dict of outputs

take torch tensors on a GPU, allocate the outputs with torch.empty and call
the entry points above on the current stream.

If libfa.so is missing or cannot be loaded, every call raises: there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

__all__ = [
    "FA_F32", "FA_F16", "FA_BF16", "FaError", "LIB_PATH", "load", "fa_fwd", "fa_fwd_varlen",
    "fa_strerror", "fa_version", "forward", "forward_varlen", "EXPORTED_SYMBOLS", "fa_bwd",
    "fa_bwd_noalloc", "load_library", "POISON_LIB_PATH", "TRACE_LIB_PATH", "fa_debug_fwd_trace",
    "backward", "fa_fwd_banded", "forward_banded", "fa_fwd_kv_outer", "forward_kv_outer",
    "fa_dropout_add_norm", "dropout_add_norm", "FA_NORM_LAYER", "FA_NORM_RMS",
]

FA_F32, FA_F16, FA_BF16 = 0, 1, 2
FA_NORM_LAYER, FA_NORM_RMS = 0, 1
STATUS = {
    0: "FA_OK", -1: "FA_ERR_NULL", -2: "FA_ERR_SHAPE", -3: "FA_ERR_HEADDIM", -4: "FA_ERR_DTYPE",
    -5: "FA_ERR_ALIGN", -6: "FA_ERR_ALIAS", -7: "FA_ERR_LAUNCH", -8: "FA_ERR_SCALE",
    -9: "FA_ERR_SIZE", -10: "FA_ERR_ARG", -11: "FA_ERR_SCRATCH", -12: "FA_ERR_UNSUPPORTED",
}
EXPORTED_SYMBOLS = ("fa_fwd", "fa_fwd_varlen", "fa_fwd_banded", "fa_fwd_kv_outer", "fa_bwd",
                    "fa_bwd_noalloc", "fa_dropout_add_norm", "fa_debug_fwd_trace", "fa_strerror",
                    "fa_version")
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")
POISON_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa_lds_poison.so")
TRACE_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa_trace.so")

_lib = None
_lib_lock = threading.Lock()


class FaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status
        self.name = STATUS.get(status, "unknown")


def load() -> ctypes.CDLL:
    """Load libfa.so once and declare its C signatures (thread-safe)."""
    if _lib is not None:
        return _lib
    with _lib_lock:
        return _lib if _lib is not None else _load_locked()


def _load_locked() -> ctypes.CDLL:
    global _lib
    _lib = load_library(LIB_PATH)
    return _lib


def load_library(path: str) -> ctypes.CDLL:
    """Load a build of the library at `path` and declare its C signatures.
    load() uses it for libfa.so; tests use it for the debug variant
    libfa_lds_poison.so (POISON_LIB_PATH) and libfa_trace.so (TRACE_LIB_PATH)."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m exact_attention_26_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, i32, vp]
    lib.fa_fwd.restype = i32
    lib.fa_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp]
    lib.fa_fwd_varlen.restype = i32
    lib.fa_fwd_banded.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp]
    lib.fa_fwd_banded.restype = i32
    lib.fa_fwd_kv_outer.argtypes = [vp] * 6 + [i32, i32, i32, i32, i32, f32, i32, vp]
    lib.fa_fwd_kv_outer.restype = i32
    u64 = ctypes.c_uint64
    lib.fa_dropout_add_norm.argtypes = ([vp] * 13 + [i32, i32, f32, u64, u64, f32, i32, i32, vp])
    lib.fa_dropout_add_norm.restype = i32
    lib.fa_bwd.argtypes = [vp] * 10 + [i32, i32, i32, i32, f32, i32, vp]
    lib.fa_bwd.restype = i32
    lib.fa_bwd_noalloc.argtypes = [vp] * 9 + [i32, i32, i32, i32, f32, i32, vp]
    lib.fa_bwd_noalloc.restype = i32
    lib.fa_debug_fwd_trace.argtypes = [i32, vp]
    lib.fa_debug_fwd_trace.restype = i32
    lib.fa_strerror.argtypes = [i32]
    lib.fa_strerror.restype = ctypes.c_char_p
    lib.fa_version.argtypes = []
    lib.fa_version.restype = i32
    return lib


def fa_strerror(status: int) -> str:
    return load().fa_strerror(int(status)).decode()


def fa_version() -> int:
    return int(load().fa_version())


def _check(status: int) -> None:
    if status != 0:
        raise FaError(status, fa_strerror(status))


def fa_fwd(Q, K, V, O, L, B, H, N, d, scale, dtype, stream) -> None:
    _check(load().fa_fwd(Q, K, V, O, L, int(B), int(H), int(N), int(d), float(scale), int(dtype),
                         stream))


def fa_fwd_varlen(Q, K, V, O, L, cu_seqlens, nseq, total_tokens, max_seqlen, H, d, scale, dtype,
                  stream) -> None:
    _check(load().fa_fwd_varlen(Q, K, V, O, L, cu_seqlens, int(nseq), int(total_tokens),
                                int(max_seqlen), int(H), int(d), float(scale), int(dtype), stream))


def fa_fwd_banded(Q, K, V, O, L, B, H, N, d, window, scale, dtype, stream) -> None:
    _check(load().fa_fwd_banded(Q, K, V, O, L, int(B), int(H), int(N), int(d), int(window),
                                float(scale), int(dtype), stream))


def fa_fwd_kv_outer(Q, K, V, O, L, acc, B, H, N, d, q_groups, scale, dtype, stream) -> None:
    _check(load().fa_fwd_kv_outer(Q, K, V, O, L, acc, int(B), int(H), int(N), int(d),
                                  int(q_groups), float(scale), int(dtype), stream))


def fa_dropout_add_norm(x0, x1, residual, gamma0, beta0, gamma1, beta1, y0, y1, z, mean, rstd,
                        mask, rows, hidden, dropout_p, seed, offset, eps, norm, dtype,
                        stream) -> None:
    _check(load().fa_dropout_add_norm(x0, x1, residual, gamma0, beta0, gamma1, beta1, y0, y1, z,
                                      mean, rstd, mask, int(rows), int(hidden), float(dropout_p),
                                      int(seed), int(offset), float(eps), int(norm), int(dtype),
                                      stream))


def fa_bwd(Q, K, V, O, dO, L, dQ, dK, dV, delta, B, H, N, d, scale, dtype, stream) -> None:
    _check(load().fa_bwd(Q, K, V, O, dO, L, dQ, dK, dV, delta, int(B), int(H), int(N), int(d),
                         float(scale), int(dtype), stream))


def fa_bwd_noalloc(Q, K, V, O, dO, L, dQ, dK, dV, B, H, N, d, scale, dtype, stream) -> None:
    _check(load().fa_bwd_noalloc(Q, K, V, O, dO, L, dQ, dK, dV, int(B), int(H), int(N), int(d),
                                 float(scale), int(dtype), stream))


def fa_debug_fwd_trace(workgroup, trace_buffer, lib=None) -> None:
    """Phase trace of the 16-bit forward; implemented by the debug build
    libfa_trace.so only (pass it as `lib`), FaError(FA_ERR_UNSUPPORTED) from
    the product library."""
    _check((lib or load()).fa_debug_fwd_trace(int(workgroup), trace_buffer))


# ---------------------------------------------------------------------------
# torch conveniences (argument marshalling only)
# ---------------------------------------------------------------------------
def _dtype_code(t) -> int:
    import torch
    codes = {torch.float32: FA_F32, torch.float16: FA_F16, torch.bfloat16: FA_BF16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}; expected float32, float16 or bfloat16")
    return codes[t.dtype]


def _stream_handle(device) -> int:
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def _require(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _inputs_on_one_gpu(*ts) -> None:
    """Every input tensor a kernel reads: a contiguous tensor on one GPU (a host
    or another device's address would be dereferenced as this GPU's memory)."""
    _require(all(t.is_cuda for t in ts), "inputs must be GPU tensors")
    _require(len({t.device for t in ts}) == 1, "inputs must be on the same GPU")
    _require(all(t.is_contiguous() for t in ts), "inputs must be contiguous")


def _check_buffer(t, shape, dtype, device, name: str):
    """A caller-supplied output or scratch buffer. The kernels write exactly
    `shape` elements of `dtype` through its address, so a smaller, strided,
    differently typed or foreign-device buffer is rejected rather than
    overrun."""
    _require(t.is_cuda and t.device == device, f"{name} must be on {device}")
    _require(tuple(t.shape) == tuple(shape),
             f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    _require(t.dtype == dtype, f"{name} must be {dtype}, got {t.dtype}")
    _require(t.is_contiguous(), f"{name} must be contiguous")
    return t


def _out_or_new(t, shape, dtype, device, name: str):
    import torch
    if t is None:
        return torch.empty(tuple(shape), dtype=dtype, device=device)
    return _check_buffer(t, shape, dtype, device, name)


def forward(q, k, v, scale: float | None = None, out=None, lse=None):
    """Dense forward on contiguous [B, H, N, d] tensors; returns (o, lse[B,H,N] fp32)."""
    import torch
    _require(q.dim() == 4 and q.shape == k.shape == v.shape, "q, k, v must share shape [B,H,N,d]")
    _require(q.dtype == k.dtype == v.dtype, "q, k, v must share a dtype")
    _inputs_on_one_gpu(q, k, v)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = _out_or_new(out, q.shape, q.dtype, q.device, "out")
    L = _out_or_new(lse, (B, H, N), torch.float32, q.device, "lse")
    fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), L.data_ptr(), B, H, N, d,
           scale, _dtype_code(q), _stream_handle(q.device))
    return o, L


def forward_banded(q, k, v, window: int, scale: float | None = None, out=None, lse=None):
    """Dense banded forward on contiguous [B, H, N, d] fp16/bf16 tensors: row r
    attends to keys c with |r - c| <= window. Returns (o, lse[B,H,N] fp32)."""
    import torch
    _require(q.dim() == 4 and q.shape == k.shape == v.shape, "q, k, v must share shape [B,H,N,d]")
    _require(q.dtype == k.dtype == v.dtype, "q, k, v must share a dtype")
    _inputs_on_one_gpu(q, k, v)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = _out_or_new(out, q.shape, q.dtype, q.device, "out")
    L = _out_or_new(lse, (B, H, N), torch.float32, q.device, "lse")
    fa_fwd_banded(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), L.data_ptr(), B, H, N,
                  d, window, scale, _dtype_code(q), _stream_handle(q.device))
    return o, L


def forward_kv_outer(q, k, v, q_groups: int = 16, scale: float | None = None, out=None,
                     lse=None, acc=None):
    """Dense forward in the K/V-outer order on contiguous [B, H, N, d] fp16/bf16
    tensors (same O and L as forward()); acc is the fp32 scratch of
    B*H*N*(d+2) floats. Returns (o, lse[B,H,N] fp32)."""
    import torch
    _require(q.dim() == 4 and q.shape == k.shape == v.shape, "q, k, v must share shape [B,H,N,d]")
    _require(q.dtype == k.dtype == v.dtype, "q, k, v must share a dtype")
    _inputs_on_one_gpu(q, k, v)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = _out_or_new(out, q.shape, q.dtype, q.device, "out")
    L = _out_or_new(lse, (B, H, N), torch.float32, q.device, "lse")
    acc = _out_or_new(acc, (B * H * N * (d + 2),), torch.float32, q.device, "acc")
    fa_fwd_kv_outer(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), L.data_ptr(),
                    acc.data_ptr(), B, H, N, d, q_groups, scale, _dtype_code(q),
                    _stream_handle(q.device))
    return o, L


def forward_varlen(q, k, v, cu_seqlens, max_seqlen: int, scale: float | None = None, out=None,
                   lse=None):
    """Packed forward on contiguous [T, H, d] tensors with int32 cu_seqlens[nseq+1]
    on the same device; returns (o, lse[H,T] fp32)."""
    import torch
    _require(q.dim() == 3 and q.shape == k.shape == v.shape, "q, k, v must share shape [T,H,d]")
    _require(q.dtype == k.dtype == v.dtype, "q, k, v must share a dtype")
    _require(cu_seqlens.dtype == torch.int32 and cu_seqlens.dim() == 1,
             "cu_seqlens must be a 1-D int32 tensor")
    _inputs_on_one_gpu(q, k, v, cu_seqlens)
    T, H, d = q.shape
    nseq = cu_seqlens.numel() - 1
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = _out_or_new(out, q.shape, q.dtype, q.device, "out")
    L = _out_or_new(lse, (H, T), torch.float32, q.device, "lse")
    fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), L.data_ptr(),
                  cu_seqlens.data_ptr(), nseq, T, int(max_seqlen), H, d, scale, _dtype_code(q),
                  _stream_handle(q.device))
    return o, L


def backward(q, k, v, o, do, lse, scale: float | None = None, dq=None, dk=None, dv=None,
             delta=None):
    """Dense backward on contiguous [B, H, N, d] tensors; o and lse as forward()
    returned them for the same q, k, v and scale. Returns (dq, dk, dv)."""
    import torch
    _require(q.dim() == 4 and q.shape == k.shape == v.shape == o.shape == do.shape,
             "q, k, v, o, do must share shape [B,H,N,d]")
    _require(q.dtype == k.dtype == v.dtype == o.dtype == do.dtype,
             "q, k, v, o, do must share a dtype")
    _inputs_on_one_gpu(q, k, v, o, do, lse)
    B, H, N, d = q.shape
    _require(lse.dtype == torch.float32 and tuple(lse.shape) == (B, H, N),
             "lse must be float32 [B,H,N]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = _out_or_new(dq, q.shape, q.dtype, q.device, "dq")
    dk = _out_or_new(dk, q.shape, q.dtype, q.device, "dk")
    dv = _out_or_new(dv, q.shape, q.dtype, q.device, "dv")
    delta = _out_or_new(delta, (B, H, N), torch.float32, q.device, "delta")
    fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
           dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(), B, H, N, d, scale,
           _dtype_code(q), _stream_handle(q.device))
    return dq, dk, dv


def dropout_add_norm(x0, gamma0, beta0=None, residual=None, x1=None, gamma1=None, beta1=None,
                     p: float = 0.0, seed: int = 0, offset: int = 0, eps: float = 1e-5,
                     rms: bool = False, prenorm: bool = True, stats: bool = True,
                     return_mask: bool = False, out=None):
    """Fused dropout + residual + LayerNorm/RMSNorm on contiguous [rows, hidden]
    fp16/bf16 GPU tensors (any leading shape is flattened into rows). Returns a
    dict: y0, y1 (None without gamma1), z (None unless prenorm), mean (LayerNorm
    only) and rstd (None unless stats), mask (uint8, None unless return_mask).
    `out` may be a dict returned by an earlier call with the same arguments:
    its tensors are written again instead of allocating new ones."""
    import torch
    hidden = x0.shape[-1]
    rows = x0.numel() // hidden if hidden else 0
    ts = [t for t in (x0, x1, residual) if t is not None]
    ws = [t for t in (gamma0, beta0, gamma1, beta1) if t is not None]
    _require(all(t.shape == x0.shape for t in ts), "x0, x1, residual must share a shape")
    _require(all(t.numel() == hidden for t in ws), "gamma/beta must have `hidden` elements")
    _require(all(t.dtype == x0.dtype for t in ts + ws), "all tensors must share a dtype")
    _inputs_on_one_gpu(*ts, *ws)
    if out is not None:
        # The same outputs a call with these arguments allocates, and no others:
        # the kernel writes each non-null one and skips the null ones.
        want = {"y0": (x0.shape, x0.dtype), "y1": (x0.shape, x0.dtype) if gamma1 is not None else None,
                "z": (x0.shape, x0.dtype) if prenorm else None,
                "mean": ((rows,), torch.float32) if stats and not rms else None,
                "rstd": ((rows,), torch.float32) if stats else None,
                "mask": ((2 if x1 is not None else 1, rows, hidden), torch.uint8)
                if return_mask else None}
        for name, spec in want.items():
            t = out.get(name)
            if spec is None:
                _require(t is None, f"out[{name!r}] must be None for these arguments")
            else:
                _require(t is not None, f"out[{name!r}] is missing")
                _check_buffer(t, spec[0], spec[1], x0.device, f"out[{name!r}]")
        o = out
        fa_dropout_add_norm(*(None if t is None else t.data_ptr() for t in
                              (x0, x1, residual, gamma0, beta0, gamma1, beta1, o["y0"], o["y1"],
                               o["z"], o["mean"], o["rstd"], o["mask"])),
                            rows, hidden, p, seed, offset, eps,
                            FA_NORM_RMS if rms else FA_NORM_LAYER, _dtype_code(x0),
                            _stream_handle(x0.device))
        return out
    y0 = torch.empty_like(x0)
    y1 = torch.empty_like(x0) if gamma1 is not None else None
    z = torch.empty_like(x0) if prenorm else None
    dev = x0.device
    mean = torch.empty(rows, dtype=torch.float32, device=dev) if stats and not rms else None
    rstd = torch.empty(rows, dtype=torch.float32, device=dev) if stats else None
    mask = (torch.empty((2 if x1 is not None else 1, rows, hidden), dtype=torch.uint8, device=dev)
            if return_mask else None)
    ptr = lambda t: None if t is None else t.data_ptr()
    fa_dropout_add_norm(ptr(x0), ptr(x1), ptr(residual), ptr(gamma0), ptr(beta0), ptr(gamma1),
                        ptr(beta1), ptr(y0), ptr(y1), ptr(z), ptr(mean), ptr(rstd), ptr(mask),
                        rows, hidden, p, seed, offset, eps, FA_NORM_RMS if rms else FA_NORM_LAYER,
                        _dtype_code(x0), _stream_handle(dev))
    return {"y0": y0, "y1": y1, "z": z, "mean": mean, "rstd": rstd, "mask": mask}
