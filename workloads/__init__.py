"""Seeded synthetic inputs for the attention forward, shared by the tests,
the benchmark and the smoke check.

This module holds no attention arithmetic: it only draws random numbers and
rounds them to the storage dtype. Both the float64 oracle and the HIP path
receive the same rounded tensors, so their results can be compared element
by element.

Workloads (sizes and value distributions are those of the five target
configurations; every draw is seeded, per workload, with
``numpy.random.default_rng(seed)``):

  single_head_fp32   B=1  H=1  N=256  d=64  fp32  Q,K,V ~ N(0,1)        scale 1/8
  short_bf16         B=4  H=16 N=1024 d=64  bf16  Q,K,V ~ N(0,1)        scale 1/8
  long_bf16          B=2  H=32 N=8192 d=128 bf16  Q,K,V ~ N(0,1)        scale 1/sqrt(128)
  large_logit_fp16   B=16 H=16 N=512  d=64  fp16  Q,K ~ N(0,4^2), V ~ U[-1,1]
                     scale 1/8 ("a") and 1.0 ("b")
  varlen_bf16        32 sequences, lengths ~ U{64..4096}, H=16 d=128 bf16,
                     Q,K,V ~ N(0,1), packed [T,H,d], scale 1/sqrt(128)

Draw order: for varlen the lengths come first, then Q, K, V; for dense
workloads Q, K, V. Values are drawn as float32 and rounded once to the
storage dtype with torch (round-to-nearest-even).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

DTYPES = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str
    d: int
    scale: float
    B: int = 0
    H: int = 0
    N: int = 0
    # varlen only
    nseq: int = 0
    min_len: int = 0
    max_len: int = 0
    qk_std: float = 1.0
    v_uniform: bool = False
    seed: int = 0

    @property
    def varlen(self) -> bool:
        return self.nseq > 0


WORKLOADS = {
    "single_head_fp32": Workload("single_head_fp32", "fp32", 64, 1.0 / 8.0, B=1, H=1, N=256),
    "short_bf16": Workload("short_bf16", "bf16", 64, 1.0 / 8.0, B=4, H=16, N=1024),
    "long_bf16": Workload("long_bf16", "bf16", 128, 1.0 / math.sqrt(128.0), B=2, H=32, N=8192),
    "large_logit_fp16_a": Workload("large_logit_fp16_a", "fp16", 64, 0.125, B=16, H=16, N=512,
                                   qk_std=4.0, v_uniform=True),
    "large_logit_fp16_b": Workload("large_logit_fp16_b", "fp16", 64, 1.0, B=16, H=16, N=512,
                                   qk_std=4.0, v_uniform=True),
    "varlen_bf16": Workload("varlen_bf16", "bf16", 128, 1.0 / math.sqrt(128.0), H=16,
                            nseq=32, min_len=64, max_len=4096),
}


def _round(a: np.ndarray, dtype: str) -> torch.Tensor:
    """float32 numpy -> torch tensor of the storage dtype (RNE), on the CPU."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DTYPES[dtype])


def draw_qkv(rng: np.random.Generator, shape, dtype: str, qk_std: float = 1.0,
             v_uniform: bool = False):
    """Q, K, V of `shape`, drawn in that order from `rng`, rounded to dtype."""
    q = rng.standard_normal(shape, dtype=np.float32)
    if qk_std != 1.0:
        q *= np.float32(qk_std)
    k = rng.standard_normal(shape, dtype=np.float32)
    if qk_std != 1.0:
        k *= np.float32(qk_std)
    if v_uniform:
        v = rng.uniform(-1.0, 1.0, size=shape).astype(np.float32)
    else:
        v = rng.standard_normal(shape, dtype=np.float32)
    return _round(q, dtype), _round(k, dtype), _round(v, dtype)


def dense_inputs(B: int, H: int, N: int, d: int, dtype: str, seed: int = 0,
                 qk_std: float = 1.0, v_uniform: bool = False):
    """Contiguous [B,H,N,d] Q, K, V (CPU tensors of `dtype`)."""
    rng = np.random.default_rng(seed)
    return draw_qkv(rng, (B, H, N, d), dtype, qk_std, v_uniform)


def moving_max_inputs(B: int, H: int, N: int, d: int, dtype: str, seed: int = 0,
                      rate: float = 0.5, spikes: int = 0):
    """Dense [B,H,N,d] Q, K, V (CPU tensors of `dtype`) whose scores make a
    running row maximum move many times along the keys.

    Q, K, V ~ N(0,1) as dense_inputs draws them; then every query gets a
    first component of at least 1, and
      spikes == 0: key c gets rate*c added to its first component, so every
                   query's scores rise along the keys and the running max
                   moves in nearly every key tile;
      spikes > 0:  `spikes` keys per head, at seeded random positions, get
                   first components 16, 32, 48, ... in key order, so the
                   running max jumps at a few tiles and stays put between.
    """
    rng = np.random.default_rng(seed)
    shape = (B, H, N, d)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    q[..., 0] = 1.0 + np.abs(q[..., 0])
    if spikes == 0:
        k[..., 0] += np.float32(rate) * np.arange(N, dtype=np.float32)
    else:
        for b in range(B):
            for h in range(H):
                pos = np.sort(rng.choice(N, size=min(spikes, N), replace=False))
                k[b, h, pos, 0] = 16.0 * np.arange(1, pos.size + 1, dtype=np.float32)
    return _round(q, dtype), _round(k, dtype), _round(v, dtype)


def dense_bwd_inputs(B: int, H: int, N: int, d: int, dtype: str, seed: int = 0,
                     qk_std: float = 1.0, v_uniform: bool = False):
    """Q, K, V as dense_inputs draws them, then the upstream gradient dO ~ N(0,1)
    from the same generator; all [B,H,N,d] CPU tensors of `dtype`."""
    rng = np.random.default_rng(seed)
    q, k, v = draw_qkv(rng, (B, H, N, d), dtype, qk_std, v_uniform)
    do = _round(rng.standard_normal((B, H, N, d), dtype=np.float32), dtype)
    return q, k, v, do


def varlen_lengths(nseq: int, lo: int, hi: int, seed: int = 0) -> np.ndarray:
    """Sequence lengths ~ U{lo..hi} (inclusive), the first draw of the seed."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi, endpoint=True, size=nseq).astype(np.int64)


def cu_seqlens_of(lengths) -> torch.Tensor:
    """int32 cumulative offsets [0, n0, n0+n1, ...] (nseq+1 entries)."""
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    np.cumsum(lengths, out=cu[1:])
    return torch.from_numpy(cu.astype(np.int32))


def device_normal(shape, dtype: str, seed: int, device) -> torch.Tensor:
    """N(0, 1) values of the storage dtype drawn on `device` by torch's seeded
    device generator: inputs of several GiB that a host draw would take
    minutes to make. The oracle side reads the same values back."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    tdt = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[dtype]
    return torch.randn(tuple(shape), generator=g, device=device, dtype=tdt)


def varlen_inputs(lengths, H: int, d: int, dtype: str, seed: int = 0,
                  rng: np.random.Generator | None = None):
    """Packed [T,H,d] Q, K, V and int32 cu_seqlens for the given lengths.

    When `rng` is None a fresh generator of `seed` is used; the workload
    generator passes the one that already drew the lengths."""
    if rng is None:
        rng = np.random.default_rng(seed)
    cu = cu_seqlens_of(lengths)
    T = int(cu[-1])
    q, k, v = draw_qkv(rng, (T, H, d), dtype)
    return q, k, v, cu


def make(name: str, seq_len: int | None = None):
    """Inputs of a named workload.

    Dense: returns dict(q,k,v, B,H,N,d, scale, dtype); seq_len, if given,
    replaces N (same B, H, d, dtype, distributions and seed).
    Varlen: returns dict(q,k,v, cu_seqlens, lengths, max_seqlen, H,d, scale, dtype).
    """
    w = WORKLOADS[name]
    if seq_len is not None:
        if w.varlen:
            raise ValueError("seq_len applies to dense workloads only")
        w = dataclasses.replace(w, N=int(seq_len))
    if w.varlen:
        rng = np.random.default_rng(w.seed)
        lengths = rng.integers(w.min_len, w.max_len, endpoint=True, size=w.nseq).astype(np.int64)
        q, k, v, cu = varlen_inputs(lengths, w.H, w.d, w.dtype, rng=rng)
        return dict(q=q, k=k, v=v, cu_seqlens=cu, lengths=lengths,
                    max_seqlen=int(lengths.max()), H=w.H, d=w.d, scale=w.scale,
                    dtype=w.dtype)
    q, k, v = dense_inputs(w.B, w.H, w.N, w.d, w.dtype, w.seed, w.qk_std, w.v_uniform)
    return dict(q=q, k=k, v=v, B=w.B, H=w.H, N=w.N, d=w.d, scale=w.scale, dtype=w.dtype)


def attention_flops(B: int, H: int, N: int, d: int) -> int:
    """Counted work of one forward: two N x N x d products per head, 2 flops per MAC."""
    return 4 * B * H * N * N * d


def varlen_flops(lengths, H: int, d: int) -> int:
    return 4 * H * d * int(sum(int(n) * int(n) for n in lengths))


def band_pairs(N: int, window: int) -> int:
    """Number of (query, key) pairs with |r - c| <= window among N x N."""
    if window >= N - 1:
        return N * N
    return N * (2 * window + 1) - window * (window + 1)


def banded_flops(B: int, H: int, N: int, d: int, window: int) -> int:
    """Counted work of one banded forward: 4 d flops per in-band pair."""
    return 4 * B * H * d * band_pairs(N, window)


def traffic_q_outer(n: int, d: int, Br: int, elem: int, stat: int = 4) -> dict:
    """Bytes one head moves between HBM and on-chip memory in the Q-outer
    (FlashAttention-2) order, counted by the trip rules of "Kernel
    visualization: Flash Attention 2" ("Counting trips across HBM") and the
    move() accounting of "FlashAttention -- for programmers, not
    researchers" (STAGE 4): Q read once, K and V read once per block of Br
    query rows, O and L written once. Returns {tensor: (read, written)}."""
    Tr = -(-n // Br)
    return {"Q": (n * d * elem, 0), "K": (Tr * n * d * elem, 0), "V": (Tr * n * d * elem, 0),
            "O": (0, n * d * elem), "L": (0, n * stat)}


def traffic_kv_outer(n: int, d: int, Bc: int, elem: int, groups: int = 1, acc: int = 4,
                     stat: int = 4) -> dict:
    """The same for the K/V-outer order: the key/value tiles are the outer
    loop (read once per group of query rows that streams them), and for
    every tile each query row reads Q, and reads back and rewrites its
    running output O (acc bytes per element) and its statistics m, l, which
    therefore cross HBM once per key tile; the last tile writes the final O
    (elem bytes) and L instead. Returns {tensor: (read, written)}."""
    Tc = -(-n // Bc)
    trips = Tc - 1
    return {"Q": (Tc * n * d * elem, 0), "K": (groups * n * d * elem, 0),
            "V": (groups * n * d * elem, 0), "O_acc": (trips * n * d * acc, trips * n * d * acc),
            "m_l": (trips * 2 * n * stat, trips * 2 * n * stat), "O": (0, n * d * elem),
            "L": (0, n * stat)}


def traffic_total(t: dict) -> tuple:
    """(bytes read, bytes written) of a traffic dict."""
    return sum(r for r, _ in t.values()), sum(w for _, w in t.values())


# Fused dropout + residual + norm workloads: the rows are the tokens of the
# attention workload above (B*N = 2*8192) and the hidden size its H*d = 4096
# (the attention output entering the residual stream), plus the largest hidden
# size the op supports with a parallel second branch and RMSNorm.
NORM_WORKLOADS = {
    "post_attention_ln_bf16": dict(rows=16384, hidden=4096, dtype="bf16", p=0.1, rms=False,
                                   x1=False, residual=True, gamma1=False, prenorm=True, seed=21),
    "parallel_rms_8192_bf16": dict(rows=8192, hidden=8192, dtype="bf16", p=0.1, rms=True,
                                   x1=True, residual=True, gamma1=True, prenorm=True, seed=22),
}


def norm_inputs(rows: int, hidden: int, dtype: str, seed: int = 0, x1: bool = False,
                residual: bool = True, beta: bool = True, gamma1: bool = False):
    """x0, x1, residual ~ N(0,1) [rows, hidden]; gamma ~ 1 + 0.1 N(0,1),
    beta ~ 0.1 N(0,1) [hidden]; drawn in that order as float32 and rounded to
    dtype. Absent tensors are None (and draw nothing)."""
    rng = np.random.default_rng(seed)
    t = DTYPES[dtype]
    draw = lambda shape, mul=1.0, add=0.0: torch.from_numpy(
        (add + mul * rng.standard_normal(shape, dtype=np.float32)).astype(np.float32)).to(t)
    out = {"x0": draw((rows, hidden))}
    out["x1"] = draw((rows, hidden)) if x1 else None
    out["residual"] = draw((rows, hidden)) if residual else None
    out["gamma0"] = draw((hidden,), 0.1, 1.0)
    out["beta0"] = draw((hidden,), 0.1) if beta else None
    out["gamma1"] = draw((hidden,), 0.1, 1.0) if gamma1 else None
    out["beta1"] = draw((hidden,), 0.1) if gamma1 and beta else None
    return out


def norm_bytes(rows: int, hidden: int, elem: int, x1: bool, residual: bool, gamma1: bool,
               prenorm: bool, stats: int = 2) -> int:
    """Compulsory HBM bytes of one fused dropout + residual + norm call: each
    row input read once, each output written once, weights once, stats."""
    row_in = 1 + int(x1) + int(residual)
    row_out = 1 + int(gamma1) + int(prenorm)
    weights = 2 * (1 + int(gamma1))
    return (row_in + row_out) * rows * hidden * elem + weights * hidden * elem + stats * rows * 4
