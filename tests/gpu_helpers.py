"""Shared helpers of the GPU tests (not a test module)."""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

import exact_attention_26_amd as fa
from exact_attention_26_amd import build as fa_build

# Acceptance bounds on max |GPU - oracle|, per storage dtype: (O, L).
TOL = {"fp32": (2e-5, 1e-5), "bf16": (2e-2, 5e-3), "fp16": (2e-2, 5e-3)}


def device() -> torch.device:
    if not torch.cuda.is_available():
        raise RuntimeError("GPU test run without a GPU")
    fa.load()  # fail loudly if the HIP library is missing
    # ... or was built from other sources than those in the tree (the tests
    # would then check old kernels).
    stale = [os.path.basename(p) for p in (fa.LIB_PATH, fa.POISON_LIB_PATH, fa.TRACE_LIB_PATH)
             if not fa_build.is_current(p)]
    if stale:
        raise RuntimeError(f"{', '.join(stale)} not built from the current sources; "
                           "run python -m exact_attention_26_amd.build")
    return torch.device("cuda:0")


def announce(msg: str) -> None:
    """Name the case before any GPU work, flushed, so a crash can be traced."""
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def f64(t) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def assert_close(name: str, got, want, tol: float) -> float:
    """Max-abs comparison that reports the worst element's index and values."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, f"{name}: shape {got.shape} vs {want.shape}"
    if got.size == 0:
        return 0.0
    bad = ~np.isfinite(got)
    if bad.any():
        idx = tuple(int(i) for i in np.argwhere(bad)[0])
        raise AssertionError(f"{name}: non-finite value {got[idx]} at index {idx}")
    err = np.abs(got - want)
    idx = tuple(int(i) for i in np.unravel_index(int(np.argmax(err)), err.shape))
    worst = float(err[idx])
    assert worst <= tol, (f"{name}: max |err| = {worst:.3e} > {tol:.1e} at index {idx}: "
                          f"got {got[idx]!r}, oracle {want[idx]!r}")
    return worst


def run_dense(q, k, v, scale, dev):
    o, lse = fa.forward(q.to(dev), k.to(dev), v.to(dev), scale)
    torch.cuda.synchronize()
    return o, lse


def run_varlen(q, k, v, cu, max_seqlen, scale, dev):
    o, lse = fa.forward_varlen(q.to(dev), k.to(dev), v.to(dev), cu.to(dev), max_seqlen, scale)
    torch.cuda.synchronize()
    return o, lse
