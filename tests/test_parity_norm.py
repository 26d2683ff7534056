"""GPU parity of the fused dropout + residual + LayerNorm/RMSNorm op
(fa_dropout_add_norm) against the float64 oracle on the same dtype-rounded
inputs.

The dropout keep masks are integer decisions from the same generator and
must match bit for bit. The float outputs (y0, y1, z) carry one rounding to
the storage dtype after fp32 arithmetic; a value near a rounding tie can go
either way, so the bound is one unit in the last place of the dtype at the
reference value (bf16 2^-7, fp16 2^-10 relative) plus 1e-4 for the fp32
sums over up to 8192 terms. mean and rstd are fp32: relative 2e-5 (rstd)
and 2e-5 absolute (mean, whose reference is O(1/sqrt(hidden))).
"""
import numpy as np
import pytest
import torch

import exact_attention_26_amd as fa
import oracle
import workloads
from gpu_helpers import announce, device, f64

pytestmark = pytest.mark.gpu

ULP = {"bf16": 2.0 ** -7, "fp16": 2.0 ** -10}


def _close(name, got, want, dtype):
    got = f64(got)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (name, got.shape, want.shape)
    if got.size == 0:
        return
    assert np.all(np.isfinite(got)), f"{name}: non-finite value"
    err = np.abs(got - want)
    bound = ULP[dtype] * np.abs(want) + 1e-4
    bad = np.argwhere(err > bound)
    if bad.size:
        idx = tuple(int(i) for i in bad[0])
        raise AssertionError(f"{name}: |err| {err[idx]:.3e} > {bound[idx]:.3e} at {idx}: "
                             f"got {got[idx]!r}, oracle {want[idx]!r} ({len(bad)} elements)")


def _check(inp, out, ref, dtype, row_ids=None):
    rows = slice(None) if row_ids is None else row_ids
    _close("y0", out["y0"][rows], ref["y0"], dtype)
    if ref["y1"] is not None:
        _close("y1", out["y1"][rows], ref["y1"], dtype)
    if out["z"] is not None:
        _close("z", out["z"][rows], ref["z"], dtype)
    if out["mask"] is not None:
        m = out["mask"].cpu().numpy()
        assert np.array_equal(m[0][rows].astype(bool), ref["keep0"]), "keep mask of x0"
        if ref["keep1"] is not None:
            assert np.array_equal(m[1][rows].astype(bool), ref["keep1"]), "keep mask of x1"
    if out["rstd"] is not None:
        r = f64(out["rstd"][rows])
        assert np.max(np.abs(r - ref["rstd"]) / ref["rstd"]) <= 2e-5, "rstd"
    if out["mean"] is not None:
        assert np.max(np.abs(f64(out["mean"][rows]) - ref["mean"])) <= 2e-5, "mean"


def _run(rows, hidden, dtype, p, rms, x1, residual, gamma1, beta, seed, offset=0):
    dev = device()
    inp = workloads.norm_inputs(rows, hidden, dtype, seed=seed, x1=x1, residual=residual,
                                beta=beta, gamma1=gamma1)
    g = {k: (None if v is None else v.to(dev)) for k, v in inp.items()}
    out = fa.dropout_add_norm(g["x0"], g["gamma0"], g["beta0"], residual=g["residual"],
                              x1=g["x1"], gamma1=g["gamma1"], beta1=g["beta1"], p=p,
                              seed=seed * 7919 + 1, offset=offset, eps=1e-5, rms=rms,
                              prenorm=True, stats=True, return_mask=True)
    torch.cuda.synchronize()
    return inp, out


HIDDEN = [8, 64, 504, 512, 520, 1024, 2048, 2056, 4096, 4104, 8192]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("rms", [False, True])
@pytest.mark.parametrize("hidden", HIDDEN)
def test_small_norm(dtype, rms, hidden):
    rows = 37 if hidden <= 4104 else 13
    seed = hidden + 3 * rms + (0 if dtype == "bf16" else 1000)
    announce(f"norm {dtype} rms={rms} rows={rows} hidden={hidden} p=0.1 residual seed={seed}")
    inp, out = _run(rows, hidden, dtype, 0.1, rms, False, True, False, True, seed)
    ref = oracle.dropout_add_norm(inp["x0"], inp["gamma0"], inp["beta0"],
                                  residual=inp["residual"], p=0.1, seed=seed * 7919 + 1,
                                  eps=1e-5, rms=rms)
    _check(inp, out, ref, dtype)


@pytest.mark.parametrize("p", [0.0, 0.5, 0.9])
@pytest.mark.parametrize("x1,residual,gamma1,beta", [(False, False, False, True),
                                                    (True, True, True, True),
                                                    (True, False, True, False),
                                                    (False, True, False, False)])
def test_norm_options(p, x1, residual, gamma1, beta):
    rows, hidden, dtype = 21, 1032, "bf16"
    seed = int(p * 10) + 2 * x1 + 4 * residual + 8 * gamma1 + 16 * beta
    announce(f"norm options p={p} x1={x1} residual={residual} gamma1={gamma1} beta={beta}")
    inp, out = _run(rows, hidden, dtype, p, False, x1, residual, gamma1, beta, seed,
                    offset=(3 << 32) | 5)
    ref = oracle.dropout_add_norm(inp["x0"], inp["gamma0"], inp["beta0"],
                                  residual=inp["residual"], x1=inp["x1"], gamma1=inp["gamma1"],
                                  beta1=inp["beta1"], p=p, seed=seed * 7919 + 1,
                                  offset=(3 << 32) | 5, eps=1e-5)
    _check(inp, out, ref, dtype)
    if p == 0.0:
        assert bool(out["mask"].all()), "p = 0 keeps every element"


def test_norm_post_norm_and_no_stats():
    # post-norm: no z output; no mean / rstd; the same y0 as the pre-norm call
    dev = device()
    announce("norm post-norm without stats bf16 rows=9 hidden=2048")
    inp = workloads.norm_inputs(9, 2048, "bf16", seed=77)
    g = {k: (None if v is None else v.to(dev)) for k, v in inp.items()}
    a = fa.dropout_add_norm(g["x0"], g["gamma0"], g["beta0"], residual=g["residual"], p=0.2,
                            seed=5, prenorm=False, stats=False)
    b = fa.dropout_add_norm(g["x0"], g["gamma0"], g["beta0"], residual=g["residual"], p=0.2,
                            seed=5, prenorm=True, stats=True)
    torch.cuda.synchronize()
    assert a["z"] is None and a["mean"] is None and a["rstd"] is None
    assert torch.equal(a["y0"], b["y0"])


def test_norm_deterministic():
    dev = device()
    announce("norm determinism bf16 rows=64 hidden=4096 p=0.1")
    inp = workloads.norm_inputs(64, 4096, "bf16", seed=78)
    g = {k: (None if v is None else v.to(dev)) for k, v in inp.items()}
    a = fa.dropout_add_norm(g["x0"], g["gamma0"], g["beta0"], residual=g["residual"], p=0.1,
                            seed=11, return_mask=True)
    b = fa.dropout_add_norm(g["x0"], g["gamma0"], g["beta0"], residual=g["residual"], p=0.1,
                            seed=11, return_mask=True)
    c = fa.dropout_add_norm(g["x0"], g["gamma0"], g["beta0"], residual=g["residual"], p=0.1,
                            seed=12, return_mask=True)
    torch.cuda.synchronize()
    assert all(torch.equal(a[k], b[k]) for k in ("y0", "z", "mask", "mean", "rstd"))
    assert not torch.equal(a["mask"], c["mask"]), "another seed draws another mask"


@pytest.mark.parametrize("name", sorted(workloads.NORM_WORKLOADS))
def test_norm_workload_sampled(name):
    w = workloads.NORM_WORKLOADS[name]
    rows, hidden = w["rows"], w["hidden"]
    announce(f"norm workload {name} rows={rows} hidden={hidden} (sampled rows)")
    inp, out = _run(rows, hidden, w["dtype"], w["p"], w["rms"], w["x1"], w["residual"],
                    w["gamma1"], True, w["seed"])
    keep_rate = float(out["mask"].float().mean())
    assert abs(keep_rate - (1 - w["p"])) < 2e-3, keep_rate
    rng = np.random.default_rng(w["seed"])
    ids = np.unique(np.r_[0, 1, rows // 2, rows - 1, rng.integers(0, rows, 28)])
    sel = lambda t: None if t is None else t[ids]
    ref = oracle.dropout_add_norm(sel(inp["x0"]), inp["gamma0"], inp["beta0"],
                                  residual=sel(inp["residual"]), x1=sel(inp["x1"]),
                                  gamma1=inp["gamma1"], beta1=inp["beta1"], p=w["p"],
                                  seed=w["seed"] * 7919 + 1, eps=1e-5, rms=w["rms"], row_ids=ids)
    _check(inp, out, ref, w["dtype"], row_ids=ids)
