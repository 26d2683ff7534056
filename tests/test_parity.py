"""GPU parity: the HIP path through the C ABI against the float64 oracle on
the same dtype-rounded inputs, element by element.

Bounds (max |GPU - oracle|): fp32 O <= 2e-5, L <= 1e-5; bf16/fp16
O <= 2e-2, L <= 5e-3.

Small problems are compared in full; they span several query blocks and
key tiles and end in ragged tails. Every full-size workload is compared in
full, every head and row (the two largest on a thread pool of oracle
calls, about 20 s each on the host); the largest are also compared on
sampled edge rows, and on properties that hold at any size.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import TOL, announce, assert_close, device, f64, run_dense, run_varlen

pytestmark = pytest.mark.gpu

SMALL_N = [1, 2, 31, 33, 63, 64, 65, 127, 128, 129, 200, 257, 1000]


@pytest.mark.parametrize("dtype", ["fp32", "bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", SMALL_N)
def test_small_dense(dtype, d, N):
    dev = device()
    B, H = (2, 3) if N <= 257 else (1, 2)
    seed = 1000 * d + N + {"fp32": 0, "bf16": 1, "fp16": 2}[dtype] * 100000
    announce(f"small dense {dtype} B={B} H={H} N={N} d={d} seed={seed}")
    q, k, v = workloads.dense_inputs(B, H, N, d, dtype, seed=seed)
    scale = 1.0 / math.sqrt(d)
    o, lse = run_dense(q, k, v, scale, dev)
    O_ref, L_ref = oracle.attention_dense(q, k, v, scale)
    tol_o, tol_l = TOL[dtype]
    assert_close("O", f64(o), O_ref, tol_o)
    assert_close("L", f64(lse), L_ref, tol_l)


# Just past the sizes that run in 4-wave workgroups: the 8-wave (two wave
# groups, three K/V stages) kernel over 33, 34 and 35 key tiles, so that its
# loop ends in each of its three phases, with and without a ragged last tile.
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [2049, 2112, 2176, 2200])
def test_dense_eight_wave_tails(dtype, d, N):
    dev = device()
    B, H = 1, 2
    seed = 3000 * d + N + (0 if dtype == "bf16" else 70000)
    announce(f"dense 8-wave tails {dtype} B={B} H={H} N={N} d={d} seed={seed}")
    q, k, v = workloads.dense_inputs(B, H, N, d, dtype, seed=seed)
    scale = 1.0 / math.sqrt(d)
    o, lse = run_dense(q, k, v, scale, dev)
    O_ref, L_ref = oracle.attention_dense(q, k, v, scale)
    tol_o, tol_l = TOL[dtype]
    assert_close("O", f64(o), O_ref, tol_o)
    assert_close("L", f64(lse), L_ref, tol_l)


@pytest.mark.parametrize("name", ["single_head_fp32", "short_bf16", "large_logit_fp16_a",
                                  "large_logit_fp16_b"])
def test_workload_full(name):
    dev = device()
    w = workloads.make(name)
    announce(f"workload {name} B={w['B']} H={w['H']} N={w['N']} d={w['d']} {w['dtype']}")
    o, lse = run_dense(w["q"], w["k"], w["v"], w["scale"], dev)
    O_ref, L_ref = oracle.attention_dense(w["q"], w["k"], w["v"], w["scale"])
    tol_o, tol_l = TOL[w["dtype"]]
    assert_close(f"{name} O", f64(o), O_ref, tol_o)
    assert_close(f"{name} L", f64(lse), L_ref, tol_l)


def _sample_rows(n, rng, extra=40):
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, 129, n // 2, n - 129, n - 128, n - 65, n - 64,
             n - 2, n - 1]
    rows = {r for r in fixed if 0 <= r < n}
    rows.update(int(x) for x in rng.integers(0, n, size=min(extra, n)))
    return np.array(sorted(rows))


def _convex_hull_check(name, o, v, tol):
    # Every output row is a convex combination of the value rows of its head:
    # min_c V[c, j] - tol <= O[r, j] <= max_c V[c, j] + tol. Holds at any size.
    vmin = v.float().amin(dim=-2, keepdim=True)
    vmax = v.float().amax(dim=-2, keepdim=True)
    of = o.float()
    assert torch.isfinite(of).all(), f"{name}: non-finite output"
    assert bool(((of >= vmin - tol) & (of <= vmax + tol)).all()), f"{name}: O outside hull of V"


def test_workload_long_bf16_sampled():
    dev = device()
    w = workloads.make("long_bf16")
    B, H, N, d = w["B"], w["H"], w["N"], w["d"]
    announce(f"workload long_bf16 B={B} H={H} N={N} d={d} (sampled rows)")
    qd, kd, vd = w["q"].to(dev), w["k"].to(dev), w["v"].to(dev)
    import exact_attention_26_amd as fa
    o, lse = fa.forward(qd, kd, vd, w["scale"])
    torch.cuda.synchronize()
    tol_o, tol_l = TOL["bf16"]
    _convex_hull_check("long_bf16", o, vd, tol_o)
    rng = np.random.default_rng(123)
    for (b, h) in [(0, 0), (1, 31), (0, 17), (1, 5)]:
        rows = _sample_rows(N, rng)
        O_ref, L_ref = oracle.attention_dense_rows(w["q"], w["k"], w["v"], w["scale"], b, h, rows)
        assert_close(f"long_bf16 O[b={b},h={h}]", f64(o[b, h, rows]), O_ref, tol_o)
        assert_close(f"long_bf16 L[b={b},h={h}]", f64(lse[b, h, rows]), L_ref, tol_l)


def _oracle_parallel(jobs, workers=8):
    """Run independent oracle calls (one per head or sequence) on a thread
    pool; numpy's BLAS and exp release the GIL. BLAS threads per call are
    capped so the pool does not oversubscribe the host."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=2, user_api="blas"), ThreadPoolExecutor(workers) as ex:
        return list(ex.map(lambda job: job(), jobs))


def test_workload_long_bf16_full():
    # Every (batch, head) of the long-sequence workload against the oracle,
    # element by element: each block runs the same steps on its own data
    # ("Kernel visualization: Flash Attention 2", "Same operations in another
    # block"), so every block is checked. About 2.2 TFLOP of float64.
    dev = device()
    w = workloads.make("long_bf16")
    B, H, N, d = w["B"], w["H"], w["N"], w["d"]
    announce(f"workload long_bf16 B={B} H={H} N={N} d={d} (every head, every row)")
    o, lse = run_dense(w["q"], w["k"], w["v"], w["scale"], dev)
    o, lse = o.cpu(), lse.cpu()
    q, k, v = (f64(t) for t in (w["q"], w["k"], w["v"]))
    heads = [(b, h) for b in range(B) for h in range(H)]
    refs = _oracle_parallel([
        (lambda b=b, h=h: oracle.attention_naive(q[b, h], k[b, h], v[b, h], w["scale"]))
        for (b, h) in heads])
    tol_o, tol_l = TOL["bf16"]
    for (b, h), (O_ref, L_ref) in zip(heads, refs):
        assert_close(f"long_bf16 O[b={b},h={h}]", f64(o[b, h]), O_ref, tol_o)
        assert_close(f"long_bf16 L[b={b},h={h}]", f64(lse[b, h]), L_ref, tol_l)


def test_workload_varlen_full():
    # Every (sequence, head) of the packed workload, element by element.
    dev = device()
    w = workloads.make("varlen_bf16")
    lengths, cu, H = w["lengths"], w["cu_seqlens"], w["H"]
    announce(f"workload varlen_bf16 nseq={len(lengths)} T={int(cu[-1])} H={H} "
             f"(every sequence and head, every row)")
    o, lse = run_varlen(w["q"], w["k"], w["v"], cu, w["max_seqlen"], w["scale"], dev)
    o, lse = o.cpu(), lse.cpu()
    q, k, v = (f64(t) for t in (w["q"], w["k"], w["v"]))
    jobs, keys = [], []
    for s in range(len(lengths)):
        a, e = int(cu[s]), int(cu[s + 1])
        for h in range(H):
            keys.append((s, h, a, e))
            jobs.append(lambda a=a, e=e, h=h: oracle.attention_naive(q[a:e, h], k[a:e, h],
                                                                      v[a:e, h], w["scale"]))
    refs = _oracle_parallel(jobs)
    tol_o, tol_l = TOL["bf16"]
    for (s, h, a, e), (O_ref, L_ref) in zip(keys, refs):
        assert_close(f"varlen O[seq={s},h={h}]", f64(o[a:e, h]), O_ref, tol_o)
        assert_close(f"varlen L[seq={s},h={h}]", f64(lse[h, a:e]), L_ref, tol_l)


def test_workload_varlen_sampled():
    dev = device()
    w = workloads.make("varlen_bf16")
    lengths = w["lengths"]
    cu = w["cu_seqlens"]
    H, d = w["H"], w["d"]
    announce(f"workload varlen_bf16 nseq={len(lengths)} T={int(cu[-1])} H={H} d={d} "
             f"max={w['max_seqlen']} (sampled rows)")
    o, lse = run_varlen(w["q"], w["k"], w["v"], cu, w["max_seqlen"], w["scale"], dev)
    tol_o, tol_l = TOL["bf16"]
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    rng = np.random.default_rng(321)
    order = np.argsort(lengths)
    seqs = [int(order[0]), int(order[1]), int(order[-1]), int(order[len(order) // 2]), 7]
    for s in seqs:
        a = int(cu[s])
        n = int(lengths[s])
        rows = np.arange(n) if n <= 200 else _sample_rows(n, rng, extra=24)
        for h in [0, 9, 15]:
            O_ref, L_ref = oracle.attention_varlen_rows(w["q"], w["k"], w["v"], cu, w["scale"], s,
                                                        h, rows)
            assert_close(f"varlen O[seq={s},h={h}]", f64(o[a + rows, h]), O_ref, tol_o)
            assert_close(f"varlen L[seq={s},h={h}]", f64(lse[h, a + rows]), L_ref, tol_l)


@pytest.mark.parametrize("dtype", ["fp32", "bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
def test_small_varlen(dtype, d):
    dev = device()
    lengths = [1, 63, 64, 65, 130, 5, 128, 129, 2]
    H = 3
    announce(f"small varlen {dtype} d={d} lengths={lengths}")
    q, k, v, cu = workloads.varlen_inputs(lengths, H, d, dtype, seed=d + len(dtype))
    scale = 1.0 / math.sqrt(d)
    o, lse = run_varlen(q, k, v, cu, max(lengths), scale, dev)
    O_ref, L_ref = oracle.attention_varlen(q, k, v, cu, scale)
    tol_o, tol_l = TOL[dtype]
    assert_close("varlen O", f64(o), O_ref, tol_o)
    assert_close("varlen L", f64(lse), L_ref, tol_l)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
def test_varlen_eight_wave_short_sequences(dtype, d):
    # One sequence longer than the 4-wave limit puts the whole batch on the
    # 8-wave kernel; the short ones then visit 1, 2 and 3 key tiles.
    dev = device()
    lengths = [1, 63, 64, 65, 130, 4160, 129, 2, 192, 150]
    H = 2
    announce(f"varlen 8-wave short sequences {dtype} d={d} lengths={lengths}")
    q, k, v, cu = workloads.varlen_inputs(lengths, H, d, dtype, seed=d + 11)
    scale = 1.0 / math.sqrt(d)
    o, lse = run_varlen(q, k, v, cu, max(lengths), scale, dev)
    tol_o, tol_l = TOL[dtype]
    rng = np.random.default_rng(d)
    for s, n in enumerate(lengths):
        a = int(cu[s])
        rows = np.arange(n) if n <= 256 else _sample_rows(n, rng, extra=16)
        for h in range(H):
            O_ref, L_ref = oracle.attention_varlen_rows(q, k, v, cu, scale, s, h, rows)
            assert_close(f"varlen O[seq={s},h={h}]", f64(o[a + rows, h]), O_ref, tol_o)
            assert_close(f"varlen L[seq={s},h={h}]", f64(lse[h, a + rows]), L_ref, tol_l)


def test_varlen_with_empty_sequences():
    dev = device()
    lengths = [0, 70, 0, 0, 3, 0]
    announce(f"varlen with empty sequences {lengths}")
    q, k, v, cu = workloads.varlen_inputs(lengths, 2, 64, "bf16", seed=5)
    o, lse = run_varlen(q, k, v, cu, max(lengths), 0.125, dev)
    O_ref, L_ref = oracle.attention_varlen(q, k, v, cu, 0.125)
    assert_close("varlen O", f64(o), O_ref, TOL["bf16"][0])
    assert_close("varlen L", f64(lse), L_ref, TOL["bf16"][1])


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_varlen_equals_dense_per_sequence(dtype):
    # The packed entry computes exactly what the dense entry computes on each
    # sequence alone (same kernel arithmetic, different strides): bitwise for
    # the 16-bit kernels. A single fp32 sequence this small runs the dense
    # entry's key-split form, which adds the keys in another order, so fp32
    # is compared at its tolerance.
    dev = device()
    lengths = [300, 17, 129, 64]
    H, d = 4, 128
    announce(f"varlen == dense per sequence {dtype} lengths={lengths}")
    q, k, v, cu = workloads.varlen_inputs(lengths, H, d, dtype, seed=77)
    o, lse = run_varlen(q, k, v, cu, max(lengths), 0.09, dev)
    for s, n in enumerate(lengths):
        a = int(cu[s])
        sl = lambda t: t[a:a + n].permute(1, 0, 2).contiguous()[None]  # [1,H,n,d]
        od, ld = run_dense(sl(q), sl(k), sl(v), 0.09, dev)
        if dtype == "fp32":
            assert_close(f"O seq {s}", f64(od[0].permute(1, 0, 2)), f64(o[a:a + n]), TOL[dtype][0])
            assert_close(f"L seq {s}", f64(ld[0]), f64(lse[:, a:a + n]), TOL[dtype][1])
            continue
        assert torch.equal(od[0].permute(1, 0, 2).cpu(), o[a:a + n].cpu()), f"O seq {s}"
        assert torch.equal(ld[0].cpu(), lse[:, a:a + n].cpu()), f"L seq {s}"


def test_long_single_head_sampled():
    # A long sequence: 2^18 keys in one head, sampled rows against the oracle.
    dev = device()
    N, d = 1 << 18, 128
    announce(f"long single head bf16 N={N} d={d} (sampled rows)")
    q, k, v = workloads.dense_inputs(1, 1, N, d, "bf16", seed=9)
    o, lse = run_dense(q, k, v, 1.0 / math.sqrt(d), dev)
    rows = _sample_rows(N, np.random.default_rng(9), extra=8)
    O_ref, L_ref = oracle.attention_dense_rows(q, k, v, 1.0 / math.sqrt(d), 0, 0, rows)
    assert_close("O", f64(o[0, 0, rows]), O_ref, TOL["bf16"][0])
    assert_close("L", f64(lse[0, 0, rows]), L_ref, TOL["bf16"][1])


@pytest.mark.parametrize("nseq", [40, 80])
def test_varlen_unit_order_with_ties(nseq):
    # Up to 64 sequences run their units longest sequence first, ranked in
    # the kernel (ties by index); more sequences keep the plain order. Both
    # with many equal lengths, empty sequences and ragged tails.
    dev = device()
    rng = np.random.default_rng(nseq)
    lengths = [int(x) for x in rng.choice([0, 1, 64, 65, 130, 200, 257], size=nseq)]
    announce(f"varlen unit order nseq={nseq} bf16 d=64 lengths={lengths}")
    q, k, v, cu = workloads.varlen_inputs(lengths, 2, 64, "bf16", seed=nseq)
    o, lse = run_varlen(q, k, v, cu, max(lengths), 0.125, dev)
    O_ref, L_ref = oracle.attention_varlen(q, k, v, cu, 0.125)
    assert_close("varlen O", f64(o), O_ref, TOL["bf16"][0])
    assert_close("varlen L", f64(lse), L_ref, TOL["bf16"][1])


def test_varlen_sequence_longer_than_max_seqlen():
    # max_seqlen sizes the grid: a longer sequence gets its first rows (up to
    # max_seqlen, rounded up to a query block of at most 256 rows) computed
    # against all of its keys; the rows past that block stay unwritten.
    dev = device()
    lengths, max_seqlen = [700, 90, 5], 100
    announce(f"varlen lengths={lengths} with max_seqlen={max_seqlen}")
    q, k, v, cu = workloads.varlen_inputs(lengths, 2, 128, "bf16", seed=31)
    import exact_attention_26_amd as fa
    T = sum(lengths)
    o = torch.full((T, 2, 128), 7.0, dtype=torch.bfloat16, device=dev)
    lse = torch.full((2, T), 7.0, dtype=torch.float32, device=dev)
    fa.forward_varlen(q.to(dev), k.to(dev), v.to(dev), cu.to(dev), max_seqlen, 0.1, out=o, lse=lse)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention_varlen(q, k, v, cu, 0.1)
    for s, n in enumerate(lengths):
        a, done = int(cu[s]), min(n, max_seqlen)
        assert_close(f"O seq {s}", f64(o[a:a + done]), O_ref[a:a + done], TOL["bf16"][0])
        assert_close(f"L seq {s}", f64(lse[:, a:a + done]), L_ref[:, a:a + done], TOL["bf16"][1])
    untouched = f64(o[256:700])
    assert (untouched == 7.0).all() and (f64(lse[:, 256:700]) == 7.0).all()


def test_dense_offsets_beyond_2_31_elements():
    # 2^31 elements per tensor (4 GiB): the last heads start past 2^31, which
    # only the 64-bit head bases reach. Q = K = V (allowed), sampled rows.
    dev = device()
    B, H, N, d = 1, 2049, 8192, 128
    announce(f"dense offsets past 2^31 elements bf16 B={B} H={H} N={N} d={d} (sampled)")
    x = workloads.device_normal((B, H, N, d), "bf16", seed=41, device=dev)
    import exact_attention_26_amd as fa
    o, lse = fa.forward(x, x, x, 1.0 / math.sqrt(d))
    torch.cuda.synchronize()
    assert (H - 1) * N * d >= 1 << 31
    rows = _sample_rows(N, np.random.default_rng(41), extra=4)
    for h in (0, H - 1):
        xh = x[0, h].cpu()
        O_ref, L_ref = oracle.attention_dense_rows(xh[None, None], xh[None, None], xh[None, None],
                                                   1.0 / math.sqrt(d), 0, 0, rows)
        assert_close(f"O h={h}", f64(o[0, h, rows]), O_ref, TOL["bf16"][0])
        assert_close(f"L h={h}", f64(lse[0, h, rows]), L_ref, TOL["bf16"][1])


@pytest.mark.parametrize("nseq", [64, 130])
def test_varlen_offsets_beyond_2_31_elements(nseq):
    # Packed [T, 16, 128] with T*H*d > 2^31: the last sequences start past
    # 2^31 elements. 64 sequences take the longest-first order, 130 the plain
    # one. Q = K = V (allowed), sampled rows of the first and last sequence.
    dev = device()
    H, d = 16, 128
    base = (1 << 31) // (H * d) // (nseq - 1) + 64
    lengths = [base + 64 * (i % 3) for i in range(nseq)]
    T = sum(lengths)
    announce(f"varlen offsets past 2^31 elements bf16 nseq={nseq} T={T} H={H} d={d} (sampled)")
    assert (T - lengths[-1]) * H * d >= 1 << 31
    x = workloads.device_normal((T, H, d), "bf16", seed=43, device=dev)
    cu = workloads.cu_seqlens_of(lengths)
    o, lse = run_varlen(x, x, x, cu, max(lengths), 1.0 / math.sqrt(d), dev)
    rng = np.random.default_rng(43)
    for s in (0, nseq - 1):
        a, n = int(cu[s]), lengths[s]
        rows = _sample_rows(n, rng, extra=4)
        for h in (0, H - 1):
            xs = x[a:a + n, h].cpu()
            O_ref, L_ref = oracle.attention_dense_rows(xs[None, None], xs[None, None],
                                                       xs[None, None], 1.0 / math.sqrt(d), 0, 0,
                                                       rows)
            assert_close(f"O seq {s} h={h}", f64(o[a + rows, h]), O_ref, TOL["bf16"][0])
            assert_close(f"L seq {s} h={h}", f64(lse[h, a + rows]), L_ref, TOL["bf16"][1])
