"""Phase trace of the 16-bit forward from the debug build libfa_trace.so.

One workgroup of the 8-wave kernel at the long-sequence shape (B=2 H=32
N=8192 d=128 bf16) records the shader-clock timestamps of the start and end
of each wave's matrix half and softmax half for 64 key-tile steps
(fa_debug_fwd_trace). Checks:
  * the trace build computes the same O and L as the product library, bit
    for bit (the timestamps change no arithmetic);
  * every wave's timestamps increase through its steps;
  * no matrix half is shorter than its 32 MFMAs of 32 clocks each (1024
    shader clocks): a floor set by the matrix core itself;
  * the product library records nothing and says so (FA_ERR_UNSUPPORTED).
The per-wave phase medians and the barrier arrival order are printed; they
are the timeline of one step of the kernel.
"""
import numpy as np
import pytest
import torch

import exact_attention_26_amd as fa
import workloads
from gpu_helpers import announce, device

pytestmark = pytest.mark.gpu

STEPS, WAVES = 64, 8
MFMA_FLOOR = 32 * 32  # MFMAs per matrix half x clocks per MFMA


def _fwd(lib, q, k, v, scale):
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty(B, H, N, dtype=torch.float32, device=q.device)
    st = lib.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H,
                    N, d, scale, fa.FA_BF16, torch.cuda.current_stream(q.device).cuda_stream)
    assert st == 0, fa.fa_strerror(st)
    return o, lse


def test_phase_trace_of_the_long_forward():
    dev = device()
    announce("phase trace bf16 B=2 H=32 N=8192 d=128, workgroup 1000")
    B, H, N, d = 2, 32, 8192, 128
    q, k, v = (workloads.device_normal((B, H, N, d), "bf16", seed=s, device=dev) for s in (1, 2, 3))
    scale = d ** -0.5
    tlib = fa.load_library(fa.TRACE_LIB_PATH)
    buf = torch.zeros(WAVES * STEPS * 4 + WAVES * 4, dtype=torch.int64, device=dev)
    assert fa.load().fa_debug_fwd_trace(1000, buf.data_ptr()) == -12  # product library
    fa.fa_debug_fwd_trace(1000, buf.data_ptr(), lib=tlib)
    try:
        for _ in range(3):
            o_t, l_t = _fwd(tlib, q, k, v, scale)
        torch.cuda.synchronize()
    finally:
        fa.fa_debug_fwd_trace(-1, None, lib=tlib)
    o_p, l_p = _fwd(fa.load(), q, k, v, scale)
    torch.cuda.synchronize()
    assert torch.equal(o_t, o_p) and torch.equal(l_t, l_p)

    t = buf.cpu().numpy().astype(np.float64)
    pts = t[:WAVES * STEPS * 4].reshape(WAVES, STEPS, 4)
    cal = t[WAVES * STEPS * 4:].reshape(WAVES, 4)
    mhz = float(np.median((cal[:, 2] - cal[:, 0]) / (cal[:, 3] - cal[:, 1]) * 100.0))
    flat = pts.reshape(WAVES, -1)
    assert np.all(np.diff(flat[:, 4:], axis=1) >= 0), "timestamps out of order"
    s = slice(8, STEPS - 1)  # steady state: past the prologue's first steps
    matrix = pts[:, s, 1] - pts[:, s, 0]
    wait1 = pts[:, s, 2] - pts[:, s, 1]
    softmax = pts[:, s, 3] - pts[:, s, 2]
    wait2 = pts[:, 9:STEPS, 0] - pts[:, s, 3]
    assert matrix.min() >= MFMA_FLOOR, matrix.min()
    print(f"[trace] s_memtime at {mhz:.0f} MHz (against the 100 MHz clock); medians over steps "
          f"8..62, shader clocks", flush=True)
    for w in range(WAVES):
        med = [float(np.median(x[w])) for x in (matrix, wait1, softmax, wait2)]
        print(f"[trace] wave {w} ({'A' if w < 4 else 'B'}): matrix {med[0]:.0f}  wait+barrier "
              f"{med[1]:.0f}  softmax{' + copies' if w >= 4 else ''} {med[2]:.0f}  barrier "
              f"{med[3]:.0f}  step {sum(med):.0f}", flush=True)
    # Group B runs one barrier behind group A: A's matrix end of step j meets
    # B's softmax end of step j-1, and A's softmax end of step j meets B's
    # matrix end of step j.
    last_b1 = int(np.sum(pts[4:, 7:STEPS - 2, 3].max(0) > pts[:4, 8:STEPS - 1, 1].max(0)))
    last_b2 = int(np.sum(pts[4:, s, 1].max(0) > pts[:4, s, 3].max(0)))
    print(f"[trace] group B last at the barrier after A's matrix half: {last_b1} of {STEPS - 9}; "
          f"after B's matrix half: {last_b2} of {STEPS - 9}", flush=True)


WAVES_NARROW = 4
STEPS_SHORT = 16  # key tiles of N = 1024


def test_phase_trace_of_a_short_forward():
    """The 4-wave kernel at the short shape (B=4 H=16 N=1024 d=64 bf16: 512
    workgroups of 128 rows, two per CU): one workgroup of each of the two
    that share a CU. Besides the bitwise and ordering checks, no matrix half
    may be shorter than its MFMAs (16, or 8 in the last step, of 32 clocks). Printed per workgroup: the
    prologue (wave start to the first matrix half), the median step and its
    matrix and softmax halves, and the write-back (last matrix half to the
    wave's end)."""
    dev = device()
    B, H, N, d = 4, 16, 1024, 64
    q, k, v = (workloads.device_normal((B, H, N, d), "bf16", seed=s, device=dev) for s in (1, 2, 3))
    scale = d ** -0.5
    tlib = fa.load_library(fa.TRACE_LIB_PATH)
    o_p, l_p = _fwd(fa.load(), q, k, v, scale)
    for wg in (100, 300):
        announce(f"phase trace bf16 B={B} H={H} N={N} d={d}, workgroup {wg}")
        buf = torch.zeros(WAVES * STEPS * 4 + WAVES * 4, dtype=torch.int64, device=dev)
        fa.fa_debug_fwd_trace(wg, buf.data_ptr(), lib=tlib)
        try:
            for _ in range(3):
                o_t, l_t = _fwd(tlib, q, k, v, scale)
            torch.cuda.synchronize()
        finally:
            fa.fa_debug_fwd_trace(-1, None, lib=tlib)
        assert torch.equal(o_t, o_p) and torch.equal(l_t, l_p)
        t = buf.cpu().numpy().astype(np.float64)
        pts = t[:WAVES * STEPS * 4].reshape(WAVES, STEPS, 4)[:WAVES_NARROW, :STEPS_SHORT]
        cal = t[WAVES * STEPS * 4:].reshape(WAVES, 4)[:WAVES_NARROW]
        mhz = float(np.median((cal[:, 2] - cal[:, 0]) / (cal[:, 3] - cal[:, 1]) * 100.0))
        # The last step has no softmax half: its points 2 and 3 follow point 1.
        assert np.all(np.diff(pts.reshape(WAVES_NARROW, -1), axis=1) >= 0), "timestamps out of order"
        assert np.all(pts[:, 0, 0] >= cal[:, 0]) and np.all(cal[:, 2] >= pts[:, -1, 3])
        matrix = pts[:, :, 1] - pts[:, :, 0]
        # 16 MFMAs per matrix half (S^T of the next tile and P.V); the last
        # has no next tile, so only its 8 P.V MFMAs.
        assert matrix[:, :-1].min() >= 16 * 32 and matrix[:, -1].min() >= 8 * 32, matrix.min()
        s = slice(1, STEPS_SHORT - 1)
        step = np.median(pts[:, 2:STEPS_SHORT, 0] - pts[:, 1:STEPS_SHORT - 1, 0])
        soft = np.median(pts[:, s, 3] - pts[:, s, 2])
        pro = np.median(pts[:, 0, 0] - cal[:, 0])
        epi = np.median(cal[:, 2] - pts[:, -1, 1])
        life = np.median(cal[:, 2] - cal[:, 0])
        print(f"[trace] workgroup {wg}: {mhz:.0f} MHz; prologue {pro:.0f}; step {step:.0f} "
              f"(matrix {np.median(matrix[:, s]):.0f}, softmax + copies {soft:.0f}); write-back "
              f"{epi:.0f}; wave life {life:.0f} = {life / mhz:.1f} us ({STEPS_SHORT} tiles)",
              flush=True)
