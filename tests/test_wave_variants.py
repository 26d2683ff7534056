"""The 8-wave (ping-pong, 256-row workgroups) and 4-wave (128-row
workgroups) forms of the 16-bit forward run the same steps per wave on the
same 32 query rows and the same key tiles in the same order, so they must
give bitwise-identical O and L. The library picks the form by size: dense
N <= 2048 and packed batches with max_seqlen <= 3072 run 4 waves, larger
problems 8. A packed batch with one sequence longer than 3072 runs 8 waves
for every sequence; each of its shorter sequences is then compared bit for
bit with a dense call on that sequence alone, which runs 4 waves. The
lengths cover one to many key tiles, ragged tails and whole tiles, so the
8-wave kernel's peeled phases and stage rotation all meet the 4-wave one.
"""
import math

import numpy as np
import pytest
import torch

import workloads
from gpu_helpers import announce, device, run_dense, run_varlen

pytestmark = pytest.mark.gpu

LENGTHS = [1, 63, 64, 65, 128, 130, 191, 257, 700, 1000, 4200, 2048, 1500, 320]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("inputs", ["normal", "moving_max"])
def test_eight_wave_packed_equals_four_wave_dense(dtype, d, inputs):
    dev = device()
    H = 2
    announce(f"8-wave packed vs 4-wave dense {dtype} d={d} {inputs} lengths={LENGTHS}")
    if inputs == "normal":
        q, k, v, cu = workloads.varlen_inputs(LENGTHS, H, d, dtype, seed=d + 5)
    else:
        rate = 0.5 if dtype == "bf16" else 0.1
        parts = [workloads.moving_max_inputs(1, H, n, d, dtype, seed=n + d, rate=rate)
                 for n in LENGTHS]
        q, k, v = (torch.cat([p[i][0].transpose(0, 1) for p in parts], dim=0).contiguous()
                   for i in range(3))
        cu = workloads.cu_seqlens_of(LENGTHS)
    scale = 1.0 / math.sqrt(d)
    o, lse = run_varlen(q, k, v, cu, max(LENGTHS), scale, dev)
    checked = 0
    for s, n in enumerate(LENGTHS):
        if n > 2048:
            continue  # dense N > 2048 would run 8 waves as well
        a, e = int(cu[s]), int(cu[s + 1])
        # [n, H, d] -> dense [1, H, n, d]
        qs, ks, vs = (t[a:e].transpose(0, 1).unsqueeze(0).contiguous() for t in (q, k, v))
        od, ld = run_dense(qs, ks, vs, scale, dev)
        assert torch.equal(o[a:e].transpose(0, 1), od[0]), f"O differs for sequence {s} (n={n})"
        assert torch.equal(lse[:, a:e], ld[0]), f"L differs for sequence {s} (n={n})"
        checked += 1
    assert checked == len(LENGTHS) - 1
