"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer,
without a GPU.

exact_attention_26_amd/csrc/fa_api.hip (argument validation, size and
alias arithmetic, grid sizing, problem descriptions) is compiled as plain
C++ with g++ -fsanitize=address,undefined, linked with tests/abi_hostcheck.cpp,
whose stub launchers check the problem description each entry point builds
and count launches. Every validation case of test_abi.py is replayed through
it (same arguments, same expected status), plus calls that pass validation
and reach a launcher, including sizes near the 32-bit and grid limits. Any
sanitizer report aborts the run and fails the test.
"""
import math
import os
import shutil
import subprocess

import pytest

import test_abi as abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_attention_26_amd", "csrc")


class Recorder:
    """Stands in for the loaded library: records each call instead of making it."""

    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        def record(*args):
            self.calls.append((name, args))
            return len(self.calls) - 1
        return record


def _arg(x) -> str:
    if x is None:
        return "0"
    if isinstance(x, float):
        if math.isnan(x):
            return "nan"
        if math.isinf(x):
            return "inf" if x > 0 else "-inf"
        return x.hex()
    return str(int(x))


@pytest.fixture(scope="module")
def hostcheck(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    out = str(tmp_path_factory.mktemp("hostcheck") / "abi_hostcheck")
    cmd = [gxx, "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, "-x", "c++", os.path.join(CSRC, "fa_api.hip"),
           "-x", "c++", os.path.join(ROOT, "tests", "abi_hostcheck.cpp"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "asan" in (r.stderr or "").lower():
        pytest.skip("sanitizer runtime not available: " + r.stderr[-300:])
    assert r.returncode == 0, r.stderr[-3000:]
    return out


def _collect():
    """(call, expected status, expected launches) for every case."""
    rec = Recorder()
    expect = []

    def add(builder, cases, status=None, launches=0, **fixed):
        for case in cases:
            kw, st = (case, status) if status is not None else case
            idx = builder(rec, **{**fixed, **kw})
            expect.append((idx, st, launches))

    add(abi.dense, abi.DENSE_VALIDATION_CASES)
    add(abi.dense, abi.DENSE_EMPTY_IS_NOOP_CASES, status=0)
    add(abi.varlen, abi.VARLEN_VALIDATION_CASES)
    add(abi.varlen, abi.VARLEN_EMPTY_IS_NOOP_CASES, status=0)
    add(abi.bwd, abi.BWD_VALIDATION_CASES)
    add(abi.bwd, abi.BWD_EMPTY_IS_NOOP_CASES, status=0)
    add(abi.banded, abi.BANDED_VALIDATION_CASES)
    add(abi.banded, abi.BANDED_EMPTY_IS_NOOP_CASES, status=0)
    add(abi.kv_outer, abi.KV_OUTER_VALIDATION_CASES)
    add(abi.kv_outer, abi.KV_OUTER_EMPTY_IS_NOOP_CASES, status=0)
    add(abi.norm, abi.NORM_VALIDATION_CASES)
    add(abi.norm, abi.NORM_EMPTY_IS_NOOP_CASES, status=0)

    # Calls that pass validation and reach a launcher. The fake buffers sit
    # 2^40 bytes apart, so even the largest problems below do not overlap.
    far = {k: (i + 1) << 40 for i, k in enumerate(("Q", "K", "V", "O", "L"))}
    # fp32: B*H*ceil(N/128) below 256 runs the key-split form, the stub checks
    # which form each call takes (255 and 256 workgroups sit on either side).
    f32 = abi.fa.FA_F32
    ok_dense = [dict(), dict(N=1), dict(N=2049, d=128), dict(dtype=f32, N=300),
                dict(dtype=f32, B=1, H=255, N=100), dict(dtype=f32, B=1, H=256, N=100, d=128),
                dict(dtype=f32, B=2, H=128, N=200), dict(dtype=f32, B=1, H=1, N=1),
                dict(B=1, H=1, N=(1 << 24) - 1, d=64), dict(B=524287, H=1, N=4096, d=64)]
    add(abi.dense, ok_dense, status=0, launches=1, **far)
    ok_varlen = [dict(), dict(maxlen=300), dict(maxlen=4097, T=9000), dict(nseq=65, T=7000),
                 dict(dtype=abi.fa.FA_F32),
                 dict(maxlen=(1 << 20) - 256, T=1 << 20, H=16, d=128)]
    add(abi.varlen, ok_varlen, status=0, launches=1, cu=6 << 40, **far)
    ok_banded = [dict(), dict(window=0), dict(window=1 << 30), dict(N=5000, window=3000)]
    add(abi.banded, ok_banded, status=0, launches=1, **far)
    far_kv = {k: (i + 1) << 40 for i, k in enumerate(("Q", "K", "V", "O", "L", "acc"))}
    add(abi.kv_outer, [dict(), dict(groups=1 << 20), dict(N=4097, d=128)], status=0, launches=1,
        **far_kv)
    far_bw = {k: (i + 1) << 40 for i, k in enumerate(abi.BW)}
    add(abi.bwd, [dict(), dict(N=1), dict(N=8192, d=128, B=2, H=32)], status=0, launches=1,
        **far_bw)
    far_nm = {k: (i + 1) << 40 for i, k in enumerate(abi.NM)}
    add(abi.norm, [dict(), dict(p=0.0), dict(hidden=8192, rows=100000), dict(kind=1)], status=0,
        launches=1, **far_nm)
    add(abi.norm, [dict(x1=0, res=0, g1=0, b1=0, y1=0, z=0, mean=0, rstd=0, mask=0)], status=0,
        launches=1, **{k: v for k, v in far_nm.items()})
    for args, st in abi.TRACE_CASES:
        expect.append((rec.fa_debug_fwd_trace(*args), st, 0))
    for code in list(abi.fa.STATUS) + [12345]:
        expect.append((rec.fa_strerror(code), 0, 0))
    expect.append((rec.fa_version(), 700, 0))
    return rec.calls, expect


def test_validation_matrix_under_sanitizers(hostcheck):
    calls, expect = _collect()
    stdin = "".join(" ".join([name] + [_arg(a) for a in args]) + "\n" for name, args in calls)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([hostcheck], input=stdin, capture_output=True, text=True, env=env,
                       timeout=120)
    assert r.returncode == 0, f"sanitized run failed ({r.returncode}):\n{r.stderr[-4000:]}"
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr[-4000:]
    got = [tuple(int(x) for x in ln.split()) for ln in r.stdout.splitlines()]
    assert len(got) == len(calls)
    bad = []
    for idx, status, launches in expect:
        if got[idx] != (status, launches):
            bad.append((calls[idx], got[idx], (status, launches)))
    assert not bad, "status/launch mismatches:\n" + "\n".join(map(str, bad[:20]))
    assert len(expect) > 150
