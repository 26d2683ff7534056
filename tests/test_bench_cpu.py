"""bench.py's host-side logic, without a GPU: the multi-GPU refusal, the
counter-summary reader and its source-hash check, the clock-sampler helper
protocol, and the byte accounting of the fused norm workloads."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402


def test_more_than_one_gpu_is_refused(monkeypatch, capsys):
    monkeypatch.setattr(sys, "argv", ["bench.py", "--gpus", "2"])
    assert bench.main() == 2
    assert "one GPU only" in capsys.readouterr().err


def test_pmc_reader_checks_the_source_hash(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    # the hash is computed from the real kernel sources
    monkeypatch.setattr(bench, "kernel_source_hash",
                        lambda order="q_outer": {"q_outer": "aaaa", "norm": "bbbb"}[order])
    (prof / "fa_fwd_w_pmc.txt").write_text(
        "# header: not parsed\nkernel_source_sha: aaaa\nhbm_bytes_per_launch: 12345\n")
    assert bench.read_pmc_traffic("w") == 12345
    (prof / "fa_norm_w_pmc.txt").write_text("kernel_source_sha: old\nhbm_bytes_per_launch: 7\n")
    assert bench.read_pmc_traffic("w", order="norm") is None      # stale summary
    assert bench.read_pmc_traffic("missing") is None


def test_source_hash_ignores_comments_only():
    code = "int f(int x) {\n  return x + 1;  // add one\n}\n"
    same = "// header\n/* block\n   comment */\nint f(int x) {\n\n  return x + 1;\n}\n"
    other = "int f(int x) {\n  return x + 2;  // add one\n}\n"
    assert bench.source_code_text(code) == bench.source_code_text(same)
    assert bench.source_code_text(code) != bench.source_code_text(other)


def test_source_hash_is_per_kernel():
    hashes = {k: bench.kernel_source_hash(k) for k in bench.KERNEL_SOURCES}
    assert len(set(hashes[k] for k in ("q_outer", "kv_outer", "norm"))) == 3
    assert hashes["band"] == hashes["q_outer"]  # the banded forward is the same source file


def test_clock_sampler_protocol(tmp_path, monkeypatch):
    fake = tmp_path / "amd-smi"
    fake.write_text("#!/bin/sh\necho 'GPU: 0'\necho '    GFX_0:'\necho '        CLK: 2100 MHz'\n"
                    "echo '    GFX_1:'\necho '        CLK: 1900 MHz'\necho '    MEM_0:'\n"
                    "echo '        CLK: 1300 MHz'\necho '    SOCKET_POWER: 1300 W'\n")
    fake.chmod(0o755)
    monkeypatch.setenv("PATH", f"{tmp_path}:{os.environ['PATH']}")
    import torch
    monkeypatch.setattr(torch.cuda, "synchronize", lambda *a, **k: None)
    bench.start_sclk_sampler()
    try:
        mhz, watts = bench.sample_sclk(lambda: None, seconds=0.2)
    finally:
        bench._sampler.stdin.close()
        bench._sampler.wait(timeout=10)
        bench._sampler = None
    assert mhz == pytest.approx(2000.0) and watts == pytest.approx(1300.0)  # MEM clock excluded


def test_clock_sampler_median_ignores_one_dip(tmp_path, monkeypatch):
    # Five amd-smi samples; the second reads a throttling dip. Each sample is
    # the mean over the GFX domains; the reported figure is their median.
    count = tmp_path / "n"
    count.write_text("0")
    fake = tmp_path / "amd-smi"
    fake.write_text(
        "#!/bin/sh\n"
        f"n=$(cat {count}); echo $((n + 1)) > {count}\n"
        "if [ \"$n\" = 1 ]; then c0=900; c1=1100; w=700; else c0=1800; c1=1600; w=1350; fi\n"
        "echo '    GFX_0:'; echo \"        CLK: $c0 MHz\"; echo '    GFX_1:'\n"
        "echo \"        CLK: $c1 MHz\"; echo '    MEM_0:'; echo '        CLK: 1300 MHz'\n"
        "echo \"    SOCKET_POWER: $w W\"\n")
    fake.chmod(0o755)
    monkeypatch.setenv("PATH", f"{tmp_path}:{os.environ['PATH']}")
    import torch
    monkeypatch.setattr(torch.cuda, "synchronize", lambda *a, **k: None)
    bench.start_sclk_sampler()
    try:
        mhz, watts = bench.sample_sclk(lambda: None, seconds=0.2)
    finally:
        bench._sampler.stdin.close()
        bench._sampler.wait(timeout=10)
        bench._sampler = None
    assert int(count.read_text()) == 5
    assert mhz == pytest.approx(1700.0) and watts == pytest.approx(1350.0)


def test_sampler_absent_gives_nulls(monkeypatch):
    monkeypatch.setattr(bench, "_sampler", None)
    assert bench.sample_sclk(lambda: None, seconds=0.0) == (None, None)


@pytest.mark.parametrize("name", sorted(workloads.NORM_WORKLOADS))
def test_norm_bytes_count_every_tensor_once(name):
    w = workloads.NORM_WORKLOADS[name]
    rows, hidden = w["rows"], w["hidden"]
    inputs = 1 + w["x1"] + w["residual"]
    outputs = 1 + w["gamma1"] + w["prenorm"]
    weights = 2 * (1 + w["gamma1"])
    stats = 1 if w["rms"] else 2
    want = (inputs + outputs) * rows * hidden * 2 + weights * hidden * 2 + stats * rows * 4
    got = workloads.norm_bytes(rows, hidden, 2, w["x1"], w["residual"], w["gamma1"],
                               w["prenorm"], stats=stats)
    assert got == want


def test_seq_len_override_keeps_the_rest_of_the_workload():
    base = workloads.make("short_bf16")
    w = workloads.make("short_bf16", seq_len=96)
    assert (w["B"], w["H"], w["N"], w["d"]) == (base["B"], base["H"], 96, base["d"])
    assert w["q"].shape == (base["B"], base["H"], 96, base["d"]) and w["q"].dtype == base["q"].dtype
    assert w["scale"] == base["scale"]
    with pytest.raises(ValueError):
        workloads.make("varlen_bf16", seq_len=96)


def test_no_sampler_under_a_profiler(monkeypatch):
    monkeypatch.setenv("ROCP_TOOL_LIBRARIES", "/opt/rocm/lib/rocprofiler-sdk/librocprofiler-sdk-tool.so")
    monkeypatch.setattr(bench, "_sampler", None)
    bench.start_sclk_sampler()
    assert bench._sampler is None


def test_cpu_baseline_packed_sample():
    # The oracle leg on a tiny packed batch, with the "GPU" output taken from
    # the oracle itself: the error is 0, the flop count is 4*d*sum(n^2) over
    # the pairs it did, and the CPU model is reported.
    import torch
    import oracle
    lengths = [3, 70, 5]
    q, k, v, cu = workloads.varlen_inputs(lengths, 2, 64, "bf16", seed=4)
    w = {"q": q, "k": k, "v": v, "cu_seqlens": cu, "H": 2, "d": 64, "scale": 0.125,
         "name": "tiny_packed"}
    O_ref, _ = oracle.attention_varlen(q, k, v, cu, 0.125)
    out = bench.cpu_baseline(w, torch.from_numpy(O_ref), budget_s=60.0)
    assert out["max_abs_err_O_vs_gpu"] == 0.0
    assert out["kind"] == "oracle" and out["cores"] >= 1 and out["cpu_model"]
    assert out["sample"].startswith("6 of 6 (sequence, head) pairs")
