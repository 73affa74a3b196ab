"""Host-side logic of bench.py (no GPU): the refusal of several GPUs, the
FLOP convention, the peaks, and how committed profile figures are matched to
the current kernel sources."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_before_touching_the_device():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_causal_flop_count_and_peaks():
    p = dict(B=1, Hq=32, S=32768, Dqk=128, Dv=128)
    # the visible half of the score matrix: B * H * S^2 * (Dqk + Dv)
    assert bench.causal_flops(p) == 8.796093022208e12
    # 256 CUs x 4 SIMDs x {2048, 1024} dense flop per clock x 2.4 GHz
    assert bench.PEAK["fp8"] == pytest.approx(256 * 4 * 2048 * 2.4e9 / 1e12, abs=0.1)
    assert bench.PEAK["bf16"] == pytest.approx(256 * 4 * 1024 * 2.4e9 / 1e12, abs=0.1)


def test_profile_lines_count_only_for_the_current_sources(tmp_path, monkeypatch):
    sha = bench.sources_sha256("fp8")
    assert sha == bench.sources_sha256("fp8") and len(sha) == 64
    f = tmp_path / "traffic.txt"
    f.write_text("# comment\n"
                 f"workload=fp8_mha_s32k kernel=k sources_sha256={'0' * 64} traffic_bytes=1\n"
                 f"workload=fp8_mha_s32k kernel=k sources_sha256={sha} traffic_bytes=1234\n"
                 f"workload=bf16_mha_s32k kernel=k sources_sha256={sha} traffic_bytes=99\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("fp8_mha_s32k", "fp8") == 1234
    # a line taken on other sources (another hash) is not reported
    assert bench.measured_traffic("bf16_mha_s32k", "bf16") is None
    assert bench.profiled_line(str(tmp_path / "missing.txt"), "fp8_mha_s32k", "fp8") is None


def test_source_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    """Profile figures stay attached to a kernel while only its comments
    change; any change to the code itself detaches them."""
    src = tmp_path / "k.hip"
    py = tmp_path / "b.py"
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setitem(bench.KERNEL_SOURCES, "fp8", ["k.hip", "b.py"])

    def sha(code, build):
        src.write_text(code)
        py.write_text(build)
        return bench.sources_sha256("fp8")

    base = sha("int f(int x) {\n  return x + 1;  // one\n}\n", "FLAGS = ['-O3']  # opt\n")
    assert base == sha("/* block\n comment */\nint f(int x) {\n\n  return x + 1;  // another\n}\n",
                       "# header\nFLAGS = ['-O3']\n")
    assert base != sha("int f(int x) {\n  return x + 2;  // one\n}\n", "FLAGS = ['-O3']  # opt\n")
    assert base != sha("int f(int x) {\n  return x + 1;  // one\n}\n", "FLAGS = ['-O2']  # opt\n")
    # a file's code does not leak into its neighbour's: the split point counts
    assert sha("ab", "c") != sha("a", "bc")


def test_balance_bound_of_causal_grids():
    # one workgroup per CU: 4 query heads x 64 blocks of 256 rows at S = 16K;
    # block qb covers 2 qb + 2 key tiles, so the largest load is 128 tiles and
    # the mean 4 * sum(2 qb + 2) / 256 = 65
    assert bench.balance_bound(1, 4, 1, 16384) == pytest.approx(65 / 128)
    # a grid smaller than the chip leaves CUs idle: 2 heads x 1 block
    assert bench.balance_bound(1, 2, 2, 256) == pytest.approx(2 * 2 / 256 / 2)
    # many workgroups, heaviest first, balance well; the bound never exceeds 1
    for B, Hq, Hkv, S in ((1, 32, 32, 32768), (1, 32, 8, 16384), (1, 4, 4, 32768), (2, 6, 3, 5000)):
        b = bench.balance_bound(B, Hq, Hkv, S)
        assert 0 < b <= 1
    assert bench.balance_bound(1, 4, 4, 32768) > 0.98


def test_clock_sampler_averages_its_samples():
    """The clock sampler's thread reads a source until stopped; with no source
    (no driver here) it reports nothing instead of a guess."""
    import time

    ck = bench.ClockSampler(period=0.001)
    vals = iter([1700.0, 1900.0] * 1000)
    ck._read = lambda: next(vals)
    with ck:
        time.sleep(0.05)
    assert ck.samples and abs(ck.mean_mhz() - 1800.0) <= 100.0
    empty = bench.ClockSampler()
    empty._read = None
    with empty:
        pass
    assert empty.mean_mhz() is None and empty.samples == []
