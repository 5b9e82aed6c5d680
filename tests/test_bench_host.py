"""Host-side logic of bench.py (no GPU): the one-GPU contract, the credited
work figures the throughput numbers divide by, and the guard that drops
committed HBM-traffic counters once the kernel source they were taken from
has changed."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth_inputs as si  # noqa: E402


def test_rejects_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "exactly one GPU" in r.stdout + r.stderr


def test_credited_prefill_flops():
    # 4 N Nk d per head, halved under the causal mask: 137.44 GFLOP at the
    # B64 x H16 x 1024 x 1024, d = 64 prefill.
    s = si.Shape(64, 16, 1024, 1024, 64, 64)
    assert bench.credited_flops(s, True) == 137438953472.0
    assert bench.credited_flops(s, False) == 2 * 137438953472.0


def test_decode_algorithmic_bytes():
    # K and V once (bf16) plus Q, O (bf16) and LSE (fp32): 4,295,099,392 B at
    # B8 x H32, Nk = 32768, d = 128.
    s = si.Shape(8, 32, 1, 32768, 128, 128)
    assert bench.decode_bytes(s) == 4295099392


def _traffic_file(tmp_path, fwd_hash, dec_hash):
    p = tmp_path / "traffic.txt"
    p.write_text("# test\n"
                 "fwd_bytes_per_launch: 1000\n"
                 f"fwd_source_sha256_16: {fwd_hash}\n"
                 "long_bytes_per_launch: 3000\n"
                 "decode_bytes_per_launch: 2000\n"
                 f"decode_source_sha256_16: {dec_hash}\n")
    return str(p)


def test_traffic_kept_while_sources_match(tmp_path, monkeypatch):
    path = _traffic_file(tmp_path, bench.source_hash(bench.FWD_KERNEL_SRC),
                         bench.source_hash(bench.DEC_KERNEL_SRC))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", path)
    assert bench.read_traffic() == {"fwd": 1000.0, "decode": 2000.0, "long": 3000.0}


def test_traffic_dropped_for_changed_source(tmp_path, monkeypatch):
    path = _traffic_file(tmp_path, "0" * 16, bench.source_hash(bench.DEC_KERNEL_SRC))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", path)
    assert bench.read_traffic() == {"fwd": None, "decode": 2000.0, "long": None}


def test_traffic_absent(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.txt"))
    assert bench.read_traffic() == {"fwd": None, "decode": None, "long": None}


@pytest.mark.parametrize("text", ["model name\t: Test CPU 9000\nflags\t: x\n", "flags\t: x\n"])
def test_cpu_model(tmp_path, monkeypatch, text):
    p = tmp_path / "cpuinfo"
    p.write_text(text)
    real_open = open

    def fake_open(path, *a, **k):
        return real_open(p, *a, **k) if path == "/proc/cpuinfo" else real_open(path, *a, **k)

    monkeypatch.setattr("builtins.open", fake_open)
    assert bench.cpu_model() == ("Test CPU 9000" if "model name" in text else "unknown")


def test_credited_long_prefill_flops():
    # 1.0995 TFLOP at B2 x H32 x 8192 x 8192, d = 128, causal.
    s = si.Shape(2, 32, 8192, 8192, 128, 128)
    assert bench.credited_flops(s, True) == 2 * 32 * 4.0 * 8192 * 8192 * 128 / 2


def test_read_sclk(tmp_path):
    # the DPM table format: the current level carries a '*'
    p = tmp_path / "pp_dpm_sclk"
    p.write_text("0: 500Mhz \n1: 2317Mhz *\n2: 2400Mhz \n")
    q = tmp_path / "other"
    q.write_text("0: 500Mhz *\n1: 2400Mhz \n")
    assert bench.read_sclk([str(p), str(q), str(tmp_path / "missing")]) == [2317.0, 500.0]
