"""Host logic of bench.py (no GPU): the algorithmic byte counts behind the
roofline, the reading of the committed HBM-traffic summary, and the one-GPU
guard of the command line."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import tq_synth  # noqa: E402


def test_decode_bytes_closed_form():
    # stress70b: 32 rows x 8 KV heads x 32768 tokens x (3-bit key record 48 B +
    # norm 4 B + value codes 48 B + norm 4 B), bf16 query in and fp32 output of
    # 32 x 64 heads x 128, and both 128 x 128 fp32 rotations
    w = tq_synth.WORKLOADS["stress70b"]
    assert bench.decode_bytes(w, w.T) == 32 * 8 * 32768 * 104 + 32 * 64 * 128 * 6 + 2 * 128 * 128 * 4
    assert bench.decode_bytes(w, w.T) == 874_119_168
    # the other workloads (4-bit keys and 2-bit values; QJL keys add 16 sign
    # bytes and a 4-byte gamma per token)
    q = tq_synth.WORKLOADS["qwen"]
    assert bench.decode_bytes(q, q.T) == 4 * 4 * 131072 * (64 + 4 + 32 + 4) + 4 * 28 * 128 * 6 + 131072
    j = tq_synth.WORKLOADS["qjl"]
    assert bench.decode_bytes(j, j.T) == 16 * 8 * 8192 * (32 + 4 + 20 + 48 + 4) + 16 * 32 * 128 * 6 + 131072


def _summary(tmp_path, workload, sha, traffic="878741648"):
    p = tmp_path / "traffic.md"
    p.write_text("# title\n\nprose = with spaces is ignored\n\n```\n"
                 f"workload={workload}\ntraffic_bytes_per_launch={traffic}\n"
                 f"algorithmic_bytes_per_launch=874119168\nkernel_source_sha256={sha}\n```\n")
    return str(p)


def test_recorded_traffic_needs_matching_sources(tmp_path, monkeypatch):
    sha = bench.kernel_source_hash()
    monkeypatch.setattr(bench, "TRAFFIC_FILE", _summary(tmp_path, "stress70b", sha))
    assert bench.recorded_traffic("stress70b") == 878741648
    assert bench.recorded_traffic("llama8b") is None            # another workload
    monkeypatch.setattr(bench, "TRAFFIC_FILE", _summary(tmp_path, "stress70b", "0" * 64))
    assert bench.recorded_traffic("stress70b") is None          # older kernel sources
    monkeypatch.setattr(bench, "TRAFFIC_FILE", _summary(tmp_path, "stress70b", sha, traffic="n/a"))
    assert bench.recorded_traffic("stress70b") is None          # unreadable figure
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.md"))
    assert bench.recorded_traffic("stress70b") is None


def test_committed_traffic_summary_is_well_formed():
    with open(bench.TRAFFIC_FILE) as f:
        kv = dict(line.strip().split("=", 1) for line in f if "=" in line and " " not in line.split("=")[0])
    w = tq_synth.WORKLOADS[kv["workload"]]
    assert int(kv["algorithmic_bytes_per_launch"]) == bench.decode_bytes(w, w.T)
    # the cache is read once: measured traffic within 2 % of the algorithmic bytes
    ratio = int(kv["traffic_bytes_per_launch"]) / int(kv["algorithmic_bytes_per_launch"])
    assert 1.0 <= ratio < 1.02
    assert len(kv["kernel_source_sha256"]) == 64


@pytest.mark.parametrize("argv", [["--gpus", "2"], ["--gpus", "8"]])
def test_more_than_one_gpu_is_refused(argv):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv, capture_output=True, text=True,
                       timeout=120, env={**os.environ, "WORLD_SIZE": "1"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
