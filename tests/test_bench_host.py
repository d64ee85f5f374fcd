"""bench.py's contract on the host (no GPU): argument checks that exit
before any device work, the algorithmic byte counts it divides by, and the
rule that counter traffic is reported only while the kernel sources match
the ones the counters were taken with."""
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.join(os.path.dirname(__file__), "..")


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_exits_with_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


def test_bad_step_counts_rejected():
    assert _run("--steps", "0").returncode != 0
    assert _run("--warmup", "-1").returncode != 0


def test_gateup_bytes_per_launch(bench):
    # 6 experts x (gate + up) x 2048 rows x 16 Q2_K blocks of 84 B, plus x in
    # and the SwiGLU row out in f32
    assert bench.GATEUP_BYTES == 6 * 2 * 2048 * 16 * 84 + 4096 * 4 + 6 * 2048 * 4 == 33_095_680


def test_decode_step_bytes(bench):
    # one token: 6 pairs, each reading its expert's gate, up and down rows
    # (8,257,536 B per expert); x read, y written, 256 logits read
    assert bench.decode_bytes(6, 1) == 6 * 8_257_536 + 4096 * 4 * 2 + 256 * 4


def test_counter_traffic_needs_matching_sources(bench, monkeypatch, tmp_path):
    line = ('traffic_json: {"kernel": "decode_gateup", "src_sha256": "abc", "fetch_kib": 100.0, '
            '"write_kib": 10.0, "fetch_factor": 2.0, "write_factor": 1.0, "dispatches": 1}\n')
    f = tmp_path / "counters.txt"
    f.write_text("header\n" + line)
    monkeypatch.setattr(bench, "COUNTER_FILE", str(f))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda sources=None: "abc")
    assert bench.counter_traffic("decode_gateup") == (100 * 2 + 10) * 1024
    assert bench.counter_traffic("decode_down") is None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda sources=None: "changed")
    assert bench.counter_traffic("decode_gateup") is None
    monkeypatch.setattr(bench, "COUNTER_FILE", str(tmp_path / "missing.txt"))
    assert bench.counter_traffic("decode_gateup") is None
