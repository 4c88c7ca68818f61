"""Host-side checks of bench.py (no GPU): the one-GPU contract, the
algorithmic bytes / FLOPs of a layer call, and the traffic record's gating."""
import dataclasses
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import get_config  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_work_of_a_layer_call():
    # per token (T = 1) of the 4K-layer shape, K (64, 32, 2) and V (160, 64, 4):
    # bytes = 2 (64 + 160) + 8 (128 (2 + 4) / 8 + 4 + 4) = 1280 plus the
    # T-independent factor, Pi and query terms; FLOPs = 8 (2*64*32 + 2 (32 + 128) 128)
    # + 32 * 2 * 128 + 32 * 2 (160 + 128) = 387072
    cfg = dataclasses.replace(get_config(1), T=1)
    alloc = [((64, 32, 2), (160, 64, 4))]
    nbytes, flops = bench.algorithmic(cfg, alloc, 0)
    fixed = 2 * (8 * (64 * 32 + 160 * 64) + 128 * (32 + 64)) + 2 * 128 * 128 + 32 * 128 * (2 + 4)
    assert nbytes == 1280 + fixed
    assert flops == 387072
    # T scales the per-token terms only
    cfg2 = dataclasses.replace(cfg, T=1000)
    nb2, fl2 = bench.algorithmic(cfg2, alloc, 0)
    assert nb2 == 1000 * 1280 + fixed and fl2 == 1000 * 387072
    # no residual: the inverse-rotation FLOPs and the code bytes drop out
    nb3, fl3 = bench.algorithmic(cfg, [((64, 32, 0), (160, 64, 0))], 0)
    assert nb3 == 2 * (64 + 160) + fixed
    assert fl3 == 8 * (2 * 64 * 32 + 2 * 32 * 128) + 32 * 2 * 128 + 32 * 2 * 160


def test_traffic_record_is_used_only_for_the_same_kernel_sources(tmp_path, monkeypatch):
    from compressed_cache_decode_jolt_amd.profiling import kernel_hash
    (tmp_path / "profiles").mkdir()
    rec = {"w/k": {"kernel_hash": kernel_hash(), "bytes_per_launch": 123.0},
           "w/old": {"kernel_hash": "0" * 16, "bytes_per_launch": 456.0}}
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("w", "k") == 123.0
    assert bench.measured_traffic("w", "old") is None
    assert bench.measured_traffic("w", "missing") is None
