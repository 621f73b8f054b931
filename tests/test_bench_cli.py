"""The benchmark's contract on the host (no GPU): more than one GPU is refused with a message,
a host without a GPU gets an error line, and the byte counts it prices the rooflines with
agree with the workload shapes' sizes."""
import json
import os
import subprocess
import sys

import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


def test_no_gpu_host_gets_an_error_line():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    r = _run("--steps", "1", "--warmup", "0")
    assert r.returncode == 1
    assert json.loads(r.stdout.strip().splitlines()[-1]) == {"error": "no GPU"}


def test_layer_and_kv_bytes_match_the_shapes():
    # 7B layer: q/k/v (3584 x 4608) + o (3584 x 3584) + gate/up/down (3 x 3584 x 18944) bf16,
    # plus q/k/v biases and two norm gains.
    S = synth.QWEN7B
    proj = 3584 * 4608 + 3584 * 3584 + 3 * 3584 * 18944
    assert bench.weight_bytes_per_layer(S) == 2 * (proj + 4608 + 2 * 3584)
    assert round(bench.weight_bytes_per_layer(S) / 1e6, 1) == 466.1
    # 0.5B: 24 layers of 29.8 MB and a 272 MB tied head: about 988 MB of weights per step.
    D = synth.QWEN05B
    assert round(bench.weight_bytes_per_layer(D) / 1e6, 1) == 29.8
    total = D.n_layers * bench.weight_bytes_per_layer(D) + D.vocab * D.hidden * 2 + D.hidden * 2
    assert abs(total - 987.9e6) < 1e6
    # K/V of one position over the 28 layers: 2 (K and V) x 4 heads x 128 x 2 bytes per layer.
    assert bench.kv_cache_bytes(S, 1) == 28 * 2 * 512 * 2
    assert bench.kv_cache_bytes(S, 10, n_layers=14) == 14 * 10 * 2 * 512 * 2


def test_spread_reports_median_and_range():
    s = bench.spread([3.0, 1.0, 2.0, 10.0, 2.5])
    assert s == {"median": 2.5, "min": 1.0, "max": 10.0, "repeats": 5}
