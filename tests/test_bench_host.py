"""Host logic of bench.py: the algorithmic bytes per frame behind its roofline figures, and the
one-GPU contract.  The expected values are the per-frame byte counts of the frame step worked out
from the Moshi-7B shape (weights 14,749,270,016 bf16 bytes; a cached position holds k and v of 32
layers x 4096 values)."""
import os
import subprocess
import sys

import numpy as np

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

W7B = 14_749_270_016


def test_frame_bytes_from_offset_zero():
    # 250 frames at positions 0..249: n = pos + 1 cached positions, mean 125.5; float32 KV
    fb = bench.frame_bytes(W7B, synth.MOSHI7B, 4, np.arange(250))
    assert fb == W7B + 125.5 * 32 * 2 * 4096 * 4 == 14_880_866_304
    # the same positions with a bf16 cache: 65.8 MB of KV per frame on average
    kv = bench.frame_bytes(W7B, synth.MOSHI7B, 2, np.arange(250)) - W7B
    assert abs(kv - 65.8e6) < 0.05e6


def test_frame_bytes_long_context_and_window():
    # positions 2900..2999: mean n = 2950.5, 1.547 GB of bf16 KV per frame
    kv = bench.frame_bytes(W7B, synth.MOSHI7B_LONG, 2, np.arange(2900, 3000)) - W7B
    assert kv == 2950.5 * 32 * 2 * 4096 * 2
    assert abs(kv - 1.547e9) < 0.001e9
    # past the 3000-position context the window holds exactly 3000 positions
    kv = bench.frame_bytes(W7B, synth.MOSHI7B_LONG, 2, np.arange(3000, 3010)) - W7B
    assert kv == 3000 * 32 * 2 * 4096 * 2


def test_frame_bytes_batched_sums_conversations():
    # two conversations at offsets 0 and 10, three frames each: per frame the weights once plus
    # both conversations' KV
    pos = np.array([[0, 1, 2], [10, 11, 12]])
    per_pos = 32 * 2 * 4096 * 4
    fb = bench.frame_bytes(W7B, synth.MOSHI7B_B64, 4, pos)
    assert fb == W7B + np.mean([1 + 11, 2 + 12, 3 + 13]) * per_pos


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
