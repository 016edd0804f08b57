"""CPU checks of bench.py's measurement arithmetic (no GPU): the algorithmic
bytes the roofline divides by, for the workloads whose totals were worked
out independently from the shapes (packed INT4 weights + fp16 group scales,
the INT4 KV cache read including the new token, the append, fp32 residual in
and out), and the one-GPU guard."""

import os
import subprocess
import sys

import numpy as np

import bench
from int4_weight_kv_amd import workload as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _block_bytes(wl):
    return bench.algorithmic_bytes(wl.dims, wl.cached_lengths(0))


def test_block_bytes_8b_batch1():
    # 112,459,776 weights+scales + 2049 tokens x 1056 B + 1056 B append + 8 x 4096 B residual
    assert 112_459_776 + 2049 * 1056 + 1056 + 8 * 4096 == 114_657_344
    assert _block_bytes(W.llama8b(1)) == 114_657_344


def test_block_bytes_tiny():
    # 417,792 weights+scales; KV 136 B per token (2 heads x 2 x (32 + 2))
    assert _block_bytes(W.tiny(1)) == 417_792 + 129 * 136 + 136 + 8 * 256


def test_block_bytes_70b_batch1():
    assert _block_bytes(W.llama70b(1)) == 441_188_352 + 4097 * 1056 + 1056 + 8 * 8192


def test_weight_bytes_per_projection():
    d = W.LLAMA8B
    assert bench.weight_bytes(6144, 4096, 128) == 6144 * 2048 + 6144 * 32 * 2
    assert bench.gateup_bytes(d, 1) == 60_600_320


def test_full_step_bytes():
    for batch, want in ((1, 4_927_847_424), (16, 9_104_769_024)):
        wl = W.llama8b_full_step(batch)
        assert bench.step_bytes_full(wl, wl.cached_lengths(0)) == want


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_ragged_lengths_in_range():
    lens = W.llama8b_ragged(32).cached_lengths(0)
    assert lens.min() >= 512 and lens.max() <= 4096 and len(np.unique(lens)) > 16
