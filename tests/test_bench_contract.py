"""bench.py's host side, on the CPU: the one-GPU refusal and the work counts behind its rates."""

import os
import subprocess
import sys

import numpy as np

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and not r.stdout.strip()


def test_prefill_flops_match_the_closed_form():
    """Chunked prefill: every query i of a row with prefix P sees P + i + 1 keys, so the visible
    pairs of a row are 512 P + 512 * 513 / 2, and each pair costs 4 * 128 FLOPs per query head."""
    b = workloads.chunked_prefill(canary=False)
    prefixes = (0, 1024, 2048, 3584)
    pairs = sum(512 * p + 512 * 513 // 2 for p in prefixes)
    assert bench.prefill_flops(b) == 4 * 128 * 32 * pairs == 64_441_286_656


def test_decode_bytes_of_a_hand_counted_batch():
    """Rows of 3, 17 and 0 keys, Hq=8, Hkv=2: K and V of 20 keys x 2 heads x 256 B each
    (20,480 B), q and out 3 x 8 x 256 B each (12,288 B), lse 3 x 8 x 4 B (96 B), and the
    metadata read: indptr 4, indices 3 (one page, two pages, none), last_page_len 3 and query
    positions 3 int32s (52 B)."""
    b = workloads.make_batch(7, [3, 17, 0], q_len=1, num_q_heads=8, num_kv_heads=2, num_pages=16)
    assert b.nnz == 3
    assert bench.decode_bytes(b) == 20_480 + 12_288 + 96 + 52


def test_decode_bytes_of_the_benchmarked_batch():
    b = workloads.qwen3_8b_decode(canary=False)
    keys = int(np.sum(b.lengths))
    assert keys == 77_078 and b.batch == 32
    assert bench.decode_bytes(b) == 158_139_652
