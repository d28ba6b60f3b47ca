"""Host-side arithmetic of bench.py (byte accounting) and its one-GPU contract; no GPU needed."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_attention_bytes_by_hand():
    # two sequences of 20 and 40 tokens, 4 query heads over 2 KV heads, D 8, bs 16, fp16
    p1, tot = bench.attention_bytes([20, 40], 4, 2, 8, 16, 2)
    kv = (20 + 40) * 2 * 8 * 2 * 2          # tokens x Hkv x D x (K and V) x bytes
    tables = (2 + 3) * 4                     # ceil(20/16) + ceil(40/16) block ids
    q = 2 * 4 * 8 * 2
    assert p1 == kv + tables + q + 2 * 4
    assert tot == p1 + 2 * 4 * 8 * 2         # plus the output


def test_unique_bytes_count_shared_blocks_once():
    # block 5 is shared by both sequences (full for both); block 3 is read 8 rows deep
    tab = np.array([[5, 7, -1], [5, 9, 3]], dtype=np.int32)
    ctx = np.array([20, 40])
    rows = 16 + 4 + 16 + 8
    assert bench.unique_kv_bytes(tab, ctx, 1, 1, 16, 1) == rows * 2
    # no sharing: unique equals logical
    tab2 = np.array([[1, 2, -1], [4, 6, 0]], dtype=np.int32)
    assert bench.unique_kv_bytes(tab2, ctx, 3, 8, 16, 2) == (20 + 40) * 3 * 8 * 2 * 2


def test_shared_block_read_to_different_depths():
    # a block shared by beams that read it to different depths counts at the deepest read
    tab = np.array([[2], [2], [2]], dtype=np.int32)
    assert bench.unique_kv_bytes(tab, np.array([3, 9, 5]), 1, 1, 16, 1) == 9 * 2


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
