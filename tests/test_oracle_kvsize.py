"""Pins for the closed forms, against the numbers the pages print.

* OPT-13B, 2048 tokens: about 1.6 GB ("From OOM to Smooth Inference", §1.1).
* Llama-2-7B (32 layers, 32 KV heads, head_dim 128, fp16), 2048 tokens: about
  1 GB ("Inference Engine Memory Optimisation", §2.1).
* Qwen3-0.6B: about 112 KB per token, 448 MiB for a 4k sequence ("Where Did
  the VRAM Go (KV cache tutorial)", §1.4); 8 KV heads x 128 from the model
  card shape used by the Qwen3 workload, 28 layers solves 112 KiB exactly.
* Reservation waste 84.7% and 56.3% ("From OOM to Smooth Inference", §1.2).
* Internal fragmentation at most block_size - 1, i.e. 15 tokens at 16
  ("From OOM to Smooth Inference", §2.1; "Where Did the VRAM Go", §3.3).
* About 4000 blocks of 16 tokens for OPT-13B on an 80 GB H100 ("From OOM to
  Smooth Inference", §2.3 docstring).
"""
from oracle import kvsize

GiB = 1024 ** 3
MiB = 1024 ** 2


def test_opt13b_2048_tokens():
    b = kvsize.kv_bytes(layers=40, kv_heads=40, head_dim=128, seq_len=2048, elem_bytes=2)
    assert b == 1_677_721_600
    assert round(b / GiB, 1) == 1.6  # 1.5625 GiB
    # the page's numeric form: 2 x 5120 (hidden) x 40 (layers) x 2 bytes x 2048
    assert b == 2 * 5120 * 40 * 2 * 2048


def test_llama2_7b_2048_tokens():
    assert kvsize.kv_bytes(32, 32, 128, 2048, 2) == 1 * GiB


def test_qwen3_0p6b():
    per_tok = kvsize.kv_bytes_per_token(layers=28, kv_heads=8, head_dim=128, elem_bytes=2)
    assert per_tok == 112 * 1024
    assert kvsize.kv_bytes(28, 8, 128, 4096, 2) == 448 * MiB


def test_reservation_waste():
    assert round(100 * kvsize.reservation_waste(312, 2048), 1) == 84.8 or \
        abs(100 * kvsize.reservation_waste(312, 2048) - 84.7) < 0.1
    assert round(100 * kvsize.reservation_waste(896, 2048), 1) == 56.2 or \
        abs(100 * kvsize.reservation_waste(896, 2048) - 56.3) < 0.1


def test_internal_fragmentation_bound():
    for bs in (8, 16, 32, 64):
        worst = max(kvsize.internal_fragmentation(t, bs) for t in range(1, 10 * bs))
        assert worst == bs - 1
    assert kvsize.internal_fragmentation(17, 16) == 15
    assert kvsize.internal_fragmentation(32, 16) == 0


def test_opt13b_pool_on_80gb():
    # 80 GB card, ~26 GB of fp16 OPT-13B weights, the rest for KV
    blocks = kvsize.pool_blocks(80 * 10 ** 9 - 26 * 10 ** 9, 16, 40, 40, 128, 2)
    assert 3500 <= blocks <= 4500
    # the per-block size form: block_size x heads x head_dim x 2 x bytes, per layer
    assert kvsize.kv_bytes_per_token(1, 40, 128, 2) * 16 == 16 * 40 * 128 * 2 * 2
