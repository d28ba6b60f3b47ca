"""Pins for the oracle's e4m3fn codec.

The format facts come from "Where Did the VRAM Go (KV cache tutorial)", §6.2
(1 sign, 4 exponent, 3 mantissa bits; largest value 448; relative precision
about 1/8). The library pin is PyTorch's float8_e4m3fn conversion, which
rounds to nearest-even like the oracle and differs only by producing NaN for
inputs above 464, the midpoint between 448 and the next binade step 480 (the
oracle saturates to 448 there).
"""
import math

import numpy as np
import pytest
import torch

from oracle import fp8


def test_format_facts():
    assert fp8.decode(0x7E) == 448.0  # largest finite
    assert fp8.decode(0xFE) == -448.0
    assert math.isnan(fp8.decode(0x7F)) and math.isnan(fp8.decode(0xFF))
    assert fp8.decode(0x08) == 2.0 ** -6  # smallest normal
    assert fp8.decode(0x01) == 2.0 ** -9  # smallest subnormal
    assert fp8.decode(0x38) == 1.0  # exponent field 7 = bias
    assert fp8.decode(0x00) == 0.0 and math.copysign(1, fp8.decode(0x80)) < 0
    finite = [fp8.decode(c) for c in range(128) if not math.isnan(fp8.decode(c))]
    assert max(finite) == 448.0
    # 3 mantissa bits: 8 codes per binade, relative spacing 1/8 at the bottom of a binade
    for e in range(1, 16):
        lo = fp8.decode(e << 3)
        nxt = fp8.decode((e << 3) | 1)
        assert (nxt - lo) / lo == 1.0 / 8.0


def test_decode_all_codes_vs_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = fp8.decode_table()
    both_nan = np.isnan(ref) & np.isnan(ours)
    assert np.array_equal(np.where(both_nan, 0, ref), np.where(both_nan, 0, ours))
    assert np.array_equal(np.isnan(ref), np.isnan(ours))


def test_roundtrip_every_finite_code():
    for c in range(256):
        v = fp8.decode(c)
        if not math.isnan(v):
            assert fp8.encode(v) == c, hex(c)


@pytest.mark.parametrize("inv_scale", [1.0, 448.0 / 5.25, 0.731, 37.0])
def test_encode_every_fp16_input_vs_torch(inv_scale):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = bits.view(np.float16)
    x = x[np.isfinite(x)]
    ours = fp8.quantize(x, inv_scale)
    xs = x.astype(np.float32) * np.float32(inv_scale)
    in_range = np.abs(xs) <= 464.0  # torch gives NaN above 464
    ref = torch.from_numpy(xs[in_range]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours[in_range], ref)
    # saturation: everything above 464 is +-448
    over = ~in_range
    if over.any():
        expect = np.where(xs[over] > 0, 0x7E, 0xFE).astype(np.uint8)
        assert np.array_equal(ours[over], expect)


def test_relative_error_bound():
    # round to nearest with 3 mantissa bits: error <= 2^-4 relative in the normal range
    g = np.random.default_rng(7)
    x = g.uniform(2.0 ** -6, 448.0, size=4000) * g.choice([-1, 1], size=4000)
    for v in x:
        r = fp8.decode(fp8.encode(float(v)))
        assert abs(r - v) <= abs(v) * 2.0 ** -4 * (1 + 1e-12)


def test_ties_to_even():
    # 1 + 1/16 lies halfway between 1 (mantissa 0, even) and 1 + 1/8 (mantissa 1)
    assert fp8.encode(1.0 + 1.0 / 16) == 0x38
    # 1 + 3/16 lies halfway between 1 + 1/8 (odd) and 1 + 2/8 (even)
    assert fp8.encode(1.0 + 3.0 / 16) == 0x3A
    # halfway between the two smallest subnormals 2^-9 and 2^-8 -> 2^-8 (m=2, even)
    assert fp8.encode(1.5 * 2.0 ** -9) == 0x02
    # below half of the smallest subnormal -> 0
    assert fp8.encode(0.49 * 2.0 ** -9) == 0x00
    assert fp8.encode(-0.0) == 0x80


# ---------------------------------------------------------------- e5m2
# Format facts from "Where Did the VRAM Go (KV cache tutorial)", §6.2: one more
# exponent bit and one less mantissa bit than e4m3 (larger range, coarser
# steps). Library pin: PyTorch's float8_e5m2. Closed form: e5m2 has fp16's
# exponent layout, so an fp16 value's e5m2 code is its 15-bit magnitude
# pattern divided by 256 and rounded to nearest even (subnormals included).

def test_e5m2_format_facts():
    d = fp8.decode_e5m2
    assert d(0x7B) == 57344.0 and d(0xFB) == -57344.0  # largest finite: 1.75 * 2^15
    assert d(0x7C) == math.inf and d(0xFC) == -math.inf
    assert all(math.isnan(d(c)) for c in (0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF))
    assert d(0x04) == 2.0 ** -14 and d(0x01) == 2.0 ** -16 and d(0x3C) == 1.0
    for e in range(1, 31):  # 2 mantissa bits: relative spacing 1/4 at the bottom of a binade
        assert (d((e << 2) | 1) - d(e << 2)) / d(e << 2) == 0.25
    finite = [d(c) for c in range(128) if math.isfinite(d(c))]
    assert max(finite) == 57344.0


def test_e5m2_decode_all_codes_vs_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e5m2).to(torch.float64).numpy()
    ours = fp8.decode_table("e5m2")
    assert np.array_equal(np.isnan(ref), np.isnan(ours))
    m = ~np.isnan(ref)
    assert np.array_equal(ref[m], ours[m])


def test_e5m2_roundtrip_every_finite_code():
    for c in range(256):
        v = fp8.decode_e5m2(c)
        if math.isfinite(v):
            assert fp8.encode_e5m2(v) == c, hex(c)


def test_e5m2_fp16_closed_form():
    bits = np.arange(65536, dtype=np.uint32)
    x = bits.astype(np.uint16).view(np.float16)
    fin = np.isfinite(x)
    ours = fp8.quantize(x[fin], 1.0, "e5m2")
    mag = (bits[fin] & 0x7FFF).astype(np.int64)
    q, r = np.divmod(mag, 256)
    q = q + ((r > 128) | ((r == 128) & (q & 1 == 1)))
    q = np.minimum(q, 0x7B)  # saturation
    sign = ((bits[fin] >> 8) & 0x80).astype(np.int64)
    assert np.array_equal(ours, (sign | q).astype(np.uint8))


@pytest.mark.parametrize("inv_scale", [1.0, 57344.0 / 5.25, 0.731, 4096.0])
def test_e5m2_encode_every_fp16_input_vs_torch(inv_scale):
    x = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    x = x[np.isfinite(x)]
    ours = fp8.quantize(x, inv_scale, "e5m2")
    xs = x.astype(np.float32) * np.float32(inv_scale)
    in_range = np.abs(xs) < 61440.0  # torch rounds to infinity from the midpoint 61440 up
    ref = torch.from_numpy(xs[in_range]).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(ours[in_range], ref)
    over = ~in_range
    if over.any():
        assert np.array_equal(ours[over], np.where(xs[over] > 0, 0x7B, 0xFB).astype(np.uint8))


def test_e5m2_ties_and_error_bound():
    assert fp8.encode_e5m2(1.0 + 1.0 / 8) == 0x3C      # halfway 1 (m=0) .. 1.25 (m=1) -> even
    assert fp8.encode_e5m2(1.0 + 3.0 / 8) == 0x3E      # halfway 1.25 (m=1) .. 1.5 (m=2) -> even
    assert fp8.encode_e5m2(1.5 * 2.0 ** -16) == 0x02   # between the two smallest subnormals
    assert fp8.encode_e5m2(math.inf) == 0x7B and fp8.encode_e5m2(-1e9) == 0xFB
    g = np.random.default_rng(3)
    for v in g.uniform(2.0 ** -14, 57344.0, size=3000) * g.choice([-1, 1], size=3000):
        assert abs(fp8.decode_e5m2(fp8.encode_e5m2(float(v))) - v) <= abs(v) * 2.0 ** -3 * (1 + 1e-12)


# ---------------------------------------------------------------- per-head scales
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_per_head_scales_apply_head_by_head(fmt):
    """A per-head scale vector gives each KV head's rows exactly the bytes a
    per-tensor scale of that head's value would ("Where Did the VRAM Go", §6.3)."""
    g = np.random.default_rng(5)
    x = (g.standard_normal((7, 4, 16)) * 3).astype(np.float16)   # [T, Hkv, D]
    inv = np.array([1.0, 85.3, 0.5, 12.25], dtype=np.float32)
    q = fp8.quantize(x, inv, fmt)
    for h in range(4):
        assert np.array_equal(q[:, h, :], fp8.quantize(x[:, h, :], float(inv[h]), fmt))
    rows = np.transpose(q, (1, 0, 2))                              # cache rows [Hkv, n, D]
    scale = np.float32(1.0) / inv
    deq = fp8.dequantize(rows, scale, fmt)
    for h in range(4):
        assert np.array_equal(deq[h], fp8.dequantize(rows[h], float(scale[h]), fmt))
