"""OCP FP8 codecs (e4m3fn and e5m2), written from the format definitions.
TEST INFRASTRUCTURE.

Source: "Where Did the VRAM Go (KV cache tutorial)", §6.1-6.3: KV values are
scaled into FP8's range by a scale factor, stored as e4m3 (1 sign bit, 4
exponent bits, 3 mantissa bits, largest value 448, relative precision about
1/8), and multiplied back by the scale when read.

Format (e4m3 "fn" flavour, exponent bias 7):
  * exponent field e in 1..15, mantissa m in 0..7: value = 2^(e-7) * (1 + m/8)
  * e == 0: subnormal, value = 2^-6 * (m/8) = m * 2^-9
  * e == 15 and m == 7 (0x7F / 0xFF): NaN. There is no infinity.
  * largest finite magnitude: e=15, m=6 -> 1.75 * 2^8 = 448.

Encoding reading (the pages fix the format and the scale, not the rounding):
round-to-nearest, ties to even, saturating to +-448 for finite inputs that
round past 448, so 0x7F/0xFF are never produced from finite data. The sign of
zero is kept. NaN input encodes to 0x7F.

The same section names the other FP8 format, e5m2: one more exponent bit and
one less mantissa bit, a larger range and coarser steps. Format (OCP e5m2,
exponent bias 15, IEEE-style specials):
  * exponent field e in 1..30, mantissa m in 0..3: value = 2^(e-15) * (1 + m/4)
  * e == 0: subnormal, value = 2^-14 * (m/4) = m * 2^-16
  * e == 31: m == 0 is +-infinity, m != 0 is NaN
  * largest finite magnitude: e=30, m=3 -> 1.75 * 2^15 = 57344.
Encoding reading, as for e4m3: round to nearest, ties to even, saturating to
+-57344 (finite data never becomes infinity; an infinite input saturates too),
sign of zero kept, NaN -> 0x7F.

Scales may be one value per tensor or one per KV head ("Where Did the VRAM Go
(KV cache tutorial)", §6.3: the granularity can go from one scale per tensor
to one per attention head); a per-head scale applies to every value of that
head's rows.

Everything here is plain Python on exact binary fractions: a float32/float64
input is exact in Python's float, and the rounding is done on integers.
"""
from __future__ import annotations

import functools
import math

import numpy as np

E4M3_MAX = 448.0
_MIN_NORMAL_EXP = -6  # 2^-6 is the smallest normal
_SUBNORMAL_QUANTUM_EXP = -9  # m * 2^-9


def decode(code: int) -> float:
    """Value of one e4m3fn byte as a Python float (exact)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 15 and m == 7:
        return math.nan
    if e == 0:
        return sign * math.ldexp(m, _SUBNORMAL_QUANTUM_EXP)
    return sign * math.ldexp(8 + m, e - 7 - 3)


def _round_half_even(num: int, den_pow2: int) -> int:
    """round(num / 2^den_pow2) with ties to even, for num >= 0 (integers only)."""
    if den_pow2 <= 0:
        return num << (-den_pow2)
    q, r = divmod(num, 1 << den_pow2)
    half = 1 << (den_pow2 - 1)
    if r > half or (r == half and (q & 1)):
        q += 1
    return q


def encode(x: float) -> int:
    """e4m3fn byte nearest to x (ties to even), saturating at +-448."""
    x = float(x)
    if math.isnan(x):
        return 0x7F
    sign = 0x80 if math.copysign(1.0, x) < 0 else 0x00
    a = abs(x)
    if a == 0.0:
        return sign
    if a >= E4M3_MAX:
        return sign | 0x7E
    # a = mant * 2^exp exactly, with mant a 53-bit integer.
    mant, exp = math.frexp(a)  # a = mant * 2^exp, 0.5 <= mant < 1
    mant_int = int(math.ldexp(mant, 53))
    exp_int = exp - 53  # a = mant_int * 2^exp_int
    e_unb = exp - 1  # floor(log2(a))
    if e_unb < _MIN_NORMAL_EXP:
        # subnormal range: count quanta of 2^-9
        q = _round_half_even(mant_int, _SUBNORMAL_QUANTUM_EXP - exp_int)
        # q == 8 is 2^-6, the smallest normal (code 0x08): encoding is continuous
        return sign | q
    # normal range: quantum is 2^(e_unb - 3); q in [8, 16]
    q = _round_half_even(mant_int, (e_unb - 3) - exp_int)
    if q == 16:
        q = 8
        e_unb += 1
    e_field = e_unb + 7
    if e_field > 15 or (e_field == 15 and q - 8 == 7):
        return sign | 0x7E
    return sign | (e_field << 3) | (q - 8)


E5M2_MAX = 57344.0


def decode_e5m2(code: int) -> float:
    """Value of one e5m2 byte as a Python float (exact)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 2) & 0x1F
    m = code & 0x3
    if e == 31:
        return sign * math.inf if m == 0 else math.nan
    if e == 0:
        return sign * math.ldexp(m, -16)
    return sign * math.ldexp(4 + m, e - 15 - 2)


def encode_e5m2(x: float) -> int:
    """e5m2 byte nearest to x (ties to even), saturating at +-57344."""
    x = float(x)
    if math.isnan(x):
        return 0x7F
    sign = 0x80 if math.copysign(1.0, x) < 0 else 0x00
    a = abs(x)
    if a == 0.0:
        return sign
    if a >= E5M2_MAX:
        return sign | 0x7B
    mant, exp = math.frexp(a)
    mant_int = int(math.ldexp(mant, 53))
    exp_int = exp - 53
    e_unb = exp - 1
    if e_unb < -14:
        # subnormal range: quanta of 2^-16; q == 4 is 2^-14, the smallest normal (code 0x04)
        return sign | _round_half_even(mant_int, -16 - exp_int)
    q = _round_half_even(mant_int, (e_unb - 2) - exp_int)  # normal range: q in [4, 8]
    if q == 8:
        q = 4
        e_unb += 1
    e_field = e_unb + 15
    if e_field > 30:
        return sign | 0x7B
    return sign | (e_field << 2) | (q - 4)


FORMATS = {"e4m3": (encode, decode), "e5m2": (encode_e5m2, decode_e5m2)}
# cache dtype names used by the workloads -> fp8 format ("fp8" alone is e4m3)
KV_FORMATS = {"fp8": "e4m3", "fp8_e5m2": "e5m2"}


@functools.lru_cache(maxsize=2)
def decode_table(fmt: str = "e4m3") -> np.ndarray:
    """All 256 codes decoded, as float64 (NaN for the NaN codes); read-only."""
    dec = FORMATS[fmt][1]
    t = np.array([dec(c) for c in range(256)], dtype=np.float64)
    t.setflags(write=False)
    return t


def _per_head(scale: np.ndarray, head_axis: int, ndim: int) -> np.ndarray:
    """A scale as an array broadcastable against values with `ndim` axes: a
    scalar stays a scalar, a per-head vector lies along `head_axis`."""
    if scale.ndim == 0:
        return scale
    view = [1] * ndim
    view[head_axis] = scale.shape[0]
    return scale.reshape(view)


def quantize(x: np.ndarray, inv_scale, fmt: str = "e4m3", head_axis: int = -2) -> np.ndarray:
    """Bytes stored for values x: encode(float32(x) * float32(inv_scale)).

    The multiply is one float32 operation (round to nearest even), the form
    in which the scale is applied before encoding. inv_scale is a scalar or
    one value per KV head, the axis `head_axis` of x ([..., Hkv, D] rows by
    default).
    """
    x = np.asarray(x)
    inv = _per_head(np.asarray(inv_scale, dtype=np.float32), head_axis % max(x.ndim, 1), x.ndim)
    xs = x.astype(np.float32) * inv
    enc = FORMATS[fmt][0]
    # encode() once per distinct float32 bit pattern (so -0.0 and +0.0 stay
    # apart), then index: the same bytes as a per-element loop.
    bits = np.ascontiguousarray(xs, dtype=np.float32).reshape(-1).view(np.uint32)
    uniq, inverse = np.unique(bits, return_inverse=True)
    vals = uniq.view(np.float32).tolist()
    codes = np.array([enc(v) for v in vals], dtype=np.uint8)
    return codes[inverse].reshape(xs.shape)


def dequantize(codes: np.ndarray, scale, fmt: str = "e4m3", head_axis: int = 0) -> np.ndarray:
    """float64 values decode(code) * scale; scale is a scalar or one value per
    KV head along `head_axis` (cache rows [Hkv, n, D] by default)."""
    table = decode_table(fmt)
    codes = np.asarray(codes, dtype=np.uint8)
    return table[codes] * _per_head(np.asarray(scale, dtype=np.float64), head_axis, codes.ndim)
