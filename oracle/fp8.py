"""OCP FP8 e4m3fn codec, written from the format definition. TEST INFRASTRUCTURE.

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


@functools.lru_cache(maxsize=1)
def decode_table() -> np.ndarray:
    """All 256 codes decoded, as float64 (NaN for 0x7F and 0xFF); read-only."""
    t = np.array([decode(c) for c in range(256)], dtype=np.float64)
    t.setflags(write=False)
    return t


def quantize(x: np.ndarray, inv_scale: float) -> np.ndarray:
    """Bytes stored for values x: encode(float32(x) * float32(inv_scale)).

    The multiply is one float32 operation (round to nearest even), the form
    in which the scale is applied before encoding.
    """
    xs = np.asarray(x).astype(np.float32) * np.float32(inv_scale)
    # encode() once per distinct float32 bit pattern (so -0.0 and +0.0 stay
    # apart), then index: the same bytes as a per-element loop.
    bits = np.ascontiguousarray(xs, dtype=np.float32).reshape(-1).view(np.uint32)
    uniq, inverse = np.unique(bits, return_inverse=True)
    vals = uniq.view(np.float32).tolist()
    codes = np.array([encode(v) for v in vals], dtype=np.uint8)
    return codes[inverse].reshape(xs.shape)


def dequantize(codes: np.ndarray, scale: float) -> np.ndarray:
    """float64 values decode(code) * scale."""
    table = decode_table()
    return table[np.asarray(codes, dtype=np.uint8)] * float(scale)
