"""OCP 8-bit floating point, E4M3 -- TEST INFRASTRUCTURE ONLY (oracle).

The fp8 KV cache stores each K/V element as an E4M3 code of x / scale (one
scale per kv head for K and one for V), and dequantises code -> value * scale.
This follows the pages' "SWA x KV quantisation" direction (paper.rainbus.top
summary, limitations and outlook); the format itself is the OCP 8-bit
floating point specification's E4M3:

  1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits;
  exponent field 0: subnormal, value = (-1)^s * 2^-6 * m/8;
  otherwise value = (-1)^s * 2^(e-7) * (1 + m/8);
  no infinities; S.1111.111 is NaN, so the largest finite value is
  0.1111.110 = 448.

Encoding rounds to the nearest representable value, ties to the even code
(even mantissa).  Values beyond +-448 are the caller's to clamp first (the
cache saturates: clamp(x / scale, -448, 448)).
"""
from __future__ import annotations

import numpy as np

MAX = 448.0


def decode(codes) -> np.ndarray:
    """E4M3 codes (uint8) -> float64 values (NaN for the two NaN codes)."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    sub = sign * (m / 8.0) * 2.0 ** -6
    nor = sign * (1.0 + m / 8.0) * np.power(2.0, (e - 7).astype(np.float64))
    out = np.where(e == 0, sub, nor)
    return np.where((e == 0xF) & ((c & 7) == 7), np.nan, out)


_CODES = np.arange(0x7F, dtype=np.int64)          # 0x00 .. 0x7E: the non-negative finite codes
_VALUES = decode(_CODES)                          # increasing


def encode(x) -> np.ndarray:
    """Nearest E4M3 code, ties to even, for finite |x| <= 448 (uint8)."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(~np.isfinite(x)) or np.any(np.abs(x) > MAX):
        raise ValueError("encode takes finite values within +-448 (clamp first)")
    a = np.abs(x)
    hi = np.searchsorted(_VALUES, a, side="left")   # first value >= a
    hi = np.minimum(hi, len(_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    vlo, vhi = _VALUES[lo], _VALUES[hi]
    exact = vhi == a
    dlo, dhi = a - vlo, vhi - a
    pick_hi = np.where(dhi < dlo, True, np.where(dlo < dhi, False, (_CODES[hi] & 1) == 0))
    code = np.where(exact, _CODES[hi], np.where(pick_hi, _CODES[hi], _CODES[lo]))
    sign = np.where(np.signbit(x), 0x80, 0)
    return (code | sign).astype(np.uint8)


def quantize(x, scale) -> np.ndarray:
    """The cache's store: E4M3 code of clamp(x / scale, -448, 448), the
    division in fp32 (as the device computes it)."""
    q = np.asarray(x, dtype=np.float32) / np.float32(scale)
    return encode(np.clip(q.astype(np.float64), -MAX, MAX))


def dequantize(codes, scale) -> np.ndarray:
    return decode(codes) * float(scale)
