"""8-bit float (e4m3) KV-cache codes — oracle; test infrastructure only.

«Servicio…presupuesto de memoria» §4 and «¿Cuánta memoria reservar para la
caché KV?» (the paragraph on quantising and offloading the cache) name cache
quantisation as a way to shrink the KV term and warn that a change of KV
precision changes the numerics; neither fixes a format.  The readings taken
here (the library follows the same ones):

* Format: the OCP 8-bit floating-point "E4M3" encoding — 1 sign bit, 4
  exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds the
  subnormals m·2^-9; S.1111.111 is NaN; there is no infinity; the largest
  finite magnitude is 448 (S.1111.110).
* Granularity: one fp32 scale per (token, KV head) row of d values, for K
  and for V separately, so a token is quantised once, when it is written,
  and a block that is still filling never needs re-quantising.
* Scale: ``s = amax / 448`` in fp32 (IEEE division, round to nearest even),
  ``amax`` the largest |x| of the row (exact in fp32).  A row of zeros gets
  ``s = 0`` and codes 0.
* Code: ``encode(x / s)``, the quotient in fp32 (IEEE division), rounded to
  the nearest E4M3 value, ties to the even code; the value a code stands for
  is ``value(code) · s`` (exact in fp64).

Plain definitions: the value table is built from the bit fields; rounding
is defined by picking the nearest table entry (``encode_nearest``) and done,
for whole pools, by the equivalent rounding onto the format's grid
(``encode``), which the tests hold equal to the table search.
"""
from __future__ import annotations

import numpy as np

MAX = 448.0


def value(code: int) -> float:
    """The number an E4M3 code stands for (NaN for S.1111.111)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# all 256 codes, and the non-negative finite ones in increasing order
VALUES = np.array([value(c) for c in range(256)], dtype=np.float64)
_POS_CODES = np.array([c for c in range(0x7F)], dtype=np.int64)      # 0x00 .. 0x7E
_POS_VALUES = VALUES[_POS_CODES]
assert np.all(np.diff(_POS_VALUES) > 0)


def decode(codes: np.ndarray) -> np.ndarray:
    """fp64 values of an array of codes."""
    return VALUES[np.asarray(codes, dtype=np.int64) & 0xFF]


def encode_nearest(y: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code to each value of ``y`` (ties to the even code),
    found by searching the value table.  |y| beyond the rounding range of
    448 (that is, > 464) gives NaN (0x7F / 0xFF); the sign of zero is kept.
    The plain definition; ``encode`` reaches the same codes faster."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    # index of the first table value >= a; compare with its lower neighbour
    hi = np.clip(np.searchsorted(_POS_VALUES, a, side="left"), 0, len(_POS_VALUES) - 1)
    lo = np.clip(hi - 1, 0, len(_POS_VALUES) - 1)
    d_hi = np.abs(_POS_VALUES[hi] - a)
    d_lo = np.abs(a - _POS_VALUES[lo])
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (_POS_CODES[lo] % 2 == 0))
    mag = np.where(pick_lo, _POS_CODES[lo], _POS_CODES[hi])
    mag = np.where(a > MAX + 16.0, 0x7F, mag)          # past the 448/480 midpoint
    mag = np.where(a == MAX + 16.0, 0x7E, mag)         # the tie itself goes to the even 448
    mag = np.where(np.isnan(a), 0x7F, mag)
    sign = np.where(np.signbit(y), 0x80, 0x00)
    return (mag | sign).astype(np.uint8)


def _binade(a: np.ndarray) -> np.ndarray:
    """floor(log2 a) for finite a > 0 (any value for a = 0), from the fp64
    exponent field (exact: every fp32 value is normal in fp64)."""
    return ((a.view(np.uint64) >> np.uint64(52)).astype(np.int64) & 0x7FF) - 1023


def _pow2(e: np.ndarray) -> np.ndarray:
    """2.0 ** e for integer arrays e in the fp64 normal range."""
    return ((e + 1023).astype(np.uint64) << np.uint64(52)).view(np.float64)


def encode(y: np.ndarray) -> np.ndarray:
    """The same codes as ``encode_nearest``, by rounding onto the format's
    grid: in the binade [2^e, 2^(e+1)) (e >= -6; below 2^-6 the subnormals
    keep the spacing of e = -6) representable magnitudes are the multiples of
    2^(e-3), so |y| rounds to rint(|y| / 2^(e-3)) * 2^(e-3) (round half to
    even on the multiple; an even multiple is an even code, also where the
    result reaches the next binade).  A result of 480 or more is past 448:
    NaN.  Scaling by powers of two is exact in fp64."""
    y = np.ascontiguousarray(y, dtype=np.float64)
    a = np.abs(y)
    nan = ~(a < MAX + 32.0)                             # NaN, or surely past 448
    a = np.where(nan, 0.0, a)
    e = np.maximum(_binade(a), -6)
    m = np.rint(a * _pow2(3 - e))                       # the rounded multiple of 2^(e-3): 0 .. 16
    # code fields: a multiple below 8 is a subnormal (e = -6) or zero; 16 is
    # the next binade's 8
    up = m >= 16
    e = e + up
    m = np.where(up, 8, m).astype(np.int64)
    normal = m >= 8
    mag = np.where(normal, ((e + 7) << 3) | (m - 8), m)
    mag = np.where(nan | (mag > 0x7E), 0x7F, mag)       # 480 and above: NaN
    sign = np.where(np.signbit(y), 0x80, 0x00)
    return (mag | sign).astype(np.uint8)


def quantize_rows(x: np.ndarray):
    """(codes uint8 [..., d], scales float32 [...]) of rows of fp32 values
    (the last axis is the row), each row by the readings above."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)                               # exact in fp32
    scale = (amax / np.float32(MAX)).astype(np.float32)             # IEEE fp32 division
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    y = (x / safe[..., None]).astype(np.float32)                    # IEEE fp32 division
    # encode element by element (in pieces that stay in the host caches)
    flat = y.reshape(-1)
    codes = np.empty(flat.shape, dtype=np.uint8)
    piece = 1 << 16
    for i in range(0, flat.size, piece):
        codes[i:i + piece] = encode(flat[i:i + piece])
    codes = np.where(scale[..., None] > 0, codes.reshape(y.shape), np.uint8(0)).astype(np.uint8)
    return codes, scale


def quantize_row(x: np.ndarray):
    """(codes uint8 [d], scale float32) of one (token, head) row."""
    codes, scale = quantize_rows(np.asarray(x, dtype=np.float32)[None])
    return codes[0], np.float32(scale[0])


def dequantize_row(codes: np.ndarray, scale) -> np.ndarray:
    """fp64 values a row of codes stands for."""
    return decode(codes) * np.float64(np.float32(scale))
