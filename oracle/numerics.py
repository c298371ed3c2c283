"""Bit-level number formats used by the oracle (test infrastructure only).

* bf16: the upper 16 bits of an IEEE-754 binary32 value.  Widening is exact;
  narrowing is round-to-nearest, ties-to-even on the 16 dropped bits.
* FP8 E4M3 in the OCP 8-bit floating point "fn" flavour: 1 sign bit, 4
  exponent bits with bias 7, 3 mantissa bits, no infinities, the single NaN
  pattern S.1111.111, largest finite magnitude 1.75 * 2^8 = 448 (code 0x7E),
  subnormal step 2^-9.  The DeepEP pages only say that dispatch may move FP8
  (one byte per element instead of two); this flavour is the reading taken
  because its 448 maximum is the divisor of the per-128-channel scales.

All routines take and return numpy arrays; nothing here is shared with the
HIP library.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32, exactly (append 16 zero bits)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_bits_rne(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even.

    Keep the upper half of the fp32 pattern; round it up by one unit when the
    dropped half is more than half a unit, or exactly half a unit and the kept
    part is odd.  Finite inputs only.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    kept = u >> np.uint64(16)
    dropped = u & np.uint64(0xFFFF)
    up = (dropped > 0x8000) | ((dropped == 0x8000) & ((kept & np.uint64(1)) == 1))
    return (kept + up.astype(np.uint64)).astype(np.uint16)


def _e4m3_magnitude_table() -> np.ndarray:
    """Values of the non-negative finite codes 0x00..0x7E, in code order (ascending)."""
    vals = np.empty(127, dtype=np.float64)
    for code in range(127):
        e = code >> 3
        m = code & 7
        if e == 0:
            vals[code] = m * 2.0 ** -9  # subnormal: m/8 * 2^(1-7)
        else:
            vals[code] = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


E4M3_MAGNITUDES = _e4m3_magnitude_table()


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """OCP E4M3 codes (uint8) -> float32; 0x7F/0xFF decode to NaN."""
    c = np.asarray(codes, dtype=np.uint8)
    mag_code = (c & 0x7F).astype(np.int64)
    out = np.where(mag_code == 0x7F, np.nan, E4M3_MAGNITUDES[np.minimum(mag_code, 126)])
    out = np.where((c & 0x80) != 0, -out, out)
    return out.astype(np.float32)


def e4m3_encode_rne(x: np.ndarray) -> np.ndarray:
    """float32 -> OCP E4M3 code: the nearest finite E4M3 value, ties to the even code.

    Magnitudes above 448 saturate to 448 (code 0x7E).  The sign bit is kept,
    so negative values that round to zero give 0x80.  Finite inputs only.
    """
    v = np.ascontiguousarray(x, dtype=np.float32)
    a = np.abs(v).astype(np.float64)
    table = E4M3_MAGNITUDES
    hi = np.searchsorted(table, a, side="left")  # table[hi-1] < a <= table[hi]
    hi = np.minimum(hi, len(table) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - table[lo]
    d_hi = table[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((hi & 1) == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= table[-1], 126, code)  # saturate at 448
    sign = np.signbit(v).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)
