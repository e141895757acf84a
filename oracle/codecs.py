"""Number formats used by the oracle: bf16 and OCP fp8 E4M3FN.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's CPU
baseline may import anything under oracle/.  Nothing here is shared with the
HIP path.

Both codecs are written from the formats' definitions:
  * bf16: the top 16 bits of an IEEE-754 binary32 value.
  * E4M3FN (OCP 8-bit floating point, "FN" = finite + NaN, no infinities):
    1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0 is
    subnormal (m/8 * 2^-6); S.1111.111 is NaN; the largest finite is
    S.1111.110 = 448.
The fp8 cache is the option named in "LLM推理优化的新范式：从内存墙到计算墙的跨越"
(zskr.cn) §5 (mixed-precision FP8/FP16 KV cache) and "DeepSeek V3 MLA 优化"
(fsdata.site) §3.1 (FP8 to compress the KV cache further).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 (ties to the even significand),
    for finite values whose result is finite.  The candidates are the bf16
    values just below and above x (truncations of x's binary32 neighbours);
    the decision is made on the exact float64 values."""
    x = np.asarray(x, dtype=np.float64)
    f = x.astype(np.float32)                       # nearest binary32 (for the neighbours only)
    u = f.view(np.uint32)
    lo = (u & np.uint32(0xFFFF0000))               # truncation toward zero in magnitude
    lo_v = lo.view(np.float32).astype(np.float64)
    # the other candidate is one bf16 step further from zero
    hi = (lo + np.uint32(0x10000)).astype(np.uint32)
    hi_v = hi.view(np.float32).astype(np.float64)
    # make (a, b) the candidates bracketing x
    below = np.abs(lo_v) <= np.abs(x)
    a_bits = np.where(below, lo, (lo - np.uint32(0x10000)).astype(np.uint32))
    b_bits = np.where(below, hi, lo)
    a_v = a_bits.view(np.float32).astype(np.float64)
    b_v = b_bits.view(np.float32).astype(np.float64)
    da, db = np.abs(x - a_v), np.abs(b_v - x)
    even_a = ((a_bits >> np.uint32(16)) & np.uint32(1)) == 0
    pick_a = (da < db) | ((da == db) & even_a)
    out = np.where(pick_a, a_bits, b_bits) >> np.uint32(16)
    out = np.where(x == 0, (u >> np.uint32(16)), out)   # +-0 keep their sign
    return out.astype(np.uint16)


def e4m3fn_decode(codes: np.ndarray) -> np.ndarray:
    """Value of each E4M3FN code (uint8) as float64; NaN codes give NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & ((c & 7) == 7), np.nan, mag)
    return sign * mag


# magnitudes of the 127 non-negative finite codes 0x00..0x7E, ascending
_POS_CODES = np.arange(0x7F, dtype=np.uint8)
_POS_VALUES = e4m3fn_decode(_POS_CODES)
assert np.all(np.diff(_POS_VALUES) > 0)


def e4m3fn_encode_satfinite(x: np.ndarray) -> np.ndarray:
    """Round float32 values to E4M3FN codes: nearest, ties to the even code,
    magnitudes beyond 448 clamp to +-448, NaN gives 0x7F.

    Works on the exact (float64) value of each float32 input by locating it
    between the two neighbouring representable magnitudes.
    """
    xf = np.asarray(x, dtype=np.float32).astype(np.float64)
    nan = np.isnan(xf)
    a = np.abs(np.where(nan, 0.0, xf))
    a = np.minimum(a, E4M3_MAX)
    hi = np.searchsorted(_POS_VALUES, a, side="left")        # first value >= a
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    v_hi = _POS_VALUES[hi]
    v_lo = _POS_VALUES[lo]
    exact = v_hi == a
    d_lo = a - v_lo
    d_hi = v_hi - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(exact, hi, np.where(pick_hi, hi, lo)).astype(np.uint8)
    neg = np.signbit(xf) & ~nan
    code = np.where(neg & (code != 0), code | 0x80, code)
    code = np.where(neg & (code == 0), 0x80, code)  # keep the sign of negative zero results
    code = np.where(nan, 0x7F, code)
    return code.astype(np.uint8)
