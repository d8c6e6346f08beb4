"""Closed-form number formats used by the method.

The #2711 page ("코드 분석" 1 and 3, "왜 이게 좋은 최적화인가?" 1) names the
operand formats Int8, BFloat16 and E4M3; the pages do not define them, so the
public definitions are written out here:

* bfloat16: the top 16 bits of an IEEE binary32; conversion rounds to nearest,
  ties to even (IEEE default rounding).
* E4M3 ("fn" variant of the OCP 8-bit floating point formats, the one NVIDIA
  calls E4M3): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no
  infinities, only S.1111.111 is NaN.  Largest finite 448, smallest normal
  2^-6, smallest subnormal 2^-9.  Encoding rounds to the nearest representable
  value, ties to the even code, and saturates at +-448.
* int8 (symmetric): round to nearest integer, ties to even, clamp to
  [-127, 127]; -128 is never produced.
"""
import numpy as np

E4M3_MAX = 448.0
INT8_MAX = 127.0


# ----------------------------------------------------------------- bfloat16
def bf16_round(x):
    """Round binary32 values to the nearest bfloat16 (ties to even).

    Returns float32 values that are exactly representable in bfloat16.  Only
    finite inputs are meaningful.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    low = u & 0xFFFF
    keep = u >> 16
    half = 0x8000
    round_up = (low > half) | ((low == half) & ((keep & 1) == 1))
    keep = keep + round_up.astype(np.uint64)
    out = (keep << 16).astype(np.uint32)
    return out.view(np.float32).reshape(x.shape)


# ----------------------------------------------------------------- E4M3
def e4m3_decode(codes):
    """Value of each E4M3 code (uint8 array) as float64; NaN for 0x7F/0xFF."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    subnormal = (m / 8.0) * 2.0 ** -6
    mag = np.where(e == 0, subnormal, normal)
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


# The 127 non-negative finite values, in code order (code i has value _POS[i]).
_POS = e4m3_decode(np.arange(0x7F, dtype=np.uint8))


def e4m3_encode(x):
    """Encode values to E4M3 codes (uint8): nearest value, ties to the even code.

    Magnitudes at or above 448 saturate to 448 (code 0x7E); NaN gives 0x7F
    with the input's sign.  The sign of zero is kept.  Decision made in fp64 on
    the exact input value.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    # index of the largest representable value <= a (clipped to the table)
    lo = np.clip(np.searchsorted(_POS, a, side="right") - 1, 0, len(_POS) - 1)
    hi = np.clip(lo + 1, 0, len(_POS) - 1)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0) & (hi != lo))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= E4M3_MAX, 0x7E, code)
    code = np.where(np.isnan(a), 0x7F, code)
    sign = np.signbit(x).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


def e4m3_round(x):
    """Quantise-then-dequantise through E4M3 (fp64 result)."""
    return e4m3_decode(e4m3_encode(x))


# ----------------------------------------------------------------- int8
def int8_encode(x):
    """Symmetric int8: round half to even, clamp to [-127, 127]."""
    r = np.rint(np.asarray(x, dtype=np.float64))
    return np.clip(r, -INT8_MAX, INT8_MAX).astype(np.int8)


def bf16_round64(x):
    """Round fp64 values directly to the nearest bfloat16 (ties to even).

    bfloat16 keeps 8 significant bits over binary32's exponent range
    (normals down to 2^-126, subnormal spacing 2^-133).  Result is fp64.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, e = np.frexp(a)  # a = f * 2^e with f in [0.5, 1)
    # spacing of the bf16 grid at a: 2^(e-8) for normals, 2^-133 below 2^-126
    spacing_exp = np.where(a >= 2.0 ** -126, e - 8, -133)
    q = np.rint(np.ldexp(a, -spacing_exp))  # rint: half to even
    return np.copysign(np.ldexp(q, spacing_exp), x)


def rounding_gap(x, p_format, eps):
    """Where x is within relative distance eps of a rounding boundary of the
    format (the midpoint of two neighbouring representable values), return
    the distance between those two values; 0 elsewhere.

    An implementation that computes x in lower precision than this oracle may
    land on the other side of such a boundary; the result then moves by one
    step of the format.  x >= 0 (softmax weights).
    """
    x = np.asarray(x, dtype=np.float64)
    if p_format == "e4m3":
        lo_i = np.clip(np.searchsorted(_POS, x, side="right") - 1, 0, len(_POS) - 2)
        lo, hi = _POS[lo_i], _POS[lo_i + 1]
    elif p_format == "bf16":
        _, e = np.frexp(np.maximum(x, 2.0 ** -133))
        step = np.ldexp(1.0, np.maximum(e - 8, -133))
        lo = np.floor(x / step) * step
        hi = lo + step
    else:
        return np.zeros_like(x)
    mid = (lo + hi) / 2
    near = np.abs(x - mid) <= eps * np.maximum(x, 2.0 ** -133)
    near &= x < E4M3_MAX if p_format == "e4m3" else True
    return np.where(near, hi - lo, 0.0)
