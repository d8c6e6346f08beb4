"""Per-token NVFP4 quantisation (test infrastructure only, like the rest of
this package).

Follows the #3237 page ("FlashInfer의 Per-token NVFP4 Quantization 커널 최적화
분석"): a kernel that quantises each token (row) of an activation matrix to
FP4 with per-block scale factors plus one scale per token, reading the row
once for its maximum and once more for the encoding (the input-caching change
of 코드 분석 2 exists because of that second pass), with the scale factors in a
linear (not swizzled) layout (코드 분석 1 dispatches the LINEAR layout).  The
page does not define the number format; the public NVFP4 definition is used:

* element: FP4 E2M1 -- 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit;
  magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; no infinities or NaN;
* 16 consecutive elements of a row share one E4M3 block scale;
* a second-level fp32 scale, here one per token.

Readings (the page gives no formulas):

* token scale ts = amax / (6 * 448), amax = max |x| over the row, so that the
  largest element maps to the top of both formats (6 for E2M1 and 448 for the
  E4M3 block scale); the block scale in units of ts is bmax / 6 / ts =
  bmax * (448 / amax);
* rows whose amax is below 2^-116 (zero rows included) take ts = 1 and a zero
  block-scale factor, so every block scale and code there is zero;
* block j: sf = E4M3(min(fl32(bmax * g6), 448)) with g6 = fl32(448 / amax);
  its step in x units is bs = fl32(dec(sf) * ts) and the element multiplier
  es = min(fl32(1 / bs), FLT_MAX), or 0 when bs is 0;
* code = E2M1(clamp(fl32(x * es), -6, 6)), nearest value with ties to the
  even code, the sign of zero kept;
* dequantisation: x ~ E2M1 value * dec(sf) * ts;
* every operation is IEEE binary32 with round-to-nearest-even and no
  flush-to-zero (emulated with numpy float32), divisions correctly rounded;
* packing: element 2i in the low nibble of byte i, element 2i + 1 in the
  high nibble.
"""
import numpy as np

from .codecs import e4m3_decode, e4m3_encode

E2M1_MAX = 6.0
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])  # code 0..7
BLOCK = 16
TOKEN_TINY = np.float32(2.0 ** -116)
FLT_MAX = np.float32(np.finfo(np.float32).max)


def e2m1_decode(codes):
    """Value of each 4-bit E2M1 code (low nibble of a uint8) as float64.

    Closed form: exponent field e, mantissa bit m; e = 0 gives m * 0.5
    (subnormal), otherwise 2^(e-1) * (1 + m / 2).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64) & 0xF
    sign = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = (c & 0x1).astype(np.float64)
    mag = np.where(e == 0, 0.5 * m, np.exp2(e.astype(np.float64) - 1.0) * (1.0 + m / 2.0))
    return sign * mag


def e2m1_encode(x):
    """Encode values to E2M1 codes (uint8 in 0..15): the nearest of the eight
    magnitudes, ties to the even code, saturating at 6, sign of zero kept."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E2M1_MAX)
    lo = np.clip(np.searchsorted(E2M1_VALUES, a, side="right") - 1, 0, 7)
    hi = np.minimum(lo + 1, 7)
    d_lo = a - E2M1_VALUES[lo]
    d_hi = E2M1_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0) & (hi != lo))
    code = np.where(pick_hi, hi, lo)
    return (code | (np.signbit(x).astype(np.int64) << 3)).astype(np.uint8)


def quantize_nvfp4(x):
    """Quantise x ([M, K] float32 holding bf16 values, K a multiple of 16)
    token by token.

    Returns (codes uint8 [M, K/2] packed two per byte, block_scales uint8
    [M, K/16] E4M3 bit patterns, token_scales float32 [M]).
    """
    x = np.asarray(x, dtype=np.float32)
    M, K = x.shape
    assert K % BLOCK == 0
    nb = K // BLOCK
    xb = x.reshape(M, nb, BLOCK)
    amax = np.abs(x).max(axis=1) if K else np.zeros(M, np.float32)        # exact
    live = amax >= TOKEN_TINY
    safe = np.where(live, amax, np.float32(1.0)).astype(np.float32)
    ts = np.where(live, (safe / np.float32(2688.0)).astype(np.float32), np.float32(1.0)).astype(np.float32)
    g6 = np.where(live, (np.float32(448.0) / safe).astype(np.float32), np.float32(0.0)).astype(np.float32)

    bmax = np.abs(xb).max(axis=2)                                           # [M, nb] exact
    sfv = np.minimum((bmax * g6[:, None]).astype(np.float32), np.float32(448.0))
    sf = e4m3_encode(sfv)
    bs = (e4m3_decode(sf).astype(np.float32) * ts[:, None]).astype(np.float32)
    with np.errstate(divide="ignore", over="ignore"):
        inv = (np.float32(1.0) / np.where(bs > 0, bs, np.float32(1.0))).astype(np.float32)
    es = np.where(bs > 0, np.minimum(inv, FLT_MAX), np.float32(0.0)).astype(np.float32)
    with np.errstate(over="ignore"):
        y = (xb * es[:, :, None]).astype(np.float32)
    y = np.clip(y, np.float32(-E2M1_MAX), np.float32(E2M1_MAX))  # keeps -0.0
    c = e2m1_encode(y).reshape(M, K)
    packed = (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
    return packed, sf.astype(np.uint8), ts


def unpack_codes(packed):
    """[M, K/2] packed bytes -> [M, K] 4-bit codes (element 2i = low nibble)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], 2 * p.shape[1]), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def dequantize_nvfp4(packed, block_scales, token_scales):
    """x ~ E2M1 value * dec(block scale) * token scale, in float64."""
    c = unpack_codes(packed)
    M, K = c.shape
    v = e2m1_decode(c).reshape(M, K // BLOCK, BLOCK)
    s = e4m3_decode(block_scales)[:, :, None] * np.asarray(token_scales, np.float64)[:, None, None]
    return (v * s).reshape(M, K)
