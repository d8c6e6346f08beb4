"""Per-block quantisation of a bf16 tensor (the SageAttention scale factors).

Follows the #2711 page, "코드 분석" 2 (scale factors are kept per block rather
than per tensor, and undo the quantisation after BMM1/BMM2) and "코드 분석" 1
(the number of elements covered by one scale factor is a kernel parameter).
The pages give neither the block shape nor the formula; the readings used here:

* one block = 64 consecutive tokens x all D channels of one (batch, head); a
  final partial block covers the tokens that exist;
* scale = amax / Qmax, with Qmax = 127 (int8) or 448 (E4M3), amax = max |x|
  over the block;
* code = encode(x * inv) with inv = Qmax / amax (one division per block, one
  multiplication per element);
* all arithmetic is IEEE binary32 with round-to-nearest-even and no
  flush-to-zero, emulated with numpy float32 operations;
* a block whose amax is zero or below 2^-126 gets scale 1.0 and all-zero codes.
"""
import numpy as np

from .codecs import e4m3_encode, int8_encode

QMAX = {"int8": np.float32(127.0), "e4m3": np.float32(448.0)}
TINY = np.float32(2.0 ** -126)


def quantize_blocks(x, qdtype, block_tokens=64):
    """Quantise ``x`` ([B, S, H, D], float32 holding bf16 values) per block.

    Returns ``(codes, scales)``: codes has x's shape (int8 for "int8", uint8
    E4M3 bit patterns for "e4m3"); scales is float32 [B, H, ceil(S/64)].
    """
    x = np.asarray(x, dtype=np.float32)
    B, S, H, D = x.shape
    nblk = -(-S // block_tokens)
    qmax = QMAX[qdtype]
    code_dtype = np.int8 if qdtype == "int8" else np.uint8
    codes = np.zeros(x.shape, dtype=code_dtype)
    scales = np.ones((B, H, nblk), dtype=np.float32)
    for k in range(nblk):
        t0, t1 = k * block_tokens, min((k + 1) * block_tokens, S)
        blk = x[:, t0:t1]                                   # [B, T, H, D]
        amax = np.abs(blk).max(axis=(1, 3))                 # [B, H] float32
        live = amax >= TINY
        safe = np.where(live, amax, np.float32(1.0)).astype(np.float32)
        scale = (safe / qmax).astype(np.float32)            # fl32(amax / Qmax)
        inv = (qmax / safe).astype(np.float32)              # fl32(Qmax / amax)
        y = (blk * inv[:, None, :, None]).astype(np.float32)  # fl32(x * inv)
        c = int8_encode(y) if qdtype == "int8" else e4m3_encode(y)
        c = np.where(live[:, None, :, None], c, 0).astype(code_dtype)
        codes[:, t0:t1] = c
        scales[:, :, k] = np.where(live, scale, np.float32(1.0))
    return codes, scales
