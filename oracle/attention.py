"""Attention forward over dequantised operands, step by step.

What is computed (the readings are stated where the pages leave a step open):

1. Dequantise Q, K, V in fp64: value = code x scale of the token's 64-token
   block (#2711 page, "코드 분석" 2: the block scales undo the quantisation
   after BMM1 / BMM2), or the bf16 value itself for an unscaled operand.
   Paged K/V (#4474 page, "코드 분석" 2 and the block-sparse paged-KV entry
   point) are first gathered into logical token order through the page table.
2. Scores in log2 units: s2 = (q . k) * softmax_scale * log2(e).
3. Valid pairs: causal (bottom-right aligned), and the block mask at
   Q64 x KV256 granularity (#4474 page, "코드 분석" 1: the Q64/KV256 tile is the
   block-sparse unit).
4. Online softmax with lazy correction (#5900 page, "코드 분석" 3, first
   bullet: O is rescaled only when the row maximum has grown by 2^8): keys are
   visited in ascending 64-key sub-tiles; a row's reference maximum m moves to
   the sub-tile maximum t only when m is unset or t - m > 8 (log2 units), and
   only then are the running numerator and denominator multiplied by 2^(m - t).
   P = 2^(s2 - m) is therefore at most 2^8.
5. P is quantised to the PV operand format before BMM2 (#5900 page title and
   "코드 분석" 1: P is an 8-bit operand of the PV product when V is 8-bit), with
   the optional static per-head P scale sfs_p (#2711 page, "코드 분석" 2 lists
   a P scale-factor pointer): w = Qp(P / sp) * sp.
6. num += sum_j w_j V_j and den += sum_j w_j (the denominator uses the same
   quantised weights as the numerator).
7. O = num / den; a row with no valid key gives 0.
8. Optional E4M3 output (``output_e4m3``): the #5900 page's reviewer-feedback
   paragraph names an FP8 output of the kernel without saying how it is
   scaled; read here as a static per-head output scale, like sfs_p:
   o = encode(O / so), nearest-even, saturating at +-448.

``mode="exact"`` replaces step 4 by the true row maximum (no rescaling);
``p_format=None`` skips step 5.  Together they give plain softmax attention.

Rounding sensitivity (``flip_eps``): the pages fix no precision for the
scores.  A kernel that forms s2 and 2^(s2 - m) in binary32 can put a P value
that lies on a rounding boundary of Qp on the other side of it, which moves
that key's weight by one step of the P format.  With ``flip_eps`` the oracle
also returns, per output element, the sum over keys whose P / sp lies within
relative distance flip_eps of such a boundary of |one-step change in w_j| *
(share of w_j left after later rescales) * |V_j - O| / den: to first order,
the most the output can move through such ties.  The output itself does not
depend on flip_eps.

``flip_eps="binary32"`` replaces the fixed relative distance by a per-pair
bound on the error of a kernel that works in IEEE binary32: it accumulates
q . k with at most D roundings (error <= gamma_D * sum_d |q_d k_d|, gamma_D =
D u / (1 - D u), u = 2^-24, the standard bound for any summation order; a
fused or integer accumulation is only more accurate), then rounds at most
four more times in forming the exponent s2 - m - log2(sp) (the scale
product, the running maximum, the log of sp and the fused multiply-add: at
most 4 u (|s2| + |m| + |log2 sp|)), and evaluates 2^x to within 2 ulp
(2^-22 relative).  The reference maximum m is itself the binary32 score of
some key of the sub-tile that set it, so its accumulation error enters the
exponent too: at most the largest gamma_D * sum_d |q_d k_d| among the keys
whose score plus that bound reaches the sub-tile's maximum (the only keys
that can come out on top).  The relative error of P is then at most ln 2 times the
exponent error plus 2^-22, to first order.
"""
import math

import numpy as np

from .codecs import bf16_round64, e4m3_decode, e4m3_encode, e4m3_round, rounding_gap

LOG2E = 1.0 / math.log(2.0)
U32 = 2.0 ** -24  # unit roundoff of IEEE binary32


def binary32_accumulation_error(q, k, D, c):
    """Bound on the error of a binary32 score c * (q . k), log2 units, for
    every pair of rows of q and k: c * gamma_D * sum_d |q_d k_d|."""
    gamma = D * U32 / (1.0 - D * U32)
    with np.errstate(invalid="ignore", over="ignore"):
        return c * gamma * (np.abs(q) @ np.abs(k).T)


def _max_error(s, err, t):
    """Error bound of a binary32 maximum of the scores s (rows; -inf where
    invalid) whose exact maximum is t: a key can come out on top only if its
    score plus its error reaches t, so the largest error among those keys
    bounds the computed maximum's distance from t."""
    with np.errstate(invalid="ignore"):
        cand = np.isfinite(s) & (s + err >= t[:, None])
    return np.where(cand, err, 0.0).max(axis=1) if s.shape[1] else np.zeros(s.shape[0])


def binary32_p_error(q, k, s, m, D, c, sp, m_err=0.0):
    """Relative error bound of P = 2^(s - m) / sp for a binary32 kernel (see
    the module docstring): s = c * (q . k) are the fp64 log2-domain scores of
    the pairs (rows of q against rows of k), m the row's reference maximum and
    m_err (per row) the accumulation error bound of the score that set it."""
    acc = binary32_accumulation_error(q, k, D, c)
    with np.errstate(invalid="ignore"):
        rnd = 4.0 * U32 * (np.abs(s) + np.abs(m)[:, None] + abs(math.log2(sp)))
    return math.log(2.0) * (acc + np.asarray(m_err, dtype=np.float64).reshape(-1, 1) + rnd) + 2.0 ** -22


def dequantize(codes, fmt, scales=None, block_tokens=64):
    """fp64 values of a [B, S, H, D] operand.

    fmt: "int8" (int8 codes), "e4m3" (uint8 bit patterns) or "bf16" (float32
    array holding bf16 values).  scales: float32 [B, H, ceil(S/64)] or None.
    """
    if fmt == "int8":
        v = np.asarray(codes, dtype=np.int8).astype(np.float64)
    elif fmt == "e4m3":
        v = e4m3_decode(codes)
    elif fmt == "bf16":
        v = np.asarray(codes, dtype=np.float32).astype(np.float64)
    else:
        raise ValueError(fmt)
    if scales is not None:
        S = v.shape[1]
        tok_blk = np.arange(S) // block_tokens                     # [S]
        s = np.asarray(scales, dtype=np.float64)[:, :, tok_blk]     # [B, H, S]
        v = v * np.transpose(s, (0, 2, 1))[..., None]
    return v


def gather_pages(pool, page_table, S, page_size=16):
    """Logical [B, S, H, D] view of a paged pool [num_pages, page_size, H, D].

    page_table[b, p] is the physical page holding logical tokens
    [p*page_size, (p+1)*page_size) of sequence b.
    """
    pool = np.asarray(pool)
    pt = np.asarray(page_table)
    tok = np.arange(S)
    phys = pt[:, tok // page_size]                 # [B, S]
    return pool[phys, tok % page_size]             # [B, S, H, D]


def _quantize_p(p, p_format):
    if p_format is None:
        return p
    if p_format == "e4m3":
        return e4m3_round(p)
    if p_format == "bf16":
        return bf16_round64(p)
    raise ValueError(p_format)


def valid_pairs(rows, Sq, Skv, causal, mask_rows):
    """Boolean [len(rows), Skv]: which (query, key) pairs take part.

    mask_rows: None or a boolean [len(rows), Skv] already expanded from the
    block mask.  Causal alignment is bottom-right: key j is visible from
    query i when j <= i + Skv - Sq.
    """
    j = np.arange(Skv)[None, :]
    v = np.ones((len(rows), Skv), dtype=bool)
    if causal:
        v &= j <= (np.asarray(rows)[:, None] + Skv - Sq)
    if mask_rows is not None:
        v &= mask_rows
    return v


def attention_head(q, k, v, rows, *, Sq, softmax_scale, causal=False,
                   mask_rows=None, mode="lazy", p_format=None, sp=1.0,
                   tau=8.0, sub_tile=64, flip_eps=None):
    """One (batch, head): q [n, D] for query indices ``rows``; k, v [Skv, D].

    Returns O [n, D] in fp64, or (O, rounding-sensitivity bound [n, D]) when
    flip_eps is given.
    """
    n, D = q.shape
    Skv = k.shape[0]
    valid = valid_pairs(rows, Sq, Skv, causal, mask_rows)
    with np.errstate(invalid="ignore", over="ignore"):
        s2 = (q @ k.T) * (softmax_scale * LOG2E)
    b32 = isinstance(flip_eps, str)
    if b32:
        assert flip_eps == "binary32", flip_eps
        acc_err = np.where(valid, binary32_accumulation_error(q, k, D, softmax_scale * LOG2E), 0.0)
    m_err = np.zeros(n)  # accumulation error bound of the score that set m (binary32 model)
    if mode == "exact":
        m = np.where(valid, s2, -np.inf).max(axis=1) if Skv else np.full(n, -np.inf)
        if b32 and Skv:
            m_err = _max_error(np.where(valid, s2, -np.inf), acc_err, m)
    else:
        m = np.full(n, -np.inf)
    num = np.zeros((n, D))
    den = np.zeros(n)
    ties = []  # (cols, weight step at the tie, row max at that time) per sub-tile
    for k0 in range(0, Skv, sub_tile):
        cols = slice(k0, min(k0 + sub_tile, Skv))
        vs = valid[:, cols]
        if not vs.any():
            continue
        with np.errstate(invalid="ignore", over="ignore"):
            s = np.where(vs, s2[:, cols], -np.inf)
        if mode == "lazy":
            t = s.max(axis=1)
            has = vs.any(axis=1)
            with np.errstate(invalid="ignore"):
                trig = has & ((m == -np.inf) | (t - m > tau))
                alpha = np.where(m == -np.inf, 0.0, np.exp2(np.where(trig, m - t, 0.0)))
            num[trig] *= alpha[trig, None]
            den[trig] *= alpha[trig]
            m = np.where(trig, t, m)
            if b32:
                m_err = np.where(trig, _max_error(s, acc_err[:, cols], t), m_err)
        with np.errstate(invalid="ignore", over="ignore"):
            p = np.where(vs, np.exp2(s - m[:, None]), 0.0)
        w = _quantize_p(p / sp, p_format) * sp
        # keys valid for no row of this block are never read (they may hold
        # anything, NaN included)
        col_used = vs.any(axis=0)
        vv = np.where(col_used[:, None], v[cols], 0.0)
        num += w @ vv
        den += w.sum(axis=1)
        if flip_eps is not None:
            eps = flip_eps
            if b32:
                eps = np.where(vs, binary32_p_error(q, k[cols], np.where(vs, s, 0.0), m, D,
                                                    softmax_scale * LOG2E, sp, m_err), 0.0)
            gap = np.where(vs, rounding_gap(p / sp, p_format, eps) * sp, 0.0)
            if gap.any():
                ties.append((cols, gap, m.copy(), vv))
    with np.errstate(invalid="ignore", divide="ignore"):
        out = np.where(den[:, None] > 0, num / np.where(den > 0, den, 1.0)[:, None], 0.0)
    if flip_eps is None:
        return out
    bound = np.zeros((n, D))
    safe_den = np.where(den > 0, den, np.inf)
    for cols, gap, m_then, vv in ties:
        with np.errstate(invalid="ignore", over="ignore"):
            share = np.where(np.isfinite(m_then), np.exp2(m_then - m), 0.0)   # later rescales
        wgt = gap * (share / safe_den)[:, None]                              # [n, keys]
        bound += np.einsum("nk,nkd->nd", wgt, np.abs(vv[None, :, :] - out[:, None, :]))
    return out, bound


def expand_block_mask(block_mask_bh, rows, Skv, mask_block_q=64, mask_block_kv=256):
    """Boolean [len(rows), Skv] from one (batch, head) block mask [nqb, nkb]."""
    bm = np.asarray(block_mask_bh) != 0
    qb = np.asarray(rows) // mask_block_q
    kb = np.arange(Skv) // mask_block_kv
    return bm[qb][:, kb]


def attention(qd, kd, vd, *, softmax_scale=None, causal=False, block_mask=None,
              mode="lazy", p_format=None, sfs_p=None, tau=8.0, sub_tile=64,
              rows=None, heads=None, mask_block_q=64, mask_block_kv=256, flip_eps=None):
    """Attention over dequantised fp64 operands.

    qd [B, Sq, Hq, D]; kd, vd [B, Skv, Hkv, D] in logical token order.  Query
    head h reads key/value head h // (Hq // Hkv) (consecutive query heads
    share a key/value head, the heads_q_per_kv grouping of the #4474 page,
    "코드 분석" 1).  block_mask: None or [B, Hq, ceil(Sq/64), ceil(Skv/256)]
    (non-zero = active).  rows: optional query indices to compute (rows are
    independent); heads: optional list of (b, hq) pairs.

    Returns fp64 [B, len(rows) or Sq, Hq, D]; entries of heads not computed
    are NaN.  With flip_eps, returns (O, rounding-sensitivity bound) of the
    same shape (see the module docstring).
    """
    B, Sq, Hq, D = qd.shape
    Skv, Hkv = kd.shape[1], kd.shape[2]
    assert Hq % Hkv == 0
    group = Hq // Hkv
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    rows = np.arange(Sq) if rows is None else np.asarray(rows)
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(Hq)]
    out = np.full((B, len(rows), Hq, D), np.nan)
    bound = np.full((B, len(rows), Hq, D), np.nan) if flip_eps is not None else None
    for b, hq in heads:
        hk = hq // group
        mrows = None
        if block_mask is not None:
            mrows = expand_block_mask(block_mask[b, hq], rows, Skv, mask_block_q, mask_block_kv)
        sp = 1.0 if sfs_p is None else float(sfs_p[hq])
        r = attention_head(
            qd[b, rows, hq], kd[b, :, hk], vd[b, :, hk], rows, Sq=Sq,
            softmax_scale=softmax_scale, causal=causal, mask_rows=mrows, mode=mode,
            p_format=p_format, sp=sp, tau=tau, sub_tile=sub_tile, flip_eps=flip_eps)
        if flip_eps is None:
            out[b, :, hq] = r
        else:
            out[b, :, hq], bound[b, :, hq] = r
    return out if flip_eps is None else (out, bound)


def output_e4m3(o, sfs_o=None):
    """Step 8: E4M3 codes (uint8) of an output O [B, S, Hq, D],
    encode(O / so[h]) with so = sfs_o[h] (fp32 [Hq]) or 1."""
    o = np.asarray(o, dtype=np.float64)
    so = np.ones(o.shape[2]) if sfs_o is None else np.asarray(sfs_o, dtype=np.float64)
    return e4m3_encode(o / so[None, None, :, None])
