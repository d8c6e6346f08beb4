"""Pins for the attention oracle: a library routine for the unquantised case,
hand-derived lazy-rescale examples, and invariants the mathematics fixes."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle.attention import attention, dequantize, gather_pages, output_e4m3
from oracle.codecs import e4m3_decode
from oracle.quantize import quantize_blocks


def _sdpa(qd, kd, vd, causal=False, block_mask=None, scale=None, mask_block_q=64, mask_block_kv=256):
    """torch's CPU scaled_dot_product_attention in fp64 (heads expanded for GQA;
    a block mask expanded to pairs by repeating each entry over its block)."""
    B, Sq, Hq, D = qd.shape
    Skv, Hkv = kd.shape[1], kd.shape[2]
    g = Hq // Hkv
    q = torch.from_numpy(qd).permute(0, 2, 1, 3)
    k = torch.from_numpy(kd).permute(0, 2, 1, 3).repeat_interleave(g, dim=1)
    v = torch.from_numpy(vd).permute(0, 2, 1, 3).repeat_interleave(g, dim=1)
    mask = torch.ones(B, Hq, Sq, Skv, dtype=torch.bool)
    if causal:
        i = torch.arange(Sq)[:, None]
        j = torch.arange(Skv)[None, :]
        mask &= (j <= i + Skv - Sq)
    if block_mask is not None:
        bm = torch.from_numpy(block_mask != 0)
        mask &= bm.repeat_interleave(mask_block_q, 2)[:, :, :Sq].repeat_interleave(mask_block_kv, 3)[..., :Skv]
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


@pytest.mark.parametrize("B,Sq,Skv,Hq,Hkv,D,causal", [
    (1, 5, 7, 1, 1, 16, False), (2, 70, 70, 4, 2, 16, True), (1, 33, 150, 6, 3, 8, False),
    (1, 150, 130, 2, 1, 8, True), (2, 64, 64, 2, 2, 32, True)])
@pytest.mark.parametrize("mode", ["lazy", "exact"])
def test_unquantized_matches_torch_sdpa(B, Sq, Skv, Hq, Hkv, D, causal, mode):
    qd = _rand((B, Sq, Hq, D), 1, 2.0)
    kd = _rand((B, Skv, Hkv, D), 2, 2.0)
    vd = _rand((B, Skv, Hkv, D), 3)
    got = attention(qd, kd, vd, causal=causal, mode=mode)
    ref = _sdpa(qd, kd, vd, causal=causal, scale=1 / math.sqrt(D))
    assert np.allclose(got, ref, rtol=1e-10, atol=1e-12)


def test_unquantized_block_mask_matches_torch_sdpa():
    B, S, H, D = 1, 600, 2, 8
    rng = np.random.default_rng(9)
    qd, kd, vd = (rng.standard_normal((B, S, H, D)) for _ in range(3))
    nqb, nkb = -(-S // 64), -(-S // 256)
    bm = (rng.random((B, H, nqb, nkb)) < 0.5).astype(np.uint8)
    for qb in range(nqb):
        bm[:, :, qb, min(qb // 4, nkb - 1)] = 1  # every row keeps a block
    got = attention(qd, kd, vd, block_mask=bm)
    assert np.allclose(got, _sdpa(qd, kd, vd, block_mask=bm, scale=1 / math.sqrt(D)), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("kv_block", [64, 192, 512])
@pytest.mark.parametrize("causal", [False, True])
def test_block_mask_key_block_sizes_match_torch_sdpa(kv_block, causal):
    """expand_block_mask at key-block sizes other than 256 (the sizes the
    kernel accepts: positive multiples of 64), with ragged last blocks on both
    axes, against torch's attention under the pair mask built by repetition."""
    B, Sq, Skv, H, D = 2, 200, 1100, 3, 8
    rng = np.random.default_rng(kv_block + 7 * causal)
    qd = rng.standard_normal((B, Sq, H, D)) * 2.0
    kd = rng.standard_normal((B, Skv, H, D)) * 2.0
    vd = rng.standard_normal((B, Skv, H, D))
    nqb, nkb = -(-Sq // 64), -(-Skv // kv_block)
    bm = (rng.random((B, H, nqb, nkb)) < 0.4).astype(np.uint8)
    bm[..., nkb - 1] = 1  # every row keeps its last key block (visible under bottom-right causal)
    for mode in ("lazy", "exact"):
        got = attention(qd, kd, vd, block_mask=bm, causal=causal, mode=mode, mask_block_kv=kv_block)
        ref = _sdpa(qd, kd, vd, causal=causal, block_mask=bm, scale=1 / math.sqrt(D), mask_block_kv=kv_block)
        assert np.allclose(got, ref, rtol=1e-10, atol=1e-12), (kv_block, mode)
    # a different key-block size is a different mask: the pin can tell them apart
    other = attention(qd, kd, vd, block_mask=bm, causal=causal, mode="exact", mask_block_kv=2 * kv_block)
    assert not np.allclose(other, ref, rtol=1e-6, atol=1e-8)


def test_softmax_scale_is_applied():
    qd, kd, vd = _rand((1, 9, 1, 4), 4), _rand((1, 11, 1, 4), 5), _rand((1, 11, 1, 4), 6)
    got = attention(qd, kd, vd, softmax_scale=0.37)
    assert np.allclose(got, _sdpa(qd, kd, vd, scale=0.37), rtol=1e-10, atol=1e-12)


def _hand_inputs(kvals):
    Skv = 66
    k = np.full(Skv, -1000.0)
    k[[0, 1, 64, 65]] = kvals
    v = np.zeros(Skv)
    v[[0, 1, 64, 65]] = [1.0, 10.0, 100.0, 1000.0]
    qd = np.ones((1, 1, 1, 1))
    return qd, k.reshape(1, Skv, 1, 1), v.reshape(1, Skv, 1, 1)


@pytest.mark.parametrize("case", [0, 1, 2])
def test_lazy_rescale_hand_examples(golden_dir, case):
    g = json.load(open(os.path.join(golden_dir, "lazy_hand.json")))["cases"][case]
    qd, kd, vd = _hand_inputs(g["k"])
    run = lambda **kw: float(attention(qd, kd, vd, softmax_scale=math.log(2.0), **kw)[0, 0, 0, 0])
    assert run(mode="lazy", p_format="e4m3") == pytest.approx(g["lazy_e4m3"], rel=1e-12)
    assert run(mode="exact", p_format="e4m3") == pytest.approx(g["exact_e4m3"], rel=1e-12)
    if "unquantized" in g:
        assert run(mode="lazy") == pytest.approx(g["unquantized"], rel=1e-12)
        assert run(mode="exact") == pytest.approx(g["unquantized"], rel=1e-12)
    if "lazy_bf16" in g:
        assert run(mode="lazy", p_format="bf16") == pytest.approx(g["lazy_bf16"], rel=1e-12)
    if "lazy_e4m3_sp_quarter" in g:
        assert run(mode="lazy", p_format="e4m3", sfs_p=[0.25]) == pytest.approx(g["lazy_e4m3_sp_quarter"], rel=1e-12)


@pytest.mark.parametrize("tau", [0.0, 3.0, 8.0, 30.0])
def test_lazy_equals_exact_without_p_quantisation(tau):
    # large score range so that rescales happen for every tau
    qd, kd, vd = _rand((1, 40, 2, 16), 11, 3.0), _rand((1, 300, 2, 16), 12, 3.0), _rand((1, 300, 2, 16), 13)
    a = attention(qd, kd, vd, mode="lazy", tau=tau)
    b = attention(qd, kd, vd, mode="exact")
    assert np.allclose(a, b, rtol=1e-10, atol=1e-12)


def test_lazy_equals_exact_when_max_is_in_first_subtile():
    rng = np.random.default_rng(14)
    D, Skv = 16, 300
    qd = rng.standard_normal((1, 50, 1, D))
    kd = rng.standard_normal((1, Skv, 1, D))
    vd = rng.standard_normal((1, Skv, 1, D))
    qd[..., 0] = 1.0
    kd[..., 0] = 0.0
    kd[0, 0, 0, 0] = 200.0  # key 0 dominates every row
    a = attention(qd, kd, vd, mode="lazy", p_format="e4m3")
    b = attention(qd, kd, vd, mode="exact", p_format="e4m3")
    assert np.array_equal(a, b)


def _quantized_case(seed, B=1, Sq=130, Skv=200, Hq=2, Hkv=2, D=32, spread=2.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Sq, Hq, D)).astype(np.float32) * spread
    k = rng.standard_normal((B, Skv, Hkv, D)).astype(np.float32) * spread
    v = rng.standard_normal((B, Skv, Hkv, D)).astype(np.float32)
    qc, qs = quantize_blocks(q, "e4m3")
    kc, ks = quantize_blocks(k, "e4m3")
    vc, vs = quantize_blocks(v, "e4m3")
    return (dequantize(qc, "e4m3", qs), dequantize(kc, "e4m3", ks), dequantize(vc, "e4m3", vs))


@pytest.mark.parametrize("mode", ["lazy", "exact"])
@pytest.mark.parametrize("causal", [False, True])
def test_rows_sum_to_one(mode, causal):
    qd, kd, vd = _quantized_case(15)
    ones = np.ones_like(vd)
    o = attention(qd, kd, ones, mode=mode, p_format="e4m3", causal=causal)
    assert np.allclose(o, 1.0, rtol=0, atol=1e-12)


@pytest.mark.parametrize("mode", ["lazy", "exact"])
def test_constant_v_gives_v(mode):
    qd, kd, vd = _quantized_case(16)
    cv = np.broadcast_to(vd[:, :1], vd.shape).copy()  # every key carries key 0's value
    o = attention(qd, kd, cv, mode=mode, p_format="e4m3")
    assert np.allclose(o, np.repeat(cv[:, :1], qd.shape[2] // kd.shape[2], axis=2)[:, [0] * qd.shape[1]], rtol=1e-12, atol=1e-12)


def test_key_permutation_invariance_unquantized():
    qd, kd, vd = _rand((1, 20, 2, 8), 17), _rand((1, 90, 2, 8), 18), _rand((1, 90, 2, 8), 19)
    perm = np.random.default_rng(20).permutation(90)
    a = attention(qd, kd, vd, mode="lazy")
    b = attention(qd, kd[:, perm], vd[:, perm], mode="lazy")
    assert np.allclose(a, b, rtol=1e-10, atol=1e-12)


def test_block_permutation_invariance_quantized_exact():
    qd, kd, vd = _quantized_case(21, Skv=256)
    perm = np.concatenate([np.arange(64) + 64 * b for b in [2, 0, 3, 1]])
    a = attention(qd, kd, vd, mode="exact", p_format="e4m3")
    b = attention(qd, kd[:, perm], vd[:, perm], mode="exact", p_format="e4m3")
    assert np.allclose(a, b, rtol=1e-12, atol=1e-13)


def test_masked_blocks_contribute_nothing_even_if_nan():
    B, S, H, D = 1, 600, 2, 16
    qd, kd, vd = (_rand((B, S, H, D), s) for s in (22, 23, 24))
    nqb, nkb = 10, 3
    bm = np.ones((B, H, nqb, nkb), dtype=np.uint8)
    bm[:, :, :, 1] = 0  # keys 256..511 inactive for every query block
    a = attention(qd, kd, vd, block_mask=bm, mode="lazy", p_format="e4m3")
    kd2, vd2 = kd.copy(), vd.copy()
    kd2[:, 256:512] = np.nan
    vd2[:, 256:512] = np.nan
    b = attention(qd, kd2, vd2, block_mask=bm, mode="lazy", p_format="e4m3")
    assert np.all(np.isfinite(b)) and np.array_equal(a, b)
    ref = _sdpa(qd, kd, vd, block_mask=bm, scale=1 / math.sqrt(D))
    assert np.allclose(attention(qd, kd2, vd2, block_mask=bm), ref, rtol=1e-10, atol=1e-12)


def test_gqa_equals_mha_with_repeated_heads():
    qd, kd, vd = _quantized_case(25, Hq=6, Hkv=2)
    a = attention(qd, kd, vd, mode="lazy", p_format="e4m3")
    b = attention(qd, np.repeat(kd, 3, axis=2), np.repeat(vd, 3, axis=2), mode="lazy", p_format="e4m3")
    assert np.array_equal(a, b)


def test_causal_row0_and_single_key():
    qd, kd, vd = _quantized_case(26, Sq=100, Skv=100)
    o = attention(qd, kd, vd, causal=True, mode="lazy", p_format="e4m3")
    assert np.array_equal(o[:, 0], vd[:, 0])
    o1 = attention(qd, kd[:, :1], vd[:, :1], mode="lazy", p_format="e4m3")
    assert np.array_equal(o1, np.broadcast_to(vd[:, :1], o1.shape))


def test_row_without_valid_key_is_zero():
    qd, kd, vd = _rand((1, 70, 1, 8), 27), _rand((1, 300, 1, 8), 28), _rand((1, 300, 1, 8), 29)
    bm = np.ones((1, 1, 2, 2), dtype=np.uint8)
    bm[0, 0, 1, :] = 0  # query block 1 (rows 64..69) sees nothing
    o = attention(qd, kd, vd, block_mask=bm, mode="lazy", p_format="e4m3")
    assert np.all(o[0, 64:] == 0) and np.all(np.abs(o[0, :64]).sum(-1) > 0)


def test_rows_subset_matches_full():
    qd, kd, vd = _quantized_case(30, Sq=200)
    rows = np.array([0, 63, 64, 199])
    full = attention(qd, kd, vd, mode="lazy", p_format="e4m3", causal=True)
    part = attention(qd, kd, vd, mode="lazy", p_format="e4m3", causal=True, rows=rows)
    assert np.array_equal(full[:, rows], part)


def test_dequantize_uses_the_tokens_block_scale():
    codes = np.zeros((1, 130, 1, 2), dtype=np.int8)
    codes[0, :, 0, 0] = 1
    scales = np.array([[[2.0, 3.0, 5.0]]], dtype=np.float32)
    d = dequantize(codes, "int8", scales)
    assert np.all(d[0, :64, 0, 0] == 2) and np.all(d[0, 64:128, 0, 0] == 3) and np.all(d[0, 128:, 0, 0] == 5)
    assert np.all(d[..., 1] == 0)
    e = dequantize(np.full((1, 1, 1, 1), 0x38, dtype=np.uint8), "e4m3", np.array([[[0.5]]], dtype=np.float32))
    assert e.item() == 0.5


def test_gather_pages():
    rng = np.random.default_rng(31)
    B, S, H, D, P = 2, 64, 1, 4, 16
    logical = rng.standard_normal((B, S, H, D))
    perm = rng.permutation(B * S // P)
    pt = perm.reshape(B, S // P)
    pool = np.zeros((B * S // P, P, H, D))
    for b in range(B):
        for p in range(S // P):
            pool[pt[b, p]] = logical[b, p * P:(p + 1) * P]
    assert np.array_equal(gather_pages(pool, pt, S, P), logical)


def test_rounding_sensitivity_bound_hand_example():
    # EXACT mode, trigger case: P(key 0) = 2^-10 lies exactly on the E4M3
    # boundary between 0 and 2^-9 (the tie goes to 0, O = 400).  Bound:
    # 2^-9 * |v0 - O| / den = 2^-9 * 399 / 1.5.
    qd, kd, vd = _hand_inputs([0.0, -1.0, 10.0, 9.0])
    o, bound = attention(qd, kd, vd, softmax_scale=math.log(2.0), mode="exact", p_format="e4m3", flip_eps=1e-6)
    assert o.item() == pytest.approx(400.0, rel=1e-12)
    assert bound.item() == pytest.approx(2.0 ** -9 * 399 / 1.5, rel=1e-9)
    # nudging key 0 over the boundary moves O by just under the bound
    qd2, kd2, vd2 = _hand_inputs([1e-6, -1.0, 10.0, 9.0])
    o2 = attention(qd2, kd2, vd2, softmax_scale=math.log(2.0), mode="exact", p_format="e4m3")
    assert 0.5 < abs(o2.item() - o.item()) <= bound.item()
    # no tie: zero bound, and the output does not depend on flip_eps
    o3, b3 = attention(qd, kd, vd, softmax_scale=math.log(2.0), mode="lazy", p_format="e4m3", flip_eps=1e-6)
    assert b3.item() == 0.0 and o3.item() == pytest.approx(399.61365853658536, rel=1e-12)


@pytest.mark.parametrize("p_format", ["e4m3", "bf16"])
def test_rounding_sensitivity_bound_covers_tiny_score_perturbations(p_format):
    qd, kd, vd = _quantized_case(32, Sq=192, Skv=700, Hq=2, Hkv=1, spread=3.0)
    o, bound = attention(qd, kd, vd, mode="lazy", p_format=p_format, flip_eps=1e-6)
    for f in (1 + 2.0 ** -30, 1 - 2.0 ** -30):
        o2 = attention(qd * f, kd, vd, mode="lazy", p_format=p_format)
        # flips are bounded by `bound`; the rescale factors move continuously
        # (relative 2^-30 of the scores, ~1e-8 here)
        assert np.all(np.abs(o2 - o) <= bound + 1e-6)


def test_output_e4m3_hand_values():
    # codes worked out by hand from the E4M3 definition: 448 = 1.75 * 2^8 is
    # S.1111.110; beyond it the encoder saturates; 0.3 = 1.2 * 2^-2 rounds to
    # 1.25 * 2^-2 (S.0101.010); 2^-10 lies half-way between 0 and the
    # smallest subnormal 2^-9 and goes to the even code 0; 0.75 * 2^-9 rounds
    # up to 2^-9 (S.0000.001)
    so = np.array([0.5, 2.0])
    vals = np.array([448.0, 500.0, -1000.0, 0.3, 2.0 ** -10, 0.75 * 2.0 ** -9, 0.0, -0.3])
    o = np.zeros((1, len(vals), 2, 1))
    o[0, :, 0, 0] = vals * so[0]
    o[0, :, 1, 0] = vals * so[1]
    want = np.array([0x7E, 0x7E, 0xFE, 0x2A, 0x00, 0x01, 0x00, 0xAA], dtype=np.uint8)
    got = output_e4m3(o, so)
    assert np.array_equal(got[0, :, 0, 0], want) and np.array_equal(got[0, :, 1, 0], want)
    # no scale: the values themselves
    assert np.array_equal(output_e4m3(o[:, :, :1] / so[0])[0, :, 0, 0], want)


@pytest.mark.parametrize("p_format", ["e4m3", "bf16"])
def test_binary32_bound_covers_a_binary32_evaluation(p_format):
    """The per-pair binary32 bound against an independent binary32 evaluation
    of the same attention (exact mode: scores by a float32 matrix product,
    scale, maximum, subtraction and exp2 in float32, then the same P format).
    Every output element lies within the bound of the fp64 result, the bound
    is needed (some P values do round the other way), and it is tighter than a
    fixed relative distance of 2^-11."""
    from oracle.codecs import bf16_round64, e4m3_round
    rng = np.random.default_rng(77)
    n, Skv, D = 256, 4096, 128
    # bf16-valued operands, exactly representable in float32
    q = W_bf16(rng.standard_normal((1, n, 1, D)) * 1.5)
    k = W_bf16(rng.standard_normal((1, Skv, 1, D)) * 1.5)
    v = W_bf16(rng.standard_normal((1, Skv, 1, D)))
    c = (1.0 / math.sqrt(D)) * (1.0 / math.log(2.0))
    o, bound = attention(q, k, v, mode="exact", p_format=p_format, flip_eps="binary32")
    s32 = (q[0, :, 0].astype(np.float32) @ k[0, :, 0].astype(np.float32).T) * np.float32(c)
    m32 = s32.max(axis=1, keepdims=True)
    p32 = np.exp2((s32 - m32).astype(np.float32)).astype(np.float64)
    w = e4m3_round(p32) if p_format == "e4m3" else bf16_round64(p32)
    o32 = (w @ v[0, :, 0]) / w.sum(axis=1, keepdims=True)
    s64 = (q[0, :, 0] @ k[0, :, 0].T) * c
    p64 = np.exp2(s64 - s64.max(axis=1, keepdims=True))
    w64 = e4m3_round(p64) if p_format == "e4m3" else bf16_round64(p64)
    flips = int((w != w64).sum())  # P values the binary32 evaluation rounds the other way
    assert flips > 0, "no P rounded the other way: the case does not exercise the bound"
    assert np.all(np.abs(o32 - o[0, :, 0]) <= bound[0, :, 0] + 1e-9)
    _, fixed = attention(q, k, v, mode="exact", p_format=p_format, flip_eps=2.0 ** -11)
    assert bound.sum() < fixed.sum()


def test_binary32_bound_covers_the_reference_maximum_error():
    """Lazy attention with every score moved to the edge of its binary32
    accumulation bound (e = c gamma_D sum_d |q_d k_d|, which some summation
    order can reach): the key holding a sub-tile's maximum moves up, every
    other key down, so each P = 2^(s - m) errs by ln 2 (e_j + e_m).  The
    output stays within the oracle's bound, and some of the P values that
    round the other way lie outside the window of the pair's own error: the
    reference maximum's accumulation error is what covers them."""
    from oracle.attention import LOG2E, binary32_accumulation_error, binary32_p_error
    from oracle.codecs import e4m3_round, rounding_gap
    rng = np.random.default_rng(5)
    n, Skv, D, tau = 128, 2048, 128, 8.0
    q = W_bf16(rng.standard_normal((1, n, 1, D)) * 1.5)
    k = W_bf16(rng.standard_normal((1, Skv, 1, D)) * 1.5)
    v = W_bf16(rng.standard_normal((1, Skv, 1, D)))
    c = (1.0 / math.sqrt(D)) * LOG2E
    o, bound = attention(q, k, v, mode="lazy", p_format="e4m3", tau=tau, flip_eps="binary32")
    qq, kk, vv = q[0, :, 0], k[0, :, 0], v[0, :, 0]
    s = (qq @ kk.T) * c
    e = binary32_accumulation_error(qq, kk, D, c)
    rows = np.arange(n)
    m = np.full(n, -np.inf)       # reference from the moved scores
    m_x = np.full(n, -np.inf)     # reference from the exact scores
    num, den = np.zeros((n, D)), np.zeros(n)
    flips = beyond_pair = 0
    for t0 in range(0, Skv, 64):
        cols = slice(t0, t0 + 64)
        sx = s[:, cols]
        top = np.argmax(sx, axis=1)
        se = sx - e[:, cols]
        se[rows, top] = sx[rows, top] + e[rows, t0 + top]
        tx, te = sx.max(axis=1), se.max(axis=1)
        trig = (m_x == -np.inf) | (tx - m_x > tau)
        assert np.array_equal(trig, (m == -np.inf) | (te - m > tau))  # margins far above e
        # rescale by the exact references' factor: the bound covers P values
        # that round the other way; the continuous error of the factor itself
        # is left to the max-abs bar
        alpha = np.where(m_x == -np.inf, 0.0, np.exp2(np.where(trig, m_x - tx, 0.0)))
        num *= alpha[:, None]
        den *= alpha
        m, m_x = np.where(trig, te, m), np.where(trig, tx, m_x)
        w = e4m3_round(np.exp2(se - m[:, None]))
        px = np.exp2(sx - m_x[:, None])
        num += w @ vv[cols]
        den += w.sum(axis=1)
        flip = w != e4m3_round(px)
        pair_only = binary32_p_error(qq, kk[cols], sx, m_x, D, c, 1.0)
        flips += int(flip.sum())
        beyond_pair += int((flip & (rounding_gap(px, "e4m3", pair_only) == 0)).sum())
    o_edge = num / den[:, None]
    assert flips > 0 and beyond_pair > 0, (flips, beyond_pair)
    # the bound is first order: 1 % covers the products of the flips
    assert np.all(np.abs(o_edge - o[0, :, 0]) <= 1.01 * bound[0, :, 0] + 1e-12)


def W_bf16(x):
    from fmha_fwd_amd.workloads import to_bf16_values
    return to_bf16_values(np.asarray(x, dtype=np.float32)).astype(np.float64)
