"""Pins for the oracle's per-token NVFP4 quantisation: the E2M1 table from
its definition, a brute-force encoder check, a hand-derived example,
closed-form round-trip bounds and exact invariants."""
import json
import os

import numpy as np
import pytest
import torch

from oracle.codecs import e4m3_decode
from oracle.nvfp4 import (dequantize_nvfp4, e2m1_decode, e2m1_encode, quantize_nvfp4, unpack_codes)


def _bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


def test_e2m1_table(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "nvfp4_hand.json")))
    got = e2m1_decode(np.arange(16, dtype=np.uint8))
    want = np.array(g["e2m1_values"])
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))


def _nearest_even_bruteforce(v):
    """Nearest of the eight magnitudes by comparing every distance; ties to
    the even code; above 6 saturates."""
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    a = min(abs(v), 6.0)
    best = None
    for c, m in enumerate(mags):
        d = abs(a - m)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1] | (8 if np.signbit(v) else 0)


def test_e2m1_encode_bruteforce():
    vals = []
    for b in [0, 0.25, 0.5, 0.75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6, 6.5, 1e30]:
        for s in (1.0, -1.0):
            v = np.float32(b)
            for _ in range(4):
                vals += [s * v]
                v = np.nextafter(v, np.float32(np.inf))
            v = np.float32(b)
            for _ in range(4):
                v = np.nextafter(v, np.float32(-np.inf))
                vals += [s * abs(v)]
    vals += list(np.random.default_rng(5).uniform(-8, 8, 5000).astype(np.float32))
    vals = np.array(vals, dtype=np.float32)
    got = e2m1_encode(vals)
    want = np.array([_nearest_even_bruteforce(float(v)) for v in vals], dtype=np.uint8)
    assert np.array_equal(got, want)


def test_hand_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "nvfp4_hand.json")))
    x = np.array(g["x"], dtype=np.float32).reshape(1, -1)
    assert np.array_equal(_bf16(x), x)
    packed, sf, ts = quantize_nvfp4(x)
    assert ts[0] == np.float32(g["token_scale"])
    assert list(sf[0]) == g["block_scales"]
    assert list(unpack_codes(packed)[0]) == g["codes"]
    assert packed[0, 0] == g["first_byte"]


def _rows(seed, M=37, K=512):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x *= np.exp(rng.uniform(-6, 6, (M, 1))).astype(np.float32)
    x[:, rng.choice(K, 4, replace=False)] *= 30
    x[3, :] = 0.0
    x[5, 16:32] = 0.0
    return _bf16(x)


def test_amax_element_and_its_block():
    x = _rows(1)
    packed, sf, ts = quantize_nvfp4(x)
    codes = unpack_codes(packed)
    for r in range(x.shape[0]):
        if not np.any(x[r]):
            continue
        j = int(np.argmax(np.abs(x[r])))
        assert codes[r, j] & 7 == 7                 # the top element is +-6
        assert sf[r, j // 16] == 0x7E               # its block scale is 448
        assert ts[r] == np.float32(np.abs(x[r]).max()) / np.float32(2688.0)


def test_roundtrip_bound():
    # |x - deq| <= max(bs, bmax - 6 bs): half the widest E2M1 gap (one step
    # of bs, between 4 and 6) inside the range, the clamp outside it
    x = _rows(2)
    packed, sf, ts = quantize_nvfp4(x)
    deq = dequantize_nvfp4(packed, sf, ts)
    M, K = x.shape
    bs = e4m3_decode(sf) * ts[:, None].astype(np.float64)
    bmax = np.abs(x.reshape(M, K // 16, 16)).max(axis=2).astype(np.float64)
    bound = np.maximum(bs, bmax - 6 * bs) * (1 + 2.0 ** -20)
    err = np.abs(x.astype(np.float64) - deq).reshape(M, K // 16, 16).max(axis=2)
    assert np.all(err <= bound)
    # relative to the block maximum: at most 1/6 (+ E4M3 rounding of sf) where
    # the block scale is an E4M3 normal
    normal = e4m3_decode(sf) >= 2.0 ** -6
    assert np.all(err[normal] <= bmax[normal] * (1 / 6) * (1 + 2.0 ** -4) * (1 + 2.0 ** -20))


def test_dead_rows_and_zero_blocks():
    x = _rows(3)
    x[7] = 0.0
    x[7, 9] = -0.0
    packed, sf, ts = quantize_nvfp4(x)
    codes = unpack_codes(packed)
    for r in (3, 7):
        assert ts[r] == 1.0 and not np.any(sf[r]) and set(codes[r].tolist()) <= {0, 8}
    assert codes[7, 9] == 8                      # sign of zero kept
    assert sf[5, 1] == 0 and set(codes[5, 16:32].tolist()) <= {0, 8}
    tiny = np.full((1, 32), 2.0 ** -120, np.float32)  # below 2^-116: a dead row
    _, sf_t, ts_t = quantize_nvfp4(tiny)
    assert ts_t[0] == 1.0 and not np.any(sf_t)


def test_power_of_two_scaling_invariance():
    # multiplying a row by 2^k scales ts by 2^k and leaves every code and
    # block scale unchanged (each fp32 step scales exactly)
    x = _rows(4)
    live = np.abs(x).max(axis=1) > 0
    x = x[live]
    p0, s0, t0 = quantize_nvfp4(x)
    for k in (-7, 3, 11):
        p1, s1, t1 = quantize_nvfp4(x * np.float32(2.0 ** k))
        assert np.array_equal(p0, p1) and np.array_equal(s0, s1)
        assert np.array_equal(t1, t0 * np.float32(2.0 ** k))


def test_block_permutation_equivariance():
    x = _rows(5)
    M, K = x.shape
    perm = np.random.default_rng(6).permutation(K // 16)
    xp = x.reshape(M, K // 16, 16)[:, perm].reshape(M, K)
    p0, s0, t0 = quantize_nvfp4(x)
    p1, s1, t1 = quantize_nvfp4(xp)
    assert np.array_equal(t0, t1)
    assert np.array_equal(s0[:, perm], s1)
    assert np.array_equal(unpack_codes(p0).reshape(M, K // 16, 16)[:, perm].reshape(M, K), unpack_codes(p1))


def test_negation_flips_only_signs():
    x = _rows(6)
    p0, s0, t0 = quantize_nvfp4(x)
    p1, s1, t1 = quantize_nvfp4(-x)
    assert np.array_equal(s0, s1) and np.array_equal(t0, t1)
    assert np.array_equal(unpack_codes(p0) ^ 8, unpack_codes(p1))
