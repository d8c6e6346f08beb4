"""Pins for the oracle's number formats: closed-form cases and torch's casts."""
import numpy as np
import pytest
import torch

from oracle.codecs import (bf16_round, bf16_round64, e4m3_decode, e4m3_encode,
                           int8_encode)


def test_e4m3_decode_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])
    assert ours[0x7E] == 448.0 and ours[0x08] == 2.0 ** -6 and ours[0x01] == 2.0 ** -9


def _midpoints_and_neighbours():
    vals = e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2
    pts = [vals, mids]
    for m in (vals, mids):
        f = m.astype(np.float32)
        pts.append(np.nextafter(f, np.float32(np.inf)).astype(np.float64))
        pts.append(np.nextafter(f, np.float32(-np.inf)).astype(np.float64))
    x = np.concatenate(pts)
    return np.concatenate([x, -x]).astype(np.float32)


def test_e4m3_encode_matches_torch_in_range():
    x = _midpoints_and_neighbours()
    rng = np.random.default_rng(0)
    x = np.concatenate([x, (rng.standard_normal(100000) * np.exp(rng.uniform(-9, 6, 100000))).astype(np.float32)])
    x = x[np.abs(x) < 448]  # torch's cast does not saturate above the range
    ours = e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


@pytest.mark.parametrize("x,code", [
    (448.0, 0x7E), (460.0, 0x7E), (464.0, 0x7E), (1e6, 0x7E), (np.inf, 0x7E),
    (-500.0, 0xFE), (0.0, 0x00), (-0.0, 0x80),
    (2.0 ** -10, 0x00),            # midpoint of 0 and 2^-9 -> even code 0
    (3 * 2.0 ** -10, 0x02),        # midpoint of 2^-9 (code 1) and 2^-8 (code 2) -> 2
    (1.0 + 1.0 / 16, 0x38),        # midpoint of 1 (0x38) and 1.125 (0x39) -> 0x38
    (1.0 + 3.0 / 16, 0x3A),        # midpoint of 1.125 (0x39) and 1.25 (0x3A) -> 0x3A
    (90.5, 0x6B),                  # nearest 88 = 1.375*2^6 (0x6B)
    (157.59, 0x72),                # nearest 160 = 1.25*2^7 (0x72)
])
def test_e4m3_encode_closed_form(x, code):
    assert int(e4m3_encode(np.array([x]))[0]) == code


def test_e4m3_encode_nan():
    assert int(e4m3_encode(np.array([np.nan]))[0]) & 0x7F == 0x7F


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-60, 60, 200000))).astype(np.float32)
    # exact ties: low 16 bits == 0x8000
    u = rng.integers(0, 2 ** 31, 1000, dtype=np.uint64).astype(np.uint32)
    ties = ((u & 0xFFFF0000) | 0x8000).view(np.float32)
    ties = ties[np.isfinite(ties)]
    x = np.concatenate([x, ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(bf16_round(x), ref)


def test_bf16_round64_agrees_on_binary32_inputs_and_ties():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(50000) * np.exp(rng.uniform(-80, 80, 50000))).astype(np.float32)
    assert np.array_equal(bf16_round64(x.astype(np.float64)), bf16_round(x).astype(np.float64))
    # fp64 ties and near-ties that a binary32 detour would round twice
    assert bf16_round64(np.array([1 + 2.0 ** -8]))[0] == 1.0
    assert bf16_round64(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6
    assert bf16_round64(np.array([1 + 2.0 ** -8 + 2.0 ** -40]))[0] == 1 + 2.0 ** -7
    assert bf16_round64(np.array([2.0 ** -133 * 0.5]))[0] == 0.0
    assert bf16_round64(np.array([2.0 ** -133 * 1.5]))[0] == 2.0 ** -132


@pytest.mark.parametrize("x,c", [(0.5, 0), (1.5, 2), (2.5, 2), (-0.5, 0), (-1.5, -2),
                                 (126.5, 126), (127.4, 127), (200.0, 127), (-200.0, -127),
                                 (-127.5, -127), (63.5, 64), (31.75, 32)])
def test_int8_encode_closed_form(x, c):
    assert int(int8_encode(np.array([x]))[0]) == c
