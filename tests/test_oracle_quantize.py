"""Pins for the oracle's block quantisation: hand example, closed-form bounds."""
import json
import os

import numpy as np
import pytest
import torch

from oracle.codecs import e4m3_decode
from oracle.quantize import quantize_blocks


def _bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


@pytest.mark.parametrize("fmt", ["int8", "e4m3"])
def test_hand_example(golden_dir, fmt):
    g = json.load(open(os.path.join(golden_dir, "quantize_hand.json")))
    x = np.array(g["x"], dtype=np.float32).reshape(1, 1, 1, 3)
    codes, scales = quantize_blocks(x, fmt)
    exp = g[fmt]
    got = codes.reshape(-1).astype(np.int64)
    want = np.array(exp["codes"], dtype=np.int64)
    if fmt == "e4m3":
        got = got & 0xFF
    assert list(got) == list(want)
    assert scales.reshape(-1)[0] == np.float32(exp["scale_num"]) / np.float32(exp["scale_den"])


def _random_blocks(seed, B=2, S=200, H=3, D=128):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, S, H, D)).astype(np.float32)
    x *= np.exp(rng.uniform(-4, 4, (B, 1, H, 1))).astype(np.float32)
    return _bf16(x)


@pytest.mark.parametrize("fmt,qmax", [("int8", 127.0), ("e4m3", 448.0)])
def test_amax_element_maps_to_qmax(fmt, qmax):
    x = _random_blocks(3)
    codes, scales = quantize_blocks(x, fmt)
    B, S, H, D = x.shape
    for b in range(B):
        for h in range(H):
            for k in range(scales.shape[2]):
                blk = x[b, 64 * k:64 * k + 64, h]
                i = np.unravel_index(np.argmax(np.abs(blk)), blk.shape)
                c = codes[b, 64 * k:64 * k + 64, h][i]
                val = float(c) if fmt == "int8" else float(e4m3_decode(np.array([c]))[0])
                assert abs(val) == qmax
                assert np.sign(val) == np.sign(blk[i])


def test_int8_round_trip_bound():
    x = _random_blocks(4)
    codes, scales = quantize_blocks(x, "int8")
    s = np.repeat(scales, 64, axis=2)[:, :, :x.shape[1]].transpose(0, 2, 1)[..., None].astype(np.float64)
    err = np.abs(x.astype(np.float64) - codes.astype(np.float64) * s)
    # |y - code| <= 1/2 after rounding; three binary32 roundings (scale, inv,
    # x*inv) move x*inv by at most 3*2^-24 relative, |x*inv| <= 127(1+2^-22)
    bound = s * (0.5 + 127.0 * 4 * 2.0 ** -24)
    assert np.all(err <= bound)
    assert np.all(np.abs(codes.astype(np.int64)) <= 127)


def test_e4m3_round_trip_bound():
    x = _random_blocks(5)
    codes, scales = quantize_blocks(x, "e4m3")
    s = np.repeat(scales, 64, axis=2)[:, :, :x.shape[1]].transpose(0, 2, 1)[..., None].astype(np.float64)
    dq = e4m3_decode(codes) * s
    xd = x.astype(np.float64)
    err = np.abs(xd - dq)
    normal = np.abs(xd) >= 2.0 ** -6 * s
    # normal range: half a unit in the 3-bit mantissa (2^-4 relative) plus
    # binary32 rounding of scale/inv/x*inv; subnormal range: half of 2^-9
    assert np.all(err[normal] <= np.abs(xd[normal]) * (2.0 ** -4 + 4 * 2.0 ** -24))


def test_e4m3_subnormal_range_bound():
    x = _random_blocks(6)
    codes, scales = quantize_blocks(x, "e4m3")
    s = np.broadcast_to(np.repeat(scales, 64, axis=2)[:, :, :x.shape[1]].transpose(0, 2, 1)[..., None], x.shape).astype(np.float64)
    xd = x.astype(np.float64)
    sub = np.abs(xd) < 2.0 ** -6 * s
    err = np.abs(xd - e4m3_decode(codes) * s)
    assert sub.any()
    assert np.all(err[sub] <= (2.0 ** -10 + 2.0 ** -18) * s[sub])


@pytest.mark.parametrize("fmt", ["int8", "e4m3"])
def test_tail_block_uses_only_existing_tokens(fmt):
    x = _random_blocks(7, B=1, S=130, H=2)
    codes, scales = quantize_blocks(x, fmt)
    assert scales.shape == (1, 2, 3)
    c2, s2 = quantize_blocks(x[:, 128:], fmt)
    assert np.array_equal(codes[:, 128:], c2) and np.array_equal(scales[:, :, 2:], s2)


@pytest.mark.parametrize("fmt", ["int8", "e4m3"])
def test_zero_and_tiny_blocks(fmt):
    x = np.zeros((1, 128, 1, 128), dtype=np.float32)
    x[0, 64:, 0, :5] = np.float32(2.0 ** -130)  # bf16-representable, below 2^-126
    codes, scales = quantize_blocks(x, fmt)
    assert np.all(codes == 0) and np.all(scales == 1.0)


def test_blocks_are_independent_across_heads():
    x = _random_blocks(8)
    codes, scales = quantize_blocks(x, "int8")
    perm = [2, 0, 1]
    c2, s2 = quantize_blocks(x[:, :, perm], "int8")
    assert np.array_equal(c2, codes[:, :, perm]) and np.array_equal(s2, scales[:, perm])
