"""The benchmark's host-side pieces (no GPU): the mask-aware pair count behind
the FLOP metric, the mixed MFMA peak, the traffic-record hash and the
one-GPU guard."""
import os
import subprocess
import sys

import numpy as np

import bench
from fmha_fwd_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_block_sparse_pair_count_matches_the_expanded_mask():
    # ragged query and key blocks (S = 300: 64-query blocks of 64 x 4 + 44,
    # 256-key blocks of 256 + 44), seeded mask with the diagonal block active
    spec = W.small_spec("sparse", 300, B=2, Hq=3, Hkv=3)
    data = W.generate(spec)
    bm = data["block_mask"].astype(bool)
    S = spec.S
    qb = np.arange(S) // 64
    kb = np.arange(S) // 256
    dense = bm[:, :, qb][:, :, :, kb]  # [B, Hq, S, S]: pair (i, j) active
    assert bench.pair_count(spec, data) == int(dense.sum())
    assert 0 < bench.pair_count(spec, data) < spec.B * spec.Hq * S * S


def test_dense_pair_count_is_the_spec_count():
    for base in ("dit", "gqa"):
        spec = W.small_spec(base, 200, B=1, Hq=4, Hkv=2)
        assert bench.pair_count(spec, {}) == spec.pairs()


def test_mixed_peak_is_the_time_weighted_mean():
    # half the FLOPs at 2500 and half at 5000 TFLOP/s: 1 / (0.5/2500 + 0.5/5000)
    assert abs(bench.mixed_peak("bf16", "e4m3") - 10000.0 / 3.0) < 1e-9
    for f in ("bf16", "e4m3", "int8"):
        assert bench.mixed_peak(f, f) == bench.PEAK[f]


def test_traffic_hash_ignores_comments_only(tmp_path):
    src = os.path.join(ROOT, "fmha_fwd_amd", "csrc", "attention.hip")
    text = open(src).read()
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    c = tmp_path / "c.hip"
    a.write_text(text)
    b.write_text("// a comment\n" + text.replace("\n", "\n\n", 3) + "/* block\ncomment */\n")
    c.write_text(text.replace("kSub = 64", "kSub = 32", 1))
    assert bench.code_text(str(a)) == bench.code_text(str(b))
    assert bench.code_text(str(a)) != bench.code_text(str(c))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_attention_bytes_closed_forms():
    # DiT-scale launch: bf16 Q, K and output, E4M3 V with one fp32 scale per 64 tokens
    dit = W.SPECS["dit"]
    n = 40 * 32760 * 128
    assert bench.attention_bytes(dit) == n * 2 + n * 2 + n * 1 + n * 2 + 40 * 512 * 4
    # 16 new positions of 64 sequences over an 8192-token E4M3 cache with 8 KV heads
    step = W.SPECS["gqa4_step"]
    q = 64 * 32 * 16 * 128
    kv = 64 * 8 * 8192 * 128
    scales = 4 * (64 * 32 * 1 + 2 * 64 * 8 * 128)
    assert bench.attention_bytes(step) == q + 2 * kv + 2 * q + scales
    # its bytes take longer at the HBM peak than its FLOPs at the fp8 peak; dit's the other way round
    assert step.pairs() * 4 * 128 / 5000e12 < bench.attention_bytes(step) / 8000e9
    assert dit.pairs() * 4 * 128 / bench.mixed_peak("bf16", "e4m3") / 1e12 > bench.attention_bytes(dit) / 8000e9
