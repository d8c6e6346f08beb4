"""Input generators (no GPU): shapes, seeding and the pair counts behind the
FLOP metric."""
import numpy as np

from fmha_fwd_amd import workloads as W


def test_query_chunk_is_the_tail_of_the_full_sequence():
    full = W.generate(W.small_spec("gqa", 300, B=1, Hq=4, Hkv=2))
    chunk = W.generate(W.small_spec("gqa", 300, B=1, Hq=4, Hkv=2, sq=40))
    assert chunk["q"].shape == (1, 40, 4, 128)
    assert np.array_equal(chunk["q"], full["q"][:, 260:])
    assert np.array_equal(chunk["k"], full["k"]) and np.array_equal(chunk["v"], full["v"])


def test_pair_counts_match_brute_force():
    for causal in (False, True):
        for sq in (0, 1, 37, 300):
            spec = W.small_spec("gqa", 300, B=2, Hq=4, Hkv=2, causal=causal, sq=sq)
            nq, S = spec.n_q, spec.S
            i = np.arange(nq)[:, None]
            j = np.arange(S)[None, :]
            valid = (j <= i + S - nq) if causal else np.ones((nq, S), bool)
            assert spec.pairs() == spec.B * spec.Hq * int(valid.sum())


def test_seeded_and_bf16_valued():
    a = W.generate(W.small_spec("dit", 130, B=1, Hq=2, Hkv=2))
    b = W.generate(W.small_spec("dit", 130, B=1, Hq=2, Hkv=2))
    for n in ("q", "k", "v"):
        assert np.array_equal(a[n], b[n])
        bits = a[n].view(np.uint32)
        assert np.all(bits & 0xFFFF == 0)  # bf16 values held in float32


def test_sweep_cases_are_seeded_and_well_formed():
    for i in range(48):
        spec, data, kvb = W.sweep_case(i)
        again = W.sweep_case(i)[1]
        B, Sq, Hq, D = data["q"].shape
        _, Skv, Hkv, _ = data["k"].shape
        assert (B, Hq, Hkv, D, Skv) == (spec.B, spec.Hq, spec.Hkv, spec.D, spec.S) and spec.n_q == Sq
        assert Hq % Hkv == 0 and D in (128, 192) and Sq >= 1 and Skv >= 1
        for n in data:
            assert np.array_equal(data[n], again[n])
        if spec.paged:
            pt = data["page_table"]
            assert pt.shape == (B, -(-Skv // spec.page_size))
            assert len(np.unique(pt)) == pt.size and pt.min() >= 0  # each page holds one sequence's tokens
        if spec.masked:
            assert data["block_mask"].shape == (B, Hq, -(-Sq // 64), -(-Skv // kvb))
