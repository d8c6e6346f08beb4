"""Seeded random sweep of fmha_fwd against the oracle: each case draws a
format combination, head dim, batch, GQA grouping, ragged query and key
lengths, causal, a block mask and paged K/V at random (workloads.sweep_case)
and is compared element by element, with the same bar as every other parity
test."""
import numpy as np
import pytest

from fmha_fwd_amd import workloads as W
import harness as Hn

N_CASES = 48


@pytest.mark.gpu
@pytest.mark.parametrize("i", range(N_CASES))
def test_random_configuration(i):
    spec, data, kvb = W.sweep_case(i)
    Sq, Skv = data["q"].shape[1], data["k"].shape[1]
    what = (f"{spec.name} D={spec.D} B={spec.B} Hq/Hkv={spec.Hq}/{spec.Hkv} Sq={Sq} Skv={Skv} causal={spec.causal} "
            f"mask={'64x%d' % kvb if spec.masked else None} pages={spec.page_size if spec.paged else None}")
    print(f"fwd sweep {what}", flush=True)
    kw = {"mask_block": (64, kvb)} if spec.masked else {}
    gpu, _ = Hn.gpu_run(spec, data, **kw)
    okw = {"mask_block_kv": kvb} if spec.masked else {}
    ops = Hn.oracle_operands(spec, data)
    ref = Hn.oracle_output(spec, data, ops, **okw)
    unq = Hn.unquantized_output(spec, data, **okw)
    Hn.assert_parity(gpu, ref, unq, what=what)
    # rows with no valid key are exactly zero
    dead = ~np.isfinite(ref[0]).all(axis=-1) | (np.abs(ref[0]).sum(axis=-1) == 0)
    assert np.all(gpu[dead] == 0)
