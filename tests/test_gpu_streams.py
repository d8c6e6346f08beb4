"""Stream semantics of the C ABI: work is enqueued on the caller's stream with
no host synchronisation, so the quantizer and fmha_fwd run on a side stream
and inside a captured HIP graph exactly as they do eagerly (bit for bit: the
kernels are deterministic)."""
import numpy as np
import pytest
import torch

from fmha_fwd_amd import workloads as W
import harness as Hn

pytestmark = pytest.mark.gpu


def _inputs(seed, shape):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).to(torch.bfloat16).cuda()


def _step(F, q, k, v, out, stream=None):
    qc, sq = F.quantize_blocks(q, "e4m3", stream=stream)
    kc, sk = F.quantize_blocks(k, "e4m3", stream=stream)
    vc, sv = F.quantize_blocks(v, "e4m3", stream=stream)
    F.fwd(qc, kc, vc, sfs_q=sq, sfs_k=sk, sfs_v=sv, causal=True, out=out, stream=stream)


def test_side_stream_matches_default_stream():
    import fmha_fwd_amd as F
    shape_q, shape_kv = (2, 700, 8, 128), (2, 700, 2, 128)
    q, k, v = _inputs(1, shape_q), _inputs(2, shape_kv), _inputs(3, shape_kv)
    ref = torch.empty(shape_q, dtype=torch.bfloat16, device="cuda")
    _step(F, q, k, v, ref)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()  # default priority
    out = torch.full(shape_q, 7.0, dtype=torch.bfloat16, device="cuda")
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(F, q, k, v, out, stream=side)
    # unrelated work on the default stream meanwhile
    junk = torch.randn(4096, 4096, device="cuda")
    junk = junk @ junk
    side.synchronize()
    assert torch.equal(out, ref)
    torch.cuda.synchronize()


def test_graph_replays_match_eager():
    # the quantize + forward step captured once, replayed on new inputs with
    # eager work and synchronisations in between; every replay against the
    # eager result of the same inputs (and the first against the oracle)
    import fmha_fwd_amd as F
    spec = W.small_spec("gqa", 320, B=1, Hq=4, Hkv=2, causal=True)
    data = W.generate(spec)
    q, k, v = (Hn.to_gpu_bf16(data[n]) for n in ("q", "k", "v"))
    out = torch.empty_like(q)
    eager = torch.empty_like(q)
    _step(F, q, k, v, eager)  # first launches configure the kernels outside the capture
    torch.cuda.synchronize()
    ops = Hn.oracle_operands(spec, data)
    Hn.assert_parity(eager.float().cpu().numpy(), Hn.oracle_output(spec, data, ops), what="graph eager")
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            _step(F, q, k, v, out, stream=cap)
    torch.cuda.synchronize()
    for r in range(4):
        if r:
            q.copy_(_inputs(10 + r, q.shape))
            k.copy_(_inputs(20 + r, k.shape))
            v.copy_(_inputs(30 + r, v.shape))
        out.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _step(F, q, k, v, eager)
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r}"
        assert np.isfinite(out.float().cpu().numpy()).all()
