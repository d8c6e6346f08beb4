"""fmha_fwd on the GPU against the oracle on the same seeded inputs.

Small shapes (full outputs, several tiles plus ragged tails) for every
supported format combination and option, then the full-size workloads on
sampled rows in the launch configuration the benchmark times.  Bar: max-abs
error <= 1.5e-2 against the bf16-rounded quantisation-emulating oracle (one
bf16 ulp differences counted apart), cosine >= 0.999 against it and >= 0.99
against unquantised fp64 attention."""
import numpy as np
import pytest

from fmha_fwd_amd import workloads as W
import harness as Hn

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _run_small(spec, **kw):
    print(f"fwd small {spec}", flush=True)
    data = W.generate(spec)
    gpu, _ = Hn.gpu_run(spec, data, **kw)
    ops = Hn.oracle_operands(spec, data)
    okw = {}
    if "sfs_p" in kw:
        okw["sfs_p"] = kw["sfs_p"].cpu().numpy()
    if "lazy_rescale_log2" in kw:
        okw["tau"] = kw["lazy_rescale_log2"]
    ukw = {}
    if "softmax_scale" in kw:
        okw["softmax_scale"] = ukw["softmax_scale"] = kw["softmax_scale"]
    ref = Hn.oracle_output(spec, data, ops, **okw)
    unq = Hn.unquantized_output(spec, data, **ukw)
    return Hn.assert_parity(gpu, ref, unq, what=spec.name)


@pytest.mark.parametrize("S", [1, 63, 64, 65, 255, 320])
@pytest.mark.parametrize("base", ["tiny", "dit_i8", "dit", "gqa", "gqa_vi8"])
def test_small_dense(base, S):
    B, Hq, Hkv = {"tiny": (1, 2, 2), "dit_i8": (1, 3, 3), "dit": (2, 2, 2), "gqa": (2, 8, 2), "gqa_vi8": (2, 8, 2)}[base]
    _run_small(W.small_spec(base, S, B=B, Hq=Hq, Hkv=Hkv))


@pytest.mark.parametrize("S", [1, 65, 200, 320])
@pytest.mark.parametrize("base", ["tiny", "dit", "dit_i8", "gqa_vi8"])
def test_small_causal(base, S):
    _run_small(W.small_spec(base, S, B=1, Hq=4, Hkv=2, causal=True))


@pytest.mark.parametrize("S", [64, 300, 768])
@pytest.mark.parametrize("causal", [False, True])
def test_small_sparse_paged(S, causal):
    _run_small(W.small_spec("sparse", S, B=2, Hq=4, Hkv=2, causal=causal))


@pytest.mark.parametrize("S", [256, 640])
def test_small_sparse_contiguous(S):
    _run_small(W.small_spec("sparse", S, B=1, Hq=2, Hkv=2, paged=False))


@pytest.mark.parametrize("base", ["tiny", "dit", "dit_i8", "gqa", "gqa_vi8"])
@pytest.mark.parametrize("masked,paged", [(True, False), (False, True), (True, True)])
def test_other_formats_masked_or_paged(base, masked, paged):
    # the block-sparse and paged paths for the other format combinations
    _run_small(W.small_spec(base, 300, B=2, Hq=4, Hkv=2, masked=masked, paged=paged))


def test_small_paged_dense():
    _run_small(W.small_spec("sparse", 300, B=2, Hq=2, Hkv=1, masked=False))


@pytest.mark.parametrize("page_size", [32, 64, 128, 256])
@pytest.mark.parametrize("masked", [False, True])
def test_small_paged_page_sizes(page_size, masked):
    # pages of 16..64 tokens split a 64-key sub-tile; longer ones hold several
    _run_small(W.small_spec("sparse", 300, B=2, Hq=2, Hkv=2, masked=masked, page_size=page_size))


@pytest.mark.parametrize("base", ["gqa", "dit", "dit_i8", "sparse", "tiny", "gqa_vi8"])
def test_sfs_p_and_tau_variants(base):
    spec = W.small_spec(base, 320, B=1, Hq=4, Hkv=2)
    sp = torch.tensor([1.0, 0.25, 0.1, 2.0], dtype=torch.float32, device="cuda")
    _run_small(spec, sfs_p=sp)
    _run_small(spec, lazy_rescale_log2=0.0)
    _run_small(spec, lazy_rescale_log2=12.0)


@pytest.mark.parametrize("base,D", [("tiny", 128), ("dit", 128), ("dit_i8", 128), ("gqa", 128), ("sparse", 128),
                                    ("gqa_vi8", 128), ("gqa", 192), ("dit", 192)])
@pytest.mark.parametrize("scale", [0.01, 0.3])
def test_softmax_scale_variants(base, D, scale):
    # a flatter (0.01) and a sharper (0.3) softmax than 1/sqrt(D): the
    # lazy reference moves more often and P spans more of the E4M3 range
    _run_small(W.small_spec(base, 300, B=1, Hq=4, Hkv=2, causal=True, D=D), softmax_scale=scale)


def test_masked_blocks_with_nan_are_never_read():
    import fmha_fwd_amd as F
    spec = W.small_spec("sparse", 768, B=1, Hq=2, Hkv=2, paged=False)
    data = W.generate(spec)
    bm = data["block_mask"].copy()
    bm[:, :, :, 1] = 0                      # keys 256..511 inactive for every query block
    for qb in range(bm.shape[2]):
        if not bm[0, 0, qb].any() or not bm[0, 1, qb].any():
            bm[:, :, qb, 0] = 1
    data["block_mask"] = bm
    ref_gpu, t = Hn.gpu_run(spec, data)
    k, v = t["k"].clone(), t["v"].clone()
    k.view(torch.uint8)[:, 256:512] = 0x7F  # E4M3 NaN
    v.view(torch.uint8)[:, 256:512] = 0x7F
    o = F.fwd(t["q"], k, v, sfs_k=t["sfs_k"], sfs_v=t["sfs_v"], block_mask=torch.from_numpy(bm).cuda())
    torch.cuda.synchronize()
    got = o.float().cpu().numpy()
    assert np.all(np.isfinite(got))
    assert np.array_equal(got, ref_gpu)
    ops = Hn.oracle_operands(spec, data)
    Hn.assert_parity(got, Hn.oracle_output(spec, data, ops), what="masked-nan")


def test_strided_q_and_output():
    import fmha_fwd_amd as F
    spec = W.small_spec("dit", 200, B=1, Hq=2, Hkv=2)
    data = W.generate(spec)
    qkv = torch.zeros((1, 200, 3, 2, 128), dtype=torch.bfloat16, device="cuda")
    qkv[:, :, 0] = Hn.to_gpu_bf16(data["q"])
    qkv[:, :, 1] = Hn.to_gpu_bf16(data["k"])
    v, sv = F.quantize_blocks(Hn.to_gpu_bf16(data["v"]), "e4m3")
    out = torch.zeros((1, 200, 4, 128), dtype=torch.bfloat16, device="cuda")
    F.fwd(qkv[:, :, 0], qkv[:, :, 1], v, sfs_v=sv, out=out[:, :, 1:3])
    torch.cuda.synchronize()
    got = out[:, :, 1:3].float().cpu().numpy()
    ops = Hn.oracle_operands(spec, data)
    Hn.assert_parity(got, Hn.oracle_output(spec, data, ops), what="strided")
    assert torch.count_nonzero(out[:, :, 0]) == 0 and torch.count_nonzero(out[:, :, 3]) == 0


@pytest.mark.parametrize("base", ["gqa", "dit_i8", "sparse"])
def test_fused_qkv_codes(base):
    # Q, K and V codes written by the quantizer into one fused [B, S, Hq + 2 Hkv,
    # D] buffer (the layout of a fused QKV projection) and read back through
    # head-strided views
    import fmha_fwd_amd as F
    spec = W.small_spec(base, 300, B=2, Hq=4, Hkv=2, causal=True, masked=False, paged=False)
    print(f"fwd fused qkv {spec}", flush=True)
    data = W.generate(spec)
    Hq, Hkv = spec.Hq, spec.Hkv
    fmts = (spec.q_fmt, spec.k_fmt, spec.v_fmt)
    tdt = {"int8": torch.int8, "e4m3": torch.float8_e4m3fn, "bf16": torch.bfloat16}
    # one fused buffer per code type (int8 Q/K beside an E4M3 V use two)
    bufs = {f: torch.zeros((2, 300, Hq + 2 * Hkv, 128), dtype=tdt[f], device="cuda") for f in set(fmts)}
    views = (bufs[fmts[0]][:, :, :Hq], bufs[fmts[1]][:, :, Hq:Hq + Hkv], bufs[fmts[2]][:, :, Hq + Hkv:])
    t, sc = [], []
    for name, fmt, view in zip(("q", "k", "v"), fmts, views):
        x = Hn.to_gpu_bf16(data[name])
        if fmt == "bf16":
            t.append(x)
            sc.append(None)
        else:
            c, s_ = F.quantize_blocks(x, fmt, codes=view)
            assert c.data_ptr() == view.data_ptr()
            t.append(view)
            sc.append(s_)
    o = F.fwd(t[0], t[1], t[2], sfs_q=sc[0], sfs_k=sc[1], sfs_v=sc[2], causal=True)
    torch.cuda.synchronize()
    ops = Hn.oracle_operands(spec, data)
    Hn.assert_parity(o.float().cpu().numpy(), Hn.oracle_output(spec, data, ops), Hn.unquantized_output(spec, data),
                     what=f"fused qkv {base}")


def test_kv_sequence_beyond_2gib():
    # K/V token strides of 4 MiB: each sequence spans more than 2^31 bytes,
    # so every tile gets a buffer resource of its own
    import fmha_fwd_amd as F
    spec = W.small_spec("dit", 640, B=1, Hq=2, Hkv=2)
    print(f"fwd {spec} with 4 MiB K/V token strides", flush=True)
    data = W.generate(spec)
    q = Hn.to_gpu_bf16(data["q"])
    v_codes, sv = F.quantize_blocks(Hn.to_gpu_bf16(data["v"]), "e4m3")
    stride = 1 << 22
    kbig = torch.empty(640 * stride // 2, dtype=torch.bfloat16, device="cuda")
    k = kbig.as_strided((1, 640, 2, 128), (640 * stride // 2, stride // 2, 128, 1))
    k.copy_(Hn.to_gpu_bf16(data["k"]))
    vbig = torch.empty(640 * stride, dtype=torch.uint8, device="cuda")
    v = vbig.as_strided((1, 640, 2, 128), (640 * stride, stride, 128, 1))
    v.copy_(v_codes.view(torch.uint8))
    o = F.fwd(q, k, v.view(torch.float8_e4m3fn), sfs_v=sv)
    torch.cuda.synchronize()
    ops = Hn.oracle_operands(spec, data)
    Hn.assert_parity(o.float().cpu().numpy(), Hn.oracle_output(spec, data, ops), Hn.unquantized_output(spec, data),
                     what="2 GiB K/V span")
    del kbig, vbig


@pytest.mark.parametrize("base,S,causal,D", [("tiny", 200, False, 128), ("dit", 320, False, 128),
                                             ("dit_i8", 300, False, 128), ("gqa", 300, True, 128),
                                             ("sparse", 300, False, 128), ("dit", 320, False, 192),
                                             ("gqa", 300, True, 192), ("gqa_vi8", 300, True, 128)])
def test_e4m3_output(base, S, causal, D):
    # O / sfs_o encoded to E4M3 in the epilogue; the per-head scales spread
    # the outputs over the E4M3 range (saturation and subnormals included).
    # Bar: each code is the encoding of a value within tol of the oracle's
    # O, tol = the oracle's P-rounding sensitivity bound + 2^-13 (max|V| +
    # |O|) (the accumulation error of O, whose elements can be small
    # differences of much larger terms; a hundred times tighter than the
    # 1.5e-2 bar of the bf16 output), and at most 1 % of the codes differ
    # from the oracle's own encoding.
    from oracle.attention import output_e4m3
    from oracle.codecs import e4m3_decode
    spec = W.small_spec(base, S, B=1, Hq=4, Hkv=2, causal=causal, D=D)
    print(f"fwd e4m3 output {spec}", flush=True)
    data = W.generate(spec)
    so = np.array([2.0 ** -11, 0.004, 0.02, 1.0], dtype=np.float32)
    _, t = Hn.gpu_run(spec, data, out_dtype="e4m3", sfs_o=torch.from_numpy(so).cuda())
    codes = t["o"].view(torch.uint8).cpu().numpy()
    ops = Hn.oracle_operands(spec, data)
    ref, bound = Hn.oracle_output(spec, data, ops)
    vmax = np.abs(ops[2]).max(axis=(0, 1, 3))[np.arange(4) // 2][None, None, :, None]
    tol = bound + 2.0 ** -13 * (vmax + np.abs(ref))
    got = e4m3_decode(codes)
    lo, hi = e4m3_decode(output_e4m3(ref - tol, so)), e4m3_decode(output_e4m3(ref + tol, so))
    ok = (got >= lo) & (got <= hi)
    bad = [(tuple(i), float(ref[tuple(i)]), float(tol[tuple(i)]), float(got[tuple(i)] * so[i[2]]))
           for i in np.argwhere(~ok)[:5]]
    assert ok.all(), f"{int((~ok).sum())} codes outside the tolerance: (index, O, tol, decoded * so) {bad}"
    want = output_e4m3(ref, so)
    n_diff = int((e4m3_decode(want) != got).sum())
    assert n_diff <= 0.01 * codes.size
    assert (codes == 0x7E).any() and (((codes & 0x7F) > 0) & ((codes & 0x7F) < 8)).any()  # saturation, subnormals
    print(f"e4m3 output {spec.name}: {n_diff} of {codes.size} codes differ from the oracle's encoding")


@pytest.mark.parametrize("base,skv", [("dit", 100), ("gqa", 70), ("dit_i8", 1), ("gqa_vi8", 130)])
@pytest.mark.parametrize("causal", [False, True])
def test_more_queries_than_keys(base, skv, causal):
    # Sq = 300 queries against fewer keys; bottom-right causal leaves the
    # first Sq - Skv rows without a valid key (zero rows)
    spec = W.small_spec(base, 300, B=1, Hq=4, Hkv=2, causal=causal)
    print(f"fwd {spec} with Skv={skv}", flush=True)
    data = W.generate(spec)
    data["k"], data["v"] = data["k"][:, :skv], data["v"][:, :skv]
    gpu, _ = Hn.gpu_run(spec, data)
    ops = Hn.oracle_operands(spec, data)
    Hn.assert_parity(gpu, Hn.oracle_output(spec, data, ops), Hn.unquantized_output(spec, data), what=f"Skv={skv}")
    if causal:
        assert np.all(gpu[:, :300 - skv] == 0)


def test_no_keys_gives_zero_rows():
    import fmha_fwd_amd as F
    spec = W.small_spec("gqa", 130, B=1, Hq=4, Hkv=2)
    data = W.generate(spec)
    q, sq = F.quantize_blocks(Hn.to_gpu_bf16(data["q"]), "e4m3")
    k = torch.zeros((1, 0, 2, 128), dtype=torch.float8_e4m3fn, device="cuda")
    sk = torch.zeros((1, 2, 0), dtype=torch.float32, device="cuda")
    o = torch.full((1, 130, 4, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    F.fwd(q, k, k, sfs_q=sq, sfs_k=sk, sfs_v=sk, out=o)
    torch.cuda.synchronize()
    assert torch.count_nonzero(o) == 0


def test_paged_pool_beyond_4gib():
    # pages 256 MiB apart: the pool spans more than 2^32 bytes, so the copies
    # take 64-bit page addresses instead of 32-bit offsets from the pool base
    import fmha_fwd_amd as F
    spec = W.small_spec("sparse", 300, B=1, Hq=2, Hkv=2)
    print(f"fwd {spec} with a pool of 256 MiB page stride", flush=True)
    data = W.generate(spec)
    pt = data["page_table"]                       # [1, 19] pool pages 0..18
    n_pages, ps = pt.size, spec.page_size
    q = Hn.to_gpu_bf16(data["q"])
    kc, sk = F.quantize_blocks(Hn.to_gpu_bf16(data["k"]), "e4m3")
    vc, sv = F.quantize_blocks(Hn.to_gpu_bf16(data["v"]), "e4m3")
    stride = 1 << 28
    assert n_pages * stride >= 1 << 32
    pools = []
    for codes in (kc, vc):
        big = torch.empty(n_pages * stride, dtype=torch.uint8, device="cuda")
        pool = big.as_strided((n_pages, ps, 2, 128), (stride, 256, 128, 1))
        padded = torch.zeros((n_pages * ps, 2, 128), dtype=torch.uint8, device="cuda")
        padded[:300] = codes.view(torch.uint8)[0]
        pool[torch.from_numpy(pt.reshape(-1)).long().cuda()] = padded.view(n_pages, ps, 2, 128)
        pools.append((big, pool.view(torch.float8_e4m3fn)))
    o = F.fwd(q, pools[0][1], pools[1][1], sfs_k=sk, sfs_v=sv, block_mask=torch.from_numpy(data["block_mask"]).cuda(),
              page_table=torch.from_numpy(pt).cuda(), page_size=ps, seq_len_kv=300)
    torch.cuda.synchronize()
    ops = Hn.oracle_operands(spec, data)
    Hn.assert_parity(o.float().cpu().numpy(), Hn.oracle_output(spec, data, ops), Hn.unquantized_output(spec, data),
                     what="pool beyond 4 GiB")
    del pools


@pytest.mark.parametrize("paged", [False, True])
def test_block_mask_broadcast_over_batch_and_heads(paged):
    # one [q_blocks, kv_blocks] mask expanded to [B, Hq, ...] (strides 0)
    spec = W.small_spec("sparse", 700, B=2, Hq=4, Hkv=2, paged=paged)
    print(f"fwd {spec} with a broadcast mask", flush=True)
    data = W.generate(spec)
    one = data["block_mask"][0, 0]
    data["block_mask"] = np.broadcast_to(one, data["block_mask"].shape).copy()
    mask = torch.from_numpy(one.copy()).cuda().expand(2, 4, *one.shape)
    assert mask.stride(0) == 0 and mask.stride(1) == 0
    gpu, _ = Hn.gpu_run(spec, data, block_mask=mask)
    ops = Hn.oracle_operands(spec, data)
    Hn.assert_parity(gpu, Hn.oracle_output(spec, data, ops), Hn.unquantized_output(spec, data), what="broadcast mask")


def test_no_valid_key_rows_are_zero():
    import fmha_fwd_amd as F
    spec = W.small_spec("sparse", 256, B=1, Hq=1, Hkv=1, paged=False)
    data = W.generate(spec)
    data["block_mask"][:, :, 2, :] = 0  # query block 2 sees nothing
    gpu, _ = Hn.gpu_run(spec, data)
    assert np.all(gpu[0, 128:192] == 0) and np.all(np.abs(gpu[0, :128]).sum(-1) > 0)


@pytest.mark.parametrize("block_kv,S,paged,causal", [(64, 4500, False, False), (192, 1000, True, False),
                                                     (512, 1500, False, True), (64, 4200, True, True)])
def test_mask_key_block_sizes(block_kv, S, paged, causal):
    # key blocks of 1, 3 and 8 sub-tiles; more than 64 key blocks per query
    # block; query blocks 1 and the last with no active key block
    spec = W.small_spec("sparse", S, B=1, Hq=2, Hkv=1, paged=paged, causal=causal)
    print(f"fwd mask blocks {spec} block_kv={block_kv}", flush=True)
    data = W.generate(spec)
    nqb = -(-S // 64)
    data["block_mask"] = W.random_block_mask(1, 2, S, S, block_kv, 0.3, stream=block_kv + S,
                                             empty_q_blocks=(1, nqb - 1))
    gpu, _ = Hn.gpu_run(spec, data, mask_block=(64, block_kv))
    rows = _sample_rows(S)
    rows = np.union1d(rows, np.arange(64, 128))
    ops = Hn.oracle_operands(spec, data)
    ref = Hn.oracle_output(spec, data, ops, rows=rows, mask_block_kv=block_kv)
    unq = Hn.unquantized_output(spec, data, rows=rows, mask_block_kv=block_kv)
    g = gpu[:, rows]
    assert np.all(g[:, np.isin(rows, np.arange(64, 128))] == 0)
    assert np.all(g[:, rows >= (nqb - 1) * 64] == 0)
    Hn.assert_parity(g, ref, unq, what=f"mask blocks {block_kv}")


@pytest.mark.parametrize("sq,S", [(1, 300), (32, 300), (40, 511), (96, 700)])
@pytest.mark.parametrize("causal", [False, True])
def test_query_chunk_gqa(sq, S, causal):
    # fewer queries than keys (a prefill chunk, bottom-right causal); with four
    # query heads per KV head the kernel packs heads into one workgroup
    _run_small(W.small_spec("gqa", S, B=1, Hq=8, Hkv=2, causal=causal, sq=sq))


@pytest.mark.parametrize("base", ["gqa", "dit", "dit_i8", "tiny", "sparse", "gqa_vi8"])
@pytest.mark.parametrize("hq,sq", [(16, 1), (16, 5), (16, 16), (32, 3), (32, 8), (64, 1), (64, 4)])
@pytest.mark.parametrize("causal", [False, True])
def test_rows_of_several_heads_per_wave(base, hq, sq, causal):
    # query chunks shorter than 16 with 8, 16 or 32 query heads per KV head:
    # a wave's 32 rows hold 2, 4 or 8 heads (16, 8 or 4 rows each)
    _run_small(W.small_spec(base, 300, B=2, Hq=hq, Hkv=2, causal=causal, sq=sq, masked=False))


@pytest.mark.parametrize("base", ["gqa", "dit", "dit_i8", "tiny", "sparse"])
@pytest.mark.parametrize("hq,sq", [(16, 1), (16, 5), (32, 3)])
def test_short_query_ranges_at_head_dim_192(base, hq, sq):
    # at d = 192 short query ranges of large groups fall back to whole-wave
    # head packing (no heads inside a wave)
    _run_small(W.small_spec(base, 300, B=2, Hq=hq, Hkv=2, causal=True, sq=sq, masked=False, D=192))


@pytest.mark.parametrize("base", ["gqa", "dit_i8", "sparse", "gqa_vi8"])
@pytest.mark.parametrize("sq", [1, 7, 16])
@pytest.mark.parametrize("causal", [False, True])
def test_rows_of_two_heads_in_two_wave_workgroups(base, sq, causal):
    # four query heads per KV head: two-wave workgroups of two heads per wave
    # (8-bit K formats)
    _run_small(W.small_spec(base, 300, B=2, Hq=8, Hkv=2, causal=causal, sq=sq, masked=False))


@pytest.mark.parametrize("sq,S", [(1, 300), (40, 511), (96, 700)])
@pytest.mark.parametrize("causal", [False, True])
def test_query_chunk_int8_v(sq, S, causal):
    # the K-fp8 / V-int8 combination on a prefill chunk of a GQA group
    _run_small(W.small_spec("gqa_vi8", S, B=1, Hq=8, Hkv=2, causal=causal, sq=sq))


@pytest.mark.parametrize("S", [1, 130, 320])
def test_small_causal_gqa_packed(S):
    _run_small(W.small_spec("gqa", S, B=2, Hq=8, Hkv=2, causal=True))


@pytest.mark.parametrize("base,B,Hq,Hkv,causal,sq", [("dit_i8", 1, 3, 3, False, 0), ("gqa", 2, 8, 2, True, 0),
                                                      ("gqa", 1, 4, 2, False, 0), ("gqa", 2, 8, 2, True, 100),
                                                      ("dit_i8", 2, 2, 1, True, 0), ("dit", 1, 2, 2, False, 0),
                                                      ("dit", 2, 4, 2, True, 0), ("gqa", 2, 16, 2, True, 5),
                                                      ("dit", 1, 16, 2, False, 3), ("tiny", 1, 2, 2, False, 0),
                                                      ("tiny", 2, 4, 2, True, 0)])
@pytest.mark.parametrize("S", [1, 65, 320, 1000])
def test_head_dim_192(base, B, Hq, Hkv, causal, sq, S):
    # head dim 192 with 8-bit Q and K, bf16 Q and K with E4M3 V, or all bf16:
    # dense, causal, GQA (whole-wave head packing for the causal groups), a
    # query chunk, ragged tails
    if sq >= S:
        sq = 0
    _run_small(W.small_spec(base, S, B=B, Hq=Hq, Hkv=Hkv, causal=causal, sq=sq, D=192))


@pytest.mark.parametrize("base", ["dit", "gqa", "dit_i8", "sparse", "gqa_vi8"])
@pytest.mark.parametrize("causal", [False, True])
def test_v_block_scales_spanning_more_than_2_64(base, causal):
    # V block scales more than 2^64 apart: the kernel then keeps O in fixed
    # units and adds every sub-tile's product with its own scale (the slow
    # V-reference path).  Block 1 of V is scaled by 2^-70 before quantisation
    # (exact: the codes stay the same, the block scale moves by 2^-70) and
    # block 3 by 4.
    spec = W.small_spec(base, 320, B=1, Hq=4, Hkv=2, causal=causal)
    print(f"fwd {spec} with V block scales spanning 2^72", flush=True)
    data = W.generate(spec)
    v = data["v"].copy()
    v[:, 64:128] *= np.float32(2.0 ** -70)
    v[:, 192:256] *= np.float32(4.0)
    data["v"] = v
    gpu, t = Hn.gpu_run(spec, data)
    sv = t["sfs_v"].cpu().numpy()
    assert sv.max() > sv.min() * 2.0 ** 64
    ops = Hn.oracle_operands(spec, data)
    Hn.assert_parity(gpu, Hn.oracle_output(spec, data, ops), Hn.unquantized_output(spec, data),
                     what=f"V scales beyond 2^64 {base}")


@pytest.mark.parametrize("S,causal", [(1, False), (320, False), (300, True), (1000, False)])
def test_unscaled_e4m3_v(S, causal):
    # bf16 Q and K with E4M3 V codes and no V scale (sage_block_v = 0): V is
    # encoded directly (nearest-even, saturating) and read as its E4M3 values
    import fmha_fwd_amd as F
    from oracle.codecs import e4m3_decode, e4m3_encode
    from oracle.attention import attention
    spec = W.small_spec("dit", S, B=2, Hq=4, Hkv=2, causal=causal)
    print(f"fwd {spec} with an unscaled E4M3 V", flush=True)
    data = W.generate(spec)
    vcodes = e4m3_encode(data["v"].astype(np.float64) * 3.0)  # values up to ~15: normals and subnormals
    q, k = Hn.to_gpu_bf16(data["q"]), Hn.to_gpu_bf16(data["k"])
    v = torch.from_numpy(vcodes).cuda().view(torch.float8_e4m3fn)
    o = F.fwd(q, k, v, causal=causal)
    torch.cuda.synchronize()
    gpu = o.float().cpu().numpy()
    qd, kd, vd = (data["q"].astype(np.float64), data["k"].astype(np.float64), e4m3_decode(vcodes))
    ref = attention(qd, kd, vd, causal=causal, mode="lazy", p_format="e4m3", flip_eps=Hn.FLIP_EPS)
    unq = attention(qd, kd, vd, causal=causal, mode="exact", p_format=None)
    Hn.assert_parity(gpu, ref, unq, what=f"unscaled e4m3 V S={S}")


@pytest.mark.parametrize("base", ["sparse", "tiny", "dit", "dit_i8", "gqa"])
@pytest.mark.parametrize("masked,paged", [(True, False), (False, True), (True, True)])
@pytest.mark.parametrize("S,causal", [(300, False), (700, True)])
def test_head_dim_192_masked_or_paged(base, masked, paged, S, causal):
    # head dim 192 with a block mask and/or paged K/V for every format, incl.
    # bf16 Q x E4M3 K (the block-sparse format, also dense)
    _run_small(W.small_spec(base, S, B=2, Hq=4, Hkv=2, masked=masked, paged=paged, causal=causal, D=192))


@pytest.mark.parametrize("S,causal", [(1, False), (130, True), (1000, False)])
def test_head_dim_192_bf16_q_e4m3_k_dense(S, causal):
    _run_small(W.small_spec("sparse", S, B=1, Hq=4, Hkv=2, masked=False, paged=False, causal=causal, D=192))


def test_deterministic():
    spec = W.small_spec("gqa", 700, B=1, Hq=8, Hkv=2, causal=True)
    data = W.generate(spec)
    a, _ = Hn.gpu_run(spec, data)
    b, _ = Hn.gpu_run(spec, data)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


# ---------------------------------------------------------------- full sizes
FULL = [
    # name, heads (b, hq) checked, rows sampled
    ("tiny", None, None),
    ("dit_i8", [(0, 0), (0, 11), (0, 23)], "sample"),
    ("dit", [(0, 0), (0, 39)], "sample"),
    ("gqa", [(0, 0), (0, 7), (1, 63)], "sample"),
    ("sparse", [(0, 0), (3, 31)], "sample"),
    ("gqa_chunk", [(0, 0), (1, 63)], None),
    ("dit_i8_d192", [(0, 0), (0, 23)], "sample"),
    ("gqa_d192", [(0, 0), (1, 63)], "sample"),
    ("dit_d192", [(0, 0), (0, 39)], "sample"),
    ("sparse_d192", [(0, 0), (3, 31)], "sample"),
    ("sparse_contig", [(1, 5), (2, 17)], "sample"),
    ("sparse_dense", [(0, 3), (3, 30)], "sample"),
    ("gqa_vi8", [(0, 0), (1, 63)], "sample"),
]


def _sample_rows(S, n=48, seed=0):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(S, size=min(n, S), replace=False).tolist())
    rows.update([0, 1, 63, 64, S - 1, S - 2, max(S - 57, 0)])
    return np.array(sorted(r for r in rows if 0 <= r < S))


@pytest.mark.parametrize("name,heads,rows", FULL)
def test_full_workload_sampled_rows(name, heads, rows, workload_cache):
    spec = W.SPECS[name]
    print(f"fwd full {name}", flush=True)
    data = workload_cache(name)
    gpu, _ = Hn.gpu_run(spec, data)
    r = None if rows is None else _sample_rows(spec.n_q)
    hq_list = None if heads is None else sorted({h for _, h in heads})
    hk_list = None if heads is None else sorted({h // (spec.Hq // spec.Hkv) for h in hq_list})
    ops = Hn.oracle_operands(spec, data, heads_q=hq_list, heads_kv=hk_list)
    ref = Hn.oracle_output(spec, data, ops, rows=r, heads=heads)
    unq = Hn.unquantized_output(spec, data, rows=r, heads=heads)
    g = gpu if r is None else gpu[:, r]
    if heads is None:
        Hn.assert_parity(g, ref, unq, what=name)
    else:
        for b, h in heads:
            Hn.assert_parity(g[b, :, h], (ref[0][b, :, h], ref[1][b, :, h]), unq[b, :, h], what=f"{name} b={b} h={h}")


def test_binding_rejects_mismatched_shapes():
    # every extent the kernels index with is checked before the launch
    import fmha_fwd_amd as F
    dev = "cuda"
    q = torch.zeros((1, 64, 4, 128), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((1, 64, 2, 128), dtype=torch.bfloat16, device=dev)
    kq = torch.zeros((1, 64, 2, 128), dtype=torch.float8_e4m3fn, device=dev)
    sv = torch.ones((1, 2, 1), dtype=torch.float32, device=dev)
    bad = [
        dict(k=torch.zeros((1, 64, 2, 192), dtype=torch.bfloat16, device=dev)),     # head dim differs
        dict(v=torch.zeros((1, 32, 2, 128), dtype=torch.float8_e4m3fn, device=dev)),  # v shorter than k
        dict(out=torch.zeros((1, 64, 4, 64), dtype=torch.bfloat16, device=dev)),
        dict(sfs_v=torch.ones((1, 2, 2), dtype=torch.float32, device=dev)),
        dict(sfs_p=torch.ones((2,), dtype=torch.float32, device=dev)),
        dict(block_mask=torch.ones((1, 4, 1, 2), dtype=torch.uint8, device=dev)),
    ]
    for kw in bad:
        args = dict(k=k, v=kq, sfs_v=sv)
        args.update(kw)
        with pytest.raises(ValueError):
            F.fwd(q, args.pop("k"), args.pop("v"), **args)
    pt = torch.zeros((1, 3), dtype=torch.int32, device=dev)
    pool = torch.zeros((8, 16, 2, 128), dtype=torch.float8_e4m3fn, device=dev)
    with pytest.raises(ValueError):  # 3 pages of 16 tokens cannot hold 64 keys
        F.fwd(q, pool, pool, sfs_k=sv, sfs_v=sv, page_table=pt, seq_len_kv=64)
