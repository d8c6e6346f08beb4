"""fmha_quantize_blocks on the GPU against the oracle: bit-exact codes and
scales (random, ragged tail, zero / tiny blocks, outliers, strided views, and
the full-size workloads)."""
import numpy as np
import pytest

from fmha_fwd_amd import workloads as W
from oracle.quantize import quantize_blocks as oracle_quantize

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _gpu_quant(x_np, fmt, view=None):
    import fmha_fwd_amd as F
    x = torch.from_numpy(np.ascontiguousarray(x_np)).to(torch.bfloat16).cuda()
    if view is not None:
        x = view(x)
    codes, scales = F.quantize_blocks(x, fmt)
    torch.cuda.synchronize()
    c = codes.view(torch.int8 if fmt == "int8" else torch.uint8).cpu().numpy()
    return x, c, scales.cpu().numpy()


def _bf16(x):
    return W.to_bf16_values(x)


def _check(x_vals, fmt, c, s):
    rc, rs = oracle_quantize(x_vals, fmt)
    assert np.array_equal(rs.view(np.uint32), s.view(np.uint32)), "scales differ"
    bad = np.nonzero(rc != c)
    assert bad[0].size == 0, f"{bad[0].size} codes differ, first at {tuple(i[0] for i in bad)}"


@pytest.mark.parametrize("fmt", ["int8", "e4m3"])
@pytest.mark.parametrize("shape", [(1, 130, 3, 128), (2, 64, 2, 128), (1, 1, 1, 128), (1, 32760, 1, 128), (3, 257, 5, 128)])
def test_random_blocks_bit_exact(fmt, shape):
    print(f"quantize {fmt} {shape}", flush=True)
    rng = np.random.default_rng(hash(shape) % 2 ** 32)
    x = rng.standard_normal(shape).astype(np.float32)
    x *= np.exp(rng.uniform(-6, 6, (shape[0], 1, shape[2], 1))).astype(np.float32)
    x = _bf16(x)
    _, c, s = _gpu_quant(x, fmt)
    _check(x, fmt, c, s)


@pytest.mark.parametrize("fmt", ["int8", "e4m3"])
def test_zero_tiny_and_outlier_blocks(fmt):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((1, 320, 2, 128)).astype(np.float32)
    x[0, 0:64] = 0.0                       # all-zero block
    x[0, 64:128] = np.float32(2.0 ** -130)   # below 2^-126: scale 1, codes 0
    x[0, 128:192, 0, 5] *= 1000.0          # outlier channel
    x[0, 192:256] *= np.float32(2.0 ** -120)   # small but normal scales
    x[0, 256:320] *= np.float32(2.0 ** 100)
    x = _bf16(x)
    _, c, s = _gpu_quant(x, fmt)
    _check(x, fmt, c, s)


@pytest.mark.parametrize("fmt", ["int8", "e4m3"])
def test_strided_views(fmt):
    import fmha_fwd_amd as F
    rng = np.random.default_rng(6)
    big = _bf16(rng.standard_normal((2, 100, 6, 128)).astype(np.float32))
    xg = torch.from_numpy(big).to(torch.bfloat16).cuda()[:, :, 1:4]          # head-strided view
    out = torch.zeros((2, 100, 8, 128), dtype=torch.int8 if fmt == "int8" else torch.float8_e4m3fn, device="cuda")
    codes_view = out[:, :, 2:5]
    F.quantize_blocks(xg, fmt, codes=codes_view)
    _, scales = F.quantize_blocks(xg, fmt)
    torch.cuda.synchronize()
    c = codes_view.contiguous().view(torch.int8 if fmt == "int8" else torch.uint8).cpu().numpy()
    _check(big[:, :, 1:4], fmt, c, scales.cpu().numpy())
    assert torch.count_nonzero(out[:, :, :2].view(torch.uint8)) == 0


@pytest.mark.parametrize("name,which,heads", [
    ("dit_i8", "q", None), ("dit_i8", "k", None), ("dit_i8", "v", None),
    ("dit", "v", [0, 17, 39]),
    ("gqa", "q", [0, 63]), ("gqa", "k", None), ("gqa", "v", [3]),
    ("sparse", "k", [0, 31]), ("sparse", "v", [5]),
])
def test_full_workloads_bit_exact(name, which, heads, workload_cache):
    spec = W.SPECS[name]
    print(f"quantize full {name}.{which} heads={heads}", flush=True)
    data = workload_cache(name)
    fmt = getattr(spec, which + "_fmt")
    x = data[which]
    _, c, s = _gpu_quant(x, fmt)
    if heads is not None:
        x, c, s = x[:, :, heads], c[:, :, heads], s[:, heads]
    _check(x, fmt, c, s)


@pytest.mark.parametrize("fmt", ["int8", "e4m3"])
@pytest.mark.parametrize("shape", [(1, 130, 3, 192), (2, 64, 2, 192), (1, 1, 1, 192), (3, 257, 5, 192)])
def test_head_dim_192_bit_exact(fmt, shape):
    print(f"quantize {fmt} {shape}", flush=True)
    rng = np.random.default_rng(hash(shape) % 2 ** 32)
    x = rng.standard_normal(shape).astype(np.float32)
    x *= np.exp(rng.uniform(-6, 6, (shape[0], 1, shape[2], 1))).astype(np.float32)
    x[0, :min(64, shape[1]), 0] = 0.0          # a zero block
    x = _bf16(x)
    _, c, s = _gpu_quant(x, fmt)
    _check(x, fmt, c, s)


@pytest.mark.parametrize("fmt", ["int8", "e4m3"])
@pytest.mark.parametrize("d", [128, 192])
def test_dead_blocks_with_negative_zeros_and_subnormals(fmt, d):
    """A block whose amax is below 2^-126 takes scale 1 and code 0x00 for
    every element, also for -0.0 and negative subnormals (whose sign an E4M3
    encoding of x * 0 would keep as 0x80)."""
    print(f"quantize dead blocks {fmt} d{d}", flush=True)
    rng = np.random.default_rng(11 + d)
    x = rng.standard_normal((1, 256 + 37, 2, d)).astype(np.float32)
    x[0, 0:64] = -0.0                                                      # all negative zeros
    x[0, 64:128] = np.where(rng.random((64, 2, d)) < 0.5, -0.0, 0.0)       # mixed signed zeros
    tiny = np.float32(2.0 ** -130) * rng.integers(1, 8, (64, 2, d)).astype(np.float32)
    x[0, 128:192] = np.where(rng.random((64, 2, d)) < 0.5, -tiny, tiny)    # signed bf16 subnormals
    x[0, 192:256] = -np.float32(2.0 ** -133)                               # the smallest negative subnormal
    x[0, 256:] = np.where(rng.random((37, 2, d)) < 0.5, -0.0, np.float32(-2.0 ** -127))  # dead ragged tail
    x = _bf16(x)
    assert np.signbit(x[0, 0:64]).all() and (x[0, 128:192] < 0).any()
    _, c, s = _gpu_quant(x, fmt)
    _check(x, fmt, c, s)
    assert not c.view(np.uint8).any(), "dead blocks must hold code 0x00 only"
    assert (s == 1.0).all()


@pytest.mark.parametrize("D", [128, 192])
def test_batch_matches_single_calls_and_oracle(D):
    # one launch for up to eight tensors of mixed formats and shapes (a GQA
    # Q / K / V set, a head-strided view, ragged tails, a dead block with
    # negative zeros): bit-identical to one call per tensor and to the oracle
    import fmha_fwd_amd as F
    rng = np.random.default_rng(31 + D)
    shapes = [(1, 300, 8, D), (1, 1000, 2, D), (1, 1000, 2, D), (2, 65, 3, D), (1, 1, 1, D), (3, 129, 2, D),
              (1, 64, 4, D), (2, 200, 1, D)]
    fmts = ["int8", "int8", "e4m3", "e4m3", "int8", "e4m3", "e4m3", "int8"]
    xs = []
    for i, sh in enumerate(shapes):
        x = rng.standard_normal(sh).astype(np.float32) * np.float32(np.exp(rng.uniform(-4, 4)))
        if i == 3:
            x[0, 0:64, 1] = -0.0  # a dead block of negative zeros
        xs.append(_bf16(x))
    gx = [torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).cuda() for x in xs]
    big = torch.zeros((1, 1000, 5, D), dtype=torch.bfloat16, device="cuda")  # job 1 read through a strided view
    big[:, :, 3:5] = gx[1]
    gx[1] = big[:, :, 3:5]
    print(f"quantize batch D={D}: {len(shapes)} jobs", flush=True)
    out = F.quantize_blocks_batch([(x, f) for x, f in zip(gx, fmts)])
    single = [F.quantize_blocks(x, f) for x, f in zip(gx, fmts)]
    torch.cuda.synchronize()
    for i, ((c, s), (c1, s1), x, f) in enumerate(zip(out, single, xs, fmts)):
        assert torch.equal(c.view(torch.uint8), c1.view(torch.uint8)), f"job {i}: codes differ from a single call"
        assert torch.equal(s.view(torch.int32), s1.view(torch.int32)), f"job {i}: scales differ from a single call"
        _check(x, f, c.view(torch.int8 if f == "int8" else torch.uint8).cpu().numpy(), s.cpu().numpy())


def test_batch_of_one_and_empty_jobs():
    import fmha_fwd_amd as F
    x = torch.randn((1, 130, 2, 128)).to(torch.bfloat16).cuda()
    e = torch.zeros((1, 0, 2, 128), dtype=torch.bfloat16, device="cuda")
    (c, s), (ce, se) = F.quantize_blocks_batch([(x, "e4m3"), (e, "int8")])
    c1, s1 = F.quantize_blocks(x, "e4m3")
    torch.cuda.synchronize()
    assert torch.equal(c.view(torch.uint8), c1.view(torch.uint8)) and torch.equal(s, s1)
    assert ce.numel() == 0 and se.numel() == 0
    assert F.quantize_blocks_batch([]) == []
