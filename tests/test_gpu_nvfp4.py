"""fmha_quantize_nvfp4 on the GPU against the oracle: bit-exact codes, block
scales and token scales (every register-resident row length class and the
streaming one, ragged block counts, strided rows, zero / tiny / subnormal /
huge rows, and sampled rows of the full-size workload)."""
import numpy as np
import pytest

from fmha_fwd_amd import workloads as W
from oracle.nvfp4 import quantize_nvfp4 as oracle_nvfp4

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _gpu(x_np, row_stride=None):
    import fmha_fwd_amd as F
    M, K = x_np.shape
    rs = row_stride or K
    buf = torch.zeros((M, rs), dtype=torch.bfloat16)
    buf[:, :K] = torch.from_numpy(np.ascontiguousarray(x_np)).to(torch.bfloat16)
    x = buf.cuda()[:, :K]
    c, sf, ts = F.quantize_nvfp4(x)
    torch.cuda.synchronize()
    return c.cpu().numpy(), sf.view(torch.uint8).cpu().numpy(), ts.cpu().numpy()


def _check(x, c, sf, ts):
    rc, rsf, rts = oracle_nvfp4(x)
    assert np.array_equal(rts.view(np.uint32), ts.view(np.uint32)), \
        f"token scales differ at rows {np.nonzero(rts.view(np.uint32) != ts.view(np.uint32))[0][:8]}"
    bad = np.nonzero(rsf != sf)
    assert bad[0].size == 0, f"{bad[0].size} block scales differ, first at {tuple(i[0] for i in bad)}"
    bad = np.nonzero(rc != c)
    assert bad[0].size == 0, f"{bad[0].size} code bytes differ, first at {tuple(i[0] for i in bad)}"


def _rows(seed, M, K):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x *= np.exp(rng.uniform(-8, 8, (M, 1))).astype(np.float32)
    x[:, rng.choice(K, max(1, K // 200), replace=False)] *= 20
    return W.to_bf16_values(x)


# K/16 blocks per row: 1, 3, 64, 259 (ragged), 448, 1024 (registers, up to 16
# per lane), 1025 and 1280 (streaming)
@pytest.mark.parametrize("M,K", [(1, 16), (5, 48), (37, 1024), (6, 4144), (9, 7168), (3, 16384), (4, 16400),
                                 (2, 20480), (130, 256)])
def test_random_rows_bit_exact(M, K):
    print(f"nvfp4 M={M} K={K}", flush=True)
    x = _rows(M * 100003 + K, M, K)
    _check(x, *_gpu(x))


@pytest.mark.parametrize("K", [512, 16400])
def test_strided_rows(K):
    print(f"nvfp4 strided K={K}", flush=True)
    x = _rows(K + 7, 11, K)
    _check(x, *_gpu(x, row_stride=K + 40))


@pytest.mark.parametrize("K", [64, 2048, 17408])
def test_zero_tiny_subnormal_and_huge_rows(K):
    print(f"nvfp4 special rows K={K}", flush=True)
    x = _rows(K, 12, K)
    x[0] = 0.0                                   # zero row: ts 1, all zero
    x[1] = -0.0                                  # negative zeros keep their sign
    for r, top in ((2, 2.0 ** -130),   # below 2^-116: dead row
                   (3, 2.0 ** -115),   # ts subnormal in fp32
                   (4, 2.0 ** -100),   # block scales down to E4M3 subnormals
                   (5, 3.0e38)):       # near the top of bf16
        x[r] = (x[r].astype(np.float64) / np.abs(x[r]).max() * top).astype(np.float32)
    x[6, : K // 2] *= np.float32(2.0 ** -40)               # half the row tiny: zero block scales
    x[7, ::3] = 0.0
    x[8, 5] = np.float32(2.0 ** -133)                      # bf16 subnormal elements
    x[9] = np.float32(1.0)                                 # constant row
    x = W.to_bf16_values(x)
    _check(x, *_gpu(x))


def test_empty_matrix():
    import fmha_fwd_amd as F
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    c, sf, ts = F.quantize_nvfp4(x)
    torch.cuda.synchronize()
    assert c.shape == (0, 32) and sf.shape == (0, 4) and ts.shape == (0,)


def test_outputs_untouched_outside_rows():
    # strided outputs: bytes between rows stay as they were
    import fmha_fwd_amd as F
    x = torch.from_numpy(_rows(3, 8, 256)).to(torch.bfloat16).cuda()
    cbuf = torch.full((8, 136), 0xAB, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((8, 24), 0xCD, dtype=torch.uint8, device="cuda")
    F.quantize_nvfp4(x, codes=cbuf[:, :128], block_scales=sbuf[:, :16].view(torch.float8_e4m3fn))
    torch.cuda.synchronize()
    assert bool((cbuf[:, 128:] == 0xAB).all()) and bool((sbuf[:, 16:] == 0xCD).all())


def test_full_size_workload_sampled_rows():
    # the benchmark's matrix quantised in one launch; rows are independent,
    # so sampled rows (first, last, spread) are checked exactly
    import fmha_fwd_amd as F
    idx, M, K = W.NVFP4_SPECS["nvfp4"]
    print(f"nvfp4 full size M={M} K={K}", flush=True)
    x_all = W.nvfp4_activations(M, K, idx)
    x = torch.from_numpy(x_all).to(torch.bfloat16).cuda()
    c, sf, ts = F.quantize_nvfp4(x)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(9).choice(M, 254, replace=False)]))
    _check(x_all[rows], c.cpu().numpy()[rows], sf.view(torch.uint8).cpu().numpy()[rows], ts.cpu().numpy()[rows])


def test_binding_rejects_mismatched_outputs():
    import fmha_fwd_amd as F
    x = torch.zeros((8, 256), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        F.quantize_nvfp4(x, codes=torch.zeros((8, 64), dtype=torch.uint8, device="cuda"))
    with pytest.raises(ValueError):
        F.quantize_nvfp4(x, token_scales=torch.zeros((4,), dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):
        F.quantize_blocks(torch.zeros((1, 64, 2, 128), dtype=torch.bfloat16, device="cuda"), "e4m3",
                          scales=torch.zeros((1, 2, 2), dtype=torch.float32, device="cuda"))
