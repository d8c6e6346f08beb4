"""The C-ABI library without a GPU: it loads, exports every declared entry
point, agrees with the header on struct layout, and rejects bad arguments
before any HIP call."""
import ctypes
import os
import re
import subprocess

import pytest

import fmha_fwd_amd as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fmha.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(F.LIB_PATH):
        pytest.skip("libfmha.so not built")
    return F.lib_handle()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[a-z_0-9 \*]+?\b(fmha_[a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    assert set(declared_functions()) == set(F.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", F.LIB_PATH], capture_output=True, text=True, check=True).stdout
    syms = {l.split()[-1] for l in out.splitlines() if l.strip()}
    for name in declared_functions():
        assert name in syms, name
        assert getattr(lib, name) is not None
    assert lib.fmha_abi_version() == 0x000400


def test_struct_layout_matches_header(tmp_path):
    fields = [f for f, _ in F.FmhaFwdParams._fields_]
    src = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{HEADER}"', "int main(void){",
           'printf("%zu %zu\\n", sizeof(fmha_fwd_params), sizeof(fmha_tensor));']
    src += [f'printf("%zu\\n", offsetof(fmha_fwd_params, {f}));' for f in fields]
    src += [f'printf("%zu\\n", offsetof(fmha_tensor, {f}));' for f, _ in F.FmhaTensor._fields_]
    src.append("return 0;}")
    c = tmp_path / "layout.c"
    c.write_text("\n".join(src))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", str(c), "-o", str(exe)], check=True)
    vals = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(F.FmhaFwdParams) and vals[1] == ctypes.sizeof(F.FmhaTensor)
    offs = vals[2:2 + len(fields)]
    assert offs == [getattr(F.FmhaFwdParams, f).offset for f in fields]
    toffs = vals[2 + len(fields):]
    assert toffs == [getattr(F.FmhaTensor, f).offset for f, _ in F.FmhaTensor._fields_]


FAKE = 0x10000  # a 16-byte aligned address that validation never dereferences


def _tensor(dtype, sb=128 * 64 * 4, ss=128 * 4, sh=128, ptr=FAKE):
    return F.FmhaTensor(ptr, dtype, sb, ss, sh)


def _params(**kw):
    p = F.FmhaFwdParams()
    p.struct_size = ctypes.sizeof(F.FmhaFwdParams)
    p.B, p.Sq, p.Skv, p.Hq, p.Hkv, p.D = 1, 64, 64, 4, 4, 128
    p.q = _tensor(F.FMHA_DT_BF16)
    p.k = _tensor(F.FMHA_DT_BF16)
    p.v = _tensor(F.FMHA_DT_E4M3)
    p.o = _tensor(F.FMHA_DT_BF16)
    p.sfs_v = FAKE
    p.sage_block_v = 64
    p.lazy_rescale_log2 = 8.0
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def _call(lib, p):
    return lib.fmha_fwd(ctypes.byref(p), None), lib.fmha_last_error().decode()


@pytest.mark.parametrize("kw,code,msg", [
    (dict(D=64), F.FMHA_ERR_UNSUPPORTED, "D=64"),
    (dict(D=192, sfs_v=None, sage_block_v=0), F.FMHA_ERR_UNSUPPORTED,
     "with D=192 the first five except"),                          # bf16/bf16/e4m3 without V scale at 192
    (dict(D=192, q=_tensor(F.FMHA_DT_E4M3), k=_tensor(F.FMHA_DT_E4M3), sfs_k=FAKE, sage_block_k=64,
          block_mask=FAKE, mask_block_q=64, mask_block_kv=256), F.FMHA_ERR_UNSUPPORTED, "no kernel"),  # unscaled E4M3 Q
    (dict(Hq=6, Hkv=4), F.FMHA_ERR_INVALID, "multiple"),
    (dict(Hkv=0), F.FMHA_ERR_INVALID, "Hkv"),
    (dict(Sq=-1), F.FMHA_ERR_INVALID, "negative"),
    (dict(struct_size=8), F.FMHA_ERR_INVALID, "struct_size"),
    (dict(q=_tensor(F.FMHA_DT_BF16, ptr=FAKE + 8)), F.FMHA_ERR_INVALID, "aligned"),
    (dict(q=_tensor(F.FMHA_DT_BF16, ptr=0)), F.FMHA_ERR_INVALID, "null"),
    (dict(k=_tensor(F.FMHA_DT_BF16, ss=100)), F.FMHA_ERR_INVALID, "stride_s"),
    (dict(k=_tensor(F.FMHA_DT_BF16, ss=0)), F.FMHA_ERR_INVALID, "below one token row"),    # broadcast K
    (dict(v=_tensor(F.FMHA_DT_E4M3, ss=0)), F.FMHA_ERR_INVALID, "below one token row"),    # broadcast V
    (dict(k=_tensor(F.FMHA_DT_BF16, ss=64)), F.FMHA_ERR_INVALID, "below one token row"),   # rows overlap
    (dict(v=_tensor(F.FMHA_DT_E4M3, ss=112)), F.FMHA_ERR_INVALID, "below one token row"),
    (dict(page_table=FAKE, page_size=16, num_pages=4, v=_tensor(F.FMHA_DT_E4M3, ss=16)), F.FMHA_ERR_INVALID,
     "below one token row"),                                                               # paged slots overlap
    (dict(o=_tensor(F.FMHA_DT_INT8)), F.FMHA_ERR_UNSUPPORTED, "bf16 or e4m3"),
    (dict(sfs_o=FAKE), F.FMHA_ERR_INVALID, "sfs_o given"),
    (dict(o=_tensor(F.FMHA_DT_E4M3), sfs_o=FAKE + 2), F.FMHA_ERR_INVALID, "sfs_o misaligned"),
    (dict(v=_tensor(F.FMHA_DT_INT8, ss=128)), F.FMHA_ERR_UNSUPPORTED, "no kernel"),            # int8 V, bf16 Q/K
    (dict(D=192, q=_tensor(F.FMHA_DT_E4M3), k=_tensor(F.FMHA_DT_E4M3), v=_tensor(F.FMHA_DT_INT8, ss=192),
          sfs_q=FAKE, sage_block_q=64, sfs_k=FAKE, sage_block_k=64), F.FMHA_ERR_UNSUPPORTED, "no kernel"),
    (dict(q=_tensor(F.FMHA_DT_E4M3), k=_tensor(F.FMHA_DT_E4M3), v=_tensor(F.FMHA_DT_INT8, ss=128),
          sfs_q=FAKE, sage_block_q=64, sfs_k=FAKE, sage_block_k=64, sfs_v=None, sage_block_v=0),
     F.FMHA_ERR_UNSUPPORTED, "no kernel"),                                                     # unscaled int8 V
    (dict(q=_tensor(7)), F.FMHA_ERR_INVALID, "dtype"),
    (dict(sage_block_v=32), F.FMHA_ERR_UNSUPPORTED, "sage_block_v"),
    (dict(sage_block_v=0), F.FMHA_ERR_INVALID, "sfs_v given"),
    (dict(q=_tensor(F.FMHA_DT_INT8)), F.FMHA_ERR_UNSUPPORTED, "no kernel"),
    (dict(k=_tensor(F.FMHA_DT_INT8)), F.FMHA_ERR_UNSUPPORTED, "no kernel"),
    (dict(lazy_rescale_log2=-1.0), F.FMHA_ERR_INVALID, "lazy"),
    (dict(lazy_rescale_log2=float("nan")), F.FMHA_ERR_INVALID, "lazy"),
    (dict(softmax_scale=float("inf")), F.FMHA_ERR_INVALID, "softmax_scale"),
    (dict(causal=2), F.FMHA_ERR_INVALID, "causal"),
    (dict(block_mask=FAKE, mask_block_q=128, mask_block_kv=256), F.FMHA_ERR_UNSUPPORTED, "mask_block_q"),
    (dict(block_mask=FAKE, mask_block_q=64, mask_block_kv=100), F.FMHA_ERR_UNSUPPORTED, "mask_block_kv"),
    (dict(page_table=FAKE, page_size=12, num_pages=4), F.FMHA_ERR_UNSUPPORTED, "page_size"),
    (dict(page_table=FAKE, page_size=8, num_pages=4), F.FMHA_ERR_UNSUPPORTED, "page_size"),
    (dict(page_table=FAKE, page_size=16, num_pages=0), F.FMHA_ERR_INVALID, "num_pages"),
    (dict(sfs_p=FAKE + 2), F.FMHA_ERR_INVALID, "sfs_p"),
])
def test_fwd_rejects_bad_arguments_before_any_hip_call(lib, kw, code, msg):
    rc, err = _call(lib, _params(**kw))
    assert rc == code and msg in err, (rc, err)


def test_fwd_accepts_the_layout_without_sfs_o(lib):
    # a caller built against the previous layout passes its smaller size;
    # the library then reads nothing past num_pages
    prev = F.FmhaFwdParams.sfs_o.offset
    rc, err = _call(lib, _params(struct_size=prev, Sq=0))
    assert rc == F.FMHA_OK and err == ""
    rc, err = _call(lib, _params(struct_size=prev + 4, Sq=0))
    assert rc == F.FMHA_ERR_INVALID and "struct_size" in err


def test_fwd_empty_key_sequence_needs_no_scales(lib):
    # Skv = 0: K/V and their scales may be null; every output row is zero
    # (the launch itself needs a GPU, so only the validation is checked here:
    # a null sfs_k with Skv > 0 is rejected, with Skv = 0 it is not)
    rc, err = _call(lib, _params(Skv=5, sfs_v=None))
    assert rc == F.FMHA_ERR_INVALID and "sfs_v is null" in err


def test_fwd_null_params(lib):
    assert lib.fmha_fwd(None, None) == F.FMHA_ERR_INVALID


def test_fwd_empty_problem_is_a_no_op(lib):
    rc, err = _call(lib, _params(Sq=0))
    assert rc == F.FMHA_OK and err == ""


def test_fwd_accepts_e4m3_k_with_int8_v(lib):
    # the K-fp8 / V-int8 combination passes validation (an empty problem, so
    # nothing is launched)
    p = _params(Sq=0, q=_tensor(F.FMHA_DT_E4M3), k=_tensor(F.FMHA_DT_E4M3), v=_tensor(F.FMHA_DT_INT8, ss=128),
                sfs_q=FAKE, sage_block_q=64, sfs_k=FAKE, sage_block_k=64)
    rc, err = _call(lib, p)
    assert rc == F.FMHA_OK and err == ""


@pytest.mark.parametrize("kw,code,msg", [
    (dict(D=64), F.FMHA_ERR_UNSUPPORTED, "D=64"),
    (dict(block=32), F.FMHA_ERR_UNSUPPORTED, "block_tokens"),
    (dict(xdt=F.FMHA_DT_E4M3), F.FMHA_ERR_INVALID, "bf16"),
    (dict(cdt=F.FMHA_DT_BF16), F.FMHA_ERR_INVALID, "int8 or e4m3"),
    (dict(S=-3), F.FMHA_ERR_INVALID, "negative"),
    (dict(xptr=FAKE + 4), F.FMHA_ERR_INVALID, "aligned"),
    (dict(scales=0), F.FMHA_ERR_INVALID, "scales"),
])
def test_quantize_rejects_bad_arguments(lib, kw, code, msg):
    x = _tensor(kw.get("xdt", F.FMHA_DT_BF16), ptr=kw.get("xptr", FAKE))
    c = _tensor(kw.get("cdt", F.FMHA_DT_E4M3))
    rc = lib.fmha_quantize_blocks(ctypes.byref(x), ctypes.byref(c), kw.get("scales", FAKE), 1, kw.get("S", 64), 4,
                                  kw.get("D", 128), kw.get("block", 64), None)
    err = lib.fmha_last_error().decode()
    assert rc == code and msg in err, (rc, err)


def test_quantize_empty_is_a_no_op(lib):
    x, c = _tensor(F.FMHA_DT_BF16), _tensor(F.FMHA_DT_INT8)
    assert lib.fmha_quantize_blocks(ctypes.byref(x), ctypes.byref(c), None, 0, 64, 4, 128, 64, None) == F.FMHA_OK


def _job(B=1, S=64, H=4, D=128, block=64, xdt=F.FMHA_DT_BF16, cdt=F.FMHA_DT_E4M3, xptr=FAKE, scales=FAKE):
    return F.FmhaQuantizeJob(_tensor(xdt, ptr=xptr), _tensor(cdt), scales, B, S, H, D, block)


def _batch(lib, jobs, n=None):
    arr = (F.FmhaQuantizeJob * max(1, len(jobs)))(*jobs)
    rc = lib.fmha_quantize_blocks_batch(arr, len(jobs) if n is None else n, None)
    return rc, lib.fmha_last_error().decode()


@pytest.mark.parametrize("jobs,n,code,msg", [
    ([_job()], -1, F.FMHA_ERR_INVALID, "n_jobs=-1"),
    ([_job()] * 9, None, F.FMHA_ERR_INVALID, "n_jobs=9"),
    ([_job(), _job(D=64)], None, F.FMHA_ERR_UNSUPPORTED, "quantize job 1: D=64"),
    ([_job(), _job(D=192)], None, F.FMHA_ERR_UNSUPPORTED, "one head dim per batch"),
    ([_job(), _job(), _job(xptr=0)], None, F.FMHA_ERR_INVALID, "quantize job 2 x: null pointer"),
    ([_job(cdt=F.FMHA_DT_BF16)], None, F.FMHA_ERR_INVALID, "quantize job 0: codes must be int8 or e4m3"),
    ([_job(), _job(scales=0)], None, F.FMHA_ERR_INVALID, "quantize job 1: null scales"),
    ([_job(block=32)], None, F.FMHA_ERR_UNSUPPORTED, "block_tokens"),
])
def test_quantize_batch_rejects_bad_arguments(lib, jobs, n, code, msg):
    rc, err = _batch(lib, jobs, n)
    assert rc == code and msg in err, (rc, err)


def test_quantize_batch_empty_is_a_no_op(lib):
    assert _batch(lib, [], 0) == (F.FMHA_OK, "")
    assert lib.fmha_quantize_blocks_batch(None, 0, None) == F.FMHA_OK
    rc, err = _batch(lib, [_job(B=0), _job(H=0)])
    assert rc == F.FMHA_OK and err == ""


def test_quantize_job_layout_matches_header(tmp_path):
    fields = [f for f, _ in F.FmhaQuantizeJob._fields_]
    src = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{HEADER}"', "int main(void){",
           'printf("%zu %d\\n", sizeof(fmha_quantize_job), FMHA_MAX_QUANTIZE_JOBS);']
    src += [f'printf("%zu\\n", offsetof(fmha_quantize_job, {f}));' for f in fields]
    src.append("return 0;}")
    c = tmp_path / "job.c"
    c.write_text("\n".join(src))
    exe = tmp_path / "job"
    subprocess.run(["gcc", str(c), "-o", str(exe)], check=True)
    vals = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(F.FmhaQuantizeJob) and vals[1] == F.MAX_QUANTIZE_JOBS
    assert vals[2:] == [getattr(F.FmhaQuantizeJob, f).offset for f in fields]


def _nvfp4(lib, **kw):
    a = dict(x=FAKE, xs=64, M=4, K=64, c=FAKE, cs=32, s=FAKE, ss=4, t=FAKE)
    a.update(kw)
    return lib.fmha_quantize_nvfp4(a["x"], a["xs"], a["M"], a["K"], a["c"], a["cs"], a["s"], a["ss"], a["t"], None)


@pytest.mark.parametrize("kw,msg", [
    (dict(K=40), "multiple of 16"),
    (dict(K=0), "multiple of 16"),
    (dict(M=-1), "negative"),
    (dict(x=0), "null"),
    (dict(t=0), "null"),
    (dict(x=FAKE + 8), "x not 16-byte aligned"),
    (dict(xs=48), "x_row_stride"),
    (dict(xs=68), "x_row_stride"),
    (dict(c=FAKE + 4), "codes not 8-byte aligned"),
    (dict(cs=16), "codes_row_stride"),
    (dict(cs=36), "codes_row_stride"),
    (dict(ss=3), "scales_row_stride"),
    (dict(t=FAKE + 2), "token_scales"),
])
def test_nvfp4_rejects_bad_arguments(lib, kw, msg):
    rc = _nvfp4(lib, **kw)
    err = lib.fmha_last_error().decode()
    assert rc == F.FMHA_ERR_INVALID and msg in err, (rc, err)


def test_nvfp4_rejects_rows_beyond_2_28(lib):
    rc = _nvfp4(lib, K=(1 << 28) + 16, xs=(1 << 28) + 16, cs=(1 << 27) + 8, ss=(1 << 24) + 1)
    assert rc == F.FMHA_ERR_UNSUPPORTED and "2^28" in lib.fmha_last_error().decode()


def test_nvfp4_empty_is_a_no_op(lib):
    assert _nvfp4(lib, M=0, x=0, c=0, s=0, t=0) == F.FMHA_OK
