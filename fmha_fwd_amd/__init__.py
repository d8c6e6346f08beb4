"""Python binding of libfmha.so, the gfx950 mixed-precision attention library.

Argument marshalling only: torch provides device memory, dtypes and the
current stream; every step of the computation runs in the HIP kernels behind
the C ABI declared in include/fmha.h.  There is no fallback: if the library is
missing, importing ``fmha_fwd_amd.lib_handle()`` raises.

    codes, scales = quantize_blocks(x, "e4m3")           # x: bf16 [B,S,H,128 or 192]
    o = fwd(q, k, v, sfs_q=..., sfs_k=..., sfs_v=..., causal=True)
    codes, block_scales, token_scales = quantize_nvfp4(a)  # a: bf16 [M, K]
"""
import ctypes
import math
import os

# FMHA_LIB selects another build of the same library (e.g. a tuning variant).
LIB_PATH = os.environ.get("FMHA_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libfmha.so")

FMHA_DT_BF16, FMHA_DT_E4M3, FMHA_DT_INT8 = 1, 2, 3
FMHA_OK, FMHA_ERR_INVALID, FMHA_ERR_UNSUPPORTED, FMHA_ERR_HIP = 0, -1, -2, -3
EXPORTED = ("fmha_quantize_blocks", "fmha_quantize_blocks_batch", "fmha_fwd", "fmha_quantize_nvfp4", "fmha_last_error",
            "fmha_abi_version")
MAX_QUANTIZE_JOBS = 8


class FmhaTensor(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("stride_b", ctypes.c_int64), ("stride_s", ctypes.c_int64), ("stride_h", ctypes.c_int64)]


class FmhaQuantizeJob(ctypes.Structure):
    _fields_ = [("x", FmhaTensor), ("codes", FmhaTensor), ("scales", ctypes.c_void_p),
                ("B", ctypes.c_int32), ("S", ctypes.c_int32), ("H", ctypes.c_int32), ("D", ctypes.c_int32),
                ("block_tokens", ctypes.c_int32)]


class FmhaFwdParams(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("B", ctypes.c_int32), ("Sq", ctypes.c_int32), ("Skv", ctypes.c_int32),
        ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32),
        ("q", FmhaTensor), ("k", FmhaTensor), ("v", FmhaTensor), ("o", FmhaTensor),
        ("sfs_q", ctypes.c_void_p), ("sfs_k", ctypes.c_void_p), ("sfs_v", ctypes.c_void_p),
        ("sage_block_q", ctypes.c_int32), ("sage_block_k", ctypes.c_int32), ("sage_block_v", ctypes.c_int32),
        ("sfs_p", ctypes.c_void_p),
        ("softmax_scale", ctypes.c_float),
        ("lazy_rescale_log2", ctypes.c_float),
        ("causal", ctypes.c_int32),
        ("block_mask", ctypes.c_void_p),
        ("mask_stride_b", ctypes.c_int64), ("mask_stride_h", ctypes.c_int64), ("mask_stride_qb", ctypes.c_int64),
        ("mask_block_q", ctypes.c_int32), ("mask_block_kv", ctypes.c_int32),
        ("page_table", ctypes.c_void_p),
        ("page_table_stride_b", ctypes.c_int64),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("sfs_o", ctypes.c_void_p),
    ]


class FmhaError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"fmha error {code}: {msg}")
        self.code = code


_lib = None


def lib_handle():
    """The loaded libfmha.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} not built; run `python -m fmha_fwd_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        lib.fmha_quantize_blocks.argtypes = [ctypes.POINTER(FmhaTensor), ctypes.POINTER(FmhaTensor), ctypes.c_void_p,
                                             ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_int32, ctypes.c_void_p]
        lib.fmha_quantize_blocks.restype = ctypes.c_int
        lib.fmha_quantize_blocks_batch.argtypes = [ctypes.POINTER(FmhaQuantizeJob), ctypes.c_int32, ctypes.c_void_p]
        lib.fmha_quantize_blocks_batch.restype = ctypes.c_int
        lib.fmha_fwd.argtypes = [ctypes.POINTER(FmhaFwdParams), ctypes.c_void_p]
        lib.fmha_fwd.restype = ctypes.c_int
        lib.fmha_quantize_nvfp4.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                            ctypes.c_void_p, ctypes.c_void_p]
        lib.fmha_quantize_nvfp4.restype = ctypes.c_int
        lib.fmha_last_error.argtypes = []
        lib.fmha_last_error.restype = ctypes.c_char_p
        lib.fmha_abi_version.argtypes = []
        lib.fmha_abi_version.restype = ctypes.c_uint32
        _lib = lib
    return _lib


def _check(rc):
    if rc != FMHA_OK:
        raise FmhaError(rc, lib_handle().fmha_last_error().decode())


def _dtype_code(t):
    import torch
    m = {torch.bfloat16: FMHA_DT_BF16, torch.float8_e4m3fn: FMHA_DT_E4M3, torch.int8: FMHA_DT_INT8}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def _tensor(t):
    if t.dim() != 4:
        raise ValueError("expected a 4-D tensor [B, S, H, D]")
    if t.stride(3) != 1:
        raise ValueError("the last (channel) dimension must be contiguous")
    return FmhaTensor(t.data_ptr(), _dtype_code(t), t.stride(0), t.stride(1), t.stride(2))


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _require_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")


def quantize_blocks(x, dtype="e4m3", *, codes=None, scales=None, stream=None):
    """Per-(batch, head, 64-token block) quantisation of bf16 x [B, S, H, D],
    D = 128 or 192.

    Returns (codes, scales): codes int8 / float8_e4m3fn of x's shape, scales
    fp32 [B, H, ceil(S/64)].
    """
    import torch
    _require_cuda(x)
    B, S, H, D = x.shape
    tdt = {"int8": torch.int8, "e4m3": torch.float8_e4m3fn}[dtype]
    if codes is None:
        codes = torch.empty((B, S, H, D), dtype=tdt, device=x.device)
    if scales is None:
        scales = torch.empty((B, H, (S + 63) // 64), dtype=torch.float32, device=x.device)
    if not scales.is_contiguous():
        raise ValueError("scales must be contiguous")
    if tuple(codes.shape) != (B, S, H, D) or tuple(scales.shape) != (B, H, (S + 63) // 64):
        raise ValueError(f"codes must be {(B, S, H, D)} and scales {(B, H, (S + 63) // 64)}")
    xt, ct = _tensor(x), _tensor(codes)
    _check(lib_handle().fmha_quantize_blocks(ctypes.byref(xt), ctypes.byref(ct), scales.data_ptr(),
                                             B, S, H, D, 64, _stream(stream)))
    return codes, scales


def quantize_blocks_batch(jobs, *, stream=None):
    """Several `quantize_blocks` calls in one launch.  jobs: a list of
    (x, dtype) or (x, dtype, codes, scales) with x bf16 [B, S, H, D] (one D
    for all).  Returns a list of (codes, scales), bit-identical to separate
    calls."""
    import torch
    if len(jobs) > MAX_QUANTIZE_JOBS:
        raise ValueError(f"at most {MAX_QUANTIZE_JOBS} jobs per launch")
    arr = (FmhaQuantizeJob * max(1, len(jobs)))()
    out = []
    for i, job in enumerate(jobs):
        x, dtype = job[0], job[1]
        codes = job[2] if len(job) > 2 else None
        scales = job[3] if len(job) > 3 else None
        _require_cuda(x)
        B, S, H, D = x.shape
        tdt = {"int8": torch.int8, "e4m3": torch.float8_e4m3fn}[dtype]
        if codes is None:
            codes = torch.empty((B, S, H, D), dtype=tdt, device=x.device)
        if scales is None:
            scales = torch.empty((B, H, (S + 63) // 64), dtype=torch.float32, device=x.device)
        if not scales.is_contiguous():
            raise ValueError("scales must be contiguous")
        if tuple(codes.shape) != (B, S, H, D) or tuple(scales.shape) != (B, H, (S + 63) // 64):
            raise ValueError(f"job {i}: codes must be {(B, S, H, D)} and scales {(B, H, (S + 63) // 64)}")
        arr[i] = FmhaQuantizeJob(_tensor(x), _tensor(codes), scales.data_ptr(), B, S, H, D, 64)
        out.append((codes, scales))
    _check(lib_handle().fmha_quantize_blocks_batch(arr, len(jobs), _stream(stream)))
    return out


def quantize_nvfp4(x, *, codes=None, block_scales=None, token_scales=None, stream=None):
    """Per-token NVFP4 quantisation of bf16 x [M, K] (K a multiple of 16,
    rows strided, last dimension contiguous).

    Returns (codes uint8 [M, K/2], two E2M1 codes per byte with element 2i in
    the low nibble; block_scales float8_e4m3fn [M, K/16]; token_scales fp32
    [M]); x ~ E2M1 value * block scale * token scale.
    """
    import torch
    _require_cuda(x, codes, block_scales, token_scales)
    if x.dim() != 2 or x.dtype != torch.bfloat16 or x.stride(1) != 1:
        raise ValueError("x must be a bf16 [M, K] tensor with a contiguous last dimension")
    M, K = x.shape
    if codes is None:
        codes = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
    if block_scales is None:
        block_scales = torch.empty((M, K // 16), dtype=torch.float8_e4m3fn, device=x.device)
    if token_scales is None:
        token_scales = torch.empty((M,), dtype=torch.float32, device=x.device)
    for t in (codes, block_scales):
        if t.dim() != 2 or t.element_size() != 1 or t.stride(1) != 1:
            raise ValueError("codes / block_scales must be 2-D byte tensors with a contiguous last dimension")
    if not token_scales.is_contiguous() or token_scales.dtype != torch.float32:
        raise ValueError("token_scales must be a contiguous fp32 tensor")
    if tuple(codes.shape) != (M, K // 2) or tuple(block_scales.shape) != (M, K // 16) or token_scales.numel() != M:
        raise ValueError(f"codes must be {(M, K // 2)}, block_scales {(M, K // 16)}, token_scales ({M},)")
    _check(lib_handle().fmha_quantize_nvfp4(x.data_ptr(), x.stride(0), M, K, codes.data_ptr(), codes.stride(0),
                                            block_scales.data_ptr(), block_scales.stride(0),
                                            token_scales.data_ptr(), _stream(stream)))
    return codes, block_scales, token_scales


def _check_shapes(q, k, v, out, sfs_q, sfs_k, sfs_v, sfs_p, sfs_o, block_mask, mask_block, page_table, page_size,
                  Skv, Hkv):
    """The C ABI sees pointers and strides only: every extent the kernels
    index with is checked here against q's [B, Sq, Hq, D]."""
    B, Sq, Hq, D = q.shape

    def need(cond, what):
        if not cond:
            raise ValueError(what)
    for name, t in (("k", k), ("v", v), ("out", out)):
        need(t.dim() == 4, f"{name} must be 4-D")
    if page_table is None:
        need(tuple(k.shape) == (B, Skv, Hkv, D), f"k must be [B, Skv, Hkv, D] = [{B}, {Skv}, {Hkv}, {D}], got {tuple(k.shape)}")
    else:
        need(k.shape[1] == page_size and k.shape[3] == D,
             f"paged k must be [pages, {page_size}, Hkv, {D}], got {tuple(k.shape)}")
        need(page_table.dim() == 2 and page_table.shape[0] == B and page_table.shape[1] * page_size >= Skv,
             f"page_table must be [B, >= ceil(Skv / page_size)] = [{B}, {-(-Skv // page_size)}]")
    need(tuple(v.shape) == tuple(k.shape), f"v must have k's shape {tuple(k.shape)}, got {tuple(v.shape)}")
    need(tuple(out.shape) == (B, Sq, Hq, D), f"out must be [B, Sq, Hq, D] = [{B}, {Sq}, {Hq}, {D}]")
    for name, t, H, S in (("sfs_q", sfs_q, Hq, Sq), ("sfs_k", sfs_k, Hkv, Skv), ("sfs_v", sfs_v, Hkv, Skv)):
        if t is not None:
            need(tuple(t.shape) == (B, H, -(-S // 64)), f"{name} must be [B, H, ceil(S / 64)] = [{B}, {H}, {-(-S // 64)}]")
    for name, t in (("sfs_p", sfs_p), ("sfs_o", sfs_o)):
        if t is not None:
            need(t.numel() >= Hq, f"{name} needs Hq = {Hq} entries")
    if block_mask is not None:
        bq, bkv = mask_block
        want = (B, Hq, -(-Sq // bq), -(-Skv // bkv))
        need(tuple(block_mask.shape) == want, f"block_mask must be {want} (expand() views broadcast), got "
                                              f"{tuple(block_mask.shape)}")


def fwd(q, k, v, *, sfs_q=None, sfs_k=None, sfs_v=None, sfs_p=None, causal=False, block_mask=None,
        mask_block=(64, 256), page_table=None, page_size=16, seq_len_kv=None, softmax_scale=None,
        lazy_rescale_log2=8.0, out=None, out_dtype="bf16", sfs_o=None, stream=None):
    """Attention forward; returns o ([B, Sq, Hq, D], bf16, or E4M3 when
    out_dtype is "e4m3" or `out` is float8_e4m3fn; sfs_o: fp32 [Hq] output
    scale of an E4M3 o, o = encode(O / sfs_o)).

    q: [B, Sq, Hq, D] bf16 / int8 / float8_e4m3fn.  k, v: [B, Skv, Hkv, D]
    (v also int8 under an E4M3 Q and K, with its block scales),
    or with page_table (int32 [B, pages]) pools [num_pages, page_size, Hkv, D]
    and seq_len_kv giving Skv.  D = 128 or 192 (at 192 a bf16 Q and K with
    an E4M3 V need its scale).  sfs_*: fp32 [B, H, ceil(S/64)] block
    scales.
    block_mask: uint8 [B, Hq, ceil(Sq/64), ceil(Skv/256)] (strides honoured;
    last dim contiguous).
    """
    import torch
    _require_cuda(q, k, v, sfs_q, sfs_k, sfs_v, sfs_p, block_mask, page_table, out, sfs_o)
    B, Sq, Hq, D = q.shape
    if page_table is None:
        Skv, Hkv = k.shape[1], k.shape[2]
    else:
        if seq_len_kv is None:
            raise ValueError("seq_len_kv is required with a page table")
        Skv, Hkv = int(seq_len_kv), k.shape[2]
    if out is None:
        odt = {"bf16": torch.bfloat16, "e4m3": torch.float8_e4m3fn}[out_dtype]
        out = torch.empty((B, Sq, Hq, D), dtype=odt, device=q.device)
    for s in (sfs_q, sfs_k, sfs_v, sfs_p, sfs_o):
        if s is not None and (s.dtype != torch.float32 or not s.is_contiguous()):
            raise ValueError("scale factors must be contiguous float32")
    _check_shapes(q, k, v, out, sfs_q, sfs_k, sfs_v, sfs_p, sfs_o, block_mask, mask_block, page_table, page_size,
                  Skv, Hkv)
    p = FmhaFwdParams()
    p.struct_size = ctypes.sizeof(FmhaFwdParams)
    p.B, p.Sq, p.Skv, p.Hq, p.Hkv, p.D = B, Sq, Skv, Hq, Hkv, D
    p.q, p.k, p.v, p.o = _tensor(q), _tensor(k), _tensor(v), _tensor(out)
    p.sfs_q, p.sfs_k, p.sfs_v = _ptr(sfs_q), _ptr(sfs_k), _ptr(sfs_v)
    p.sage_block_q = 64 if sfs_q is not None else 0
    p.sage_block_k = 64 if sfs_k is not None else 0
    p.sage_block_v = 64 if sfs_v is not None else 0
    p.sfs_p = _ptr(sfs_p)
    p.sfs_o = _ptr(sfs_o)
    p.softmax_scale = 0.0 if softmax_scale is None else float(softmax_scale)
    p.lazy_rescale_log2 = float(lazy_rescale_log2)
    p.causal = 1 if causal else 0
    if block_mask is not None:
        if block_mask.dtype != torch.uint8 or block_mask.dim() != 4 or block_mask.stride(3) != 1:
            raise ValueError("block_mask must be uint8 [B, Hq, q_blocks, kv_blocks] with a contiguous last dim")
        p.block_mask = block_mask.data_ptr()
        p.mask_stride_b, p.mask_stride_h, p.mask_stride_qb = block_mask.stride(0), block_mask.stride(1), block_mask.stride(2)
        p.mask_block_q, p.mask_block_kv = mask_block
    if page_table is not None:
        if page_table.dtype != torch.int32 or page_table.dim() != 2 or page_table.stride(1) != 1:
            raise ValueError("page_table must be int32 [B, pages] with a contiguous last dim")
        p.page_table = page_table.data_ptr()
        p.page_table_stride_b = page_table.stride(0)
        p.page_size = page_size
        p.num_pages = k.shape[0]
    _check(lib_handle().fmha_fwd(ctypes.byref(p), _stream(stream)))
    return out


def default_softmax_scale(d=128):
    return 1.0 / math.sqrt(d)
