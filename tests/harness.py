"""Shared test plumbing: run a workload through the HIP library and through
the oracle on the same seeded inputs, and compare the outputs."""
import numpy as np

from fmha_fwd_amd import workloads as W
from oracle.attention import attention, dequantize
from oracle.codecs import bf16_round64
from oracle.quantize import quantize_blocks as oracle_quantize

TOL_MAXABS = 1.5e-2
TOL_COS_Q = 0.999
TOL_COS_U = 0.99
# Distance from a P rounding boundary within which a binary32 kernel may
# round the other way: the oracle's per-pair bound for a kernel that
# accumulates the scores in binary32 (at most D roundings), rounds at most
# four more times in the exponent and evaluates exp2 within 2 ulp.
FLIP_EPS = "binary32"
# Elements over the max-abs bar that the P-rounding bound excuses: at most
# five in ten thousand of those compared (measured up to 2.8e-4 on the E4M3
# Q/K inputs with per-head deviations up to 2 at the default softmax scale),
# or one row's worth in small cases, or as many as the oracle finds able to
# cross the bar on a tie (elements whose bound exceeds it: a sharper softmax
# concentrates a row on a few keys whose flipped P code moves the whole row).
TIE_FRACTION = 5e-4
TIE_FLOOR = 128
# every parity comparison of the session, printed by the terminal summary
RECORDS = []


# ------------------------------------------------------------------ oracle side
def oracle_operands(spec, data, heads_q=None, heads_kv=None):
    """fp64 dequantised Q, K, V (logical token order) computed by the oracle.

    heads_q / heads_kv restrict the heads that are quantised (the others are
    left NaN); blocks are per (batch, head), so a head subset is exact.
    """
    def prep(x, fmt, heads):
        if heads is not None:
            out = np.full(x.shape, np.nan)
            sub = x[:, :, heads]
        else:
            sub = x
        if fmt == "bf16":
            d = sub.astype(np.float64)
        else:
            c, s = oracle_quantize(sub, fmt)
            d = dequantize(c, fmt, s)
        if heads is None:
            return d
        out[:, :, heads] = d
        return out
    return (prep(data["q"], spec.q_fmt, heads_q), prep(data["k"], spec.k_fmt, heads_kv),
            prep(data["v"], spec.v_fmt, heads_kv))


def oracle_output(spec, data, operands, rows=None, heads=None, quantized=True, **kw):
    """(O, rounding-sensitivity bound) of the quantisation-emulating oracle."""
    qd, kd, vd = operands
    p_fmt = spec.p_fmt if quantized else None
    return attention(qd, kd, vd, causal=spec.causal, block_mask=data.get("block_mask"), mode="lazy",
                     p_format=p_fmt, rows=rows, heads=heads, flip_eps=FLIP_EPS, **kw)


def unquantized_output(spec, data, rows=None, heads=None, **kw):
    qd, kd, vd = (data[n].astype(np.float64) for n in ("q", "k", "v"))
    return attention(qd, kd, vd, causal=spec.causal, block_mask=data.get("block_mask"), mode="exact",
                     p_format=None, rows=rows, heads=heads, **kw)


# ------------------------------------------------------------------ GPU side
def to_gpu_bf16(x, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).to(device)


def gpu_run(spec, data, device="cuda", **fwd_kw):
    """Quantise on the GPU as the spec says, then run fmha_fwd.  Returns
    (o as float32 numpy, dict of GPU tensors used)."""
    import torch
    import fmha_fwd_amd as F
    t = {}
    q = to_gpu_bf16(data["q"], device)
    k = to_gpu_bf16(data["k"], device)
    v = to_gpu_bf16(data["v"], device)
    if spec.q_scaled:
        q, t["sfs_q"] = F.quantize_blocks(q, spec.q_fmt)
    if spec.k_scaled:
        k, t["sfs_k"] = F.quantize_blocks(k, spec.k_fmt)
    if spec.v_scaled:
        v, t["sfs_v"] = F.quantize_blocks(v, spec.v_fmt)
    kw = dict(causal=spec.causal)
    if spec.paged:
        pt = torch.from_numpy(data["page_table"]).to(device)
        ps = spec.page_size
        n_pages = max(pt.numel(), int(data["page_table"].max()) + 1)  # pages no table entry names stay zero
        S = spec.S
        kpool = torch.zeros((n_pages, ps) + tuple(k.shape[2:]), dtype=k.dtype, device=device)
        vpool = torch.zeros((n_pages, ps) + tuple(v.shape[2:]), dtype=v.dtype, device=device)
        for b in range(spec.B):
            for p in range(pt.shape[1]):
                lo, hi = p * ps, min(p * ps + ps, S)
                kpool[int(data["page_table"][b, p]), :hi - lo] = k[b, lo:hi]
                vpool[int(data["page_table"][b, p]), :hi - lo] = v[b, lo:hi]
        k, v = kpool, vpool
        kw.update(page_table=pt, page_size=ps, seq_len_kv=S)
    if spec.masked:
        kw["block_mask"] = torch.from_numpy(data["block_mask"]).to(device)
    kw.update(fwd_kw)
    o = F.fwd(q, k, v, sfs_q=t.get("sfs_q"), sfs_k=t.get("sfs_k"), sfs_v=t.get("sfs_v"), **kw)
    torch.cuda.synchronize()
    t.update(q=q, k=k, v=v, o=o)
    return o.float().cpu().numpy(), t


# ------------------------------------------------------------------ comparison
def bad_mask(gpu, ref, bound):
    """Elements that fail the max-abs bar (the n_bad of `compare`)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref_bf = bf16_round64(np.asarray(ref, dtype=np.float64))
    diff = np.abs(gpu - ref_bf)
    _, e = np.frexp(np.maximum(np.abs(gpu), np.abs(ref_bf)))
    one_ulp = (diff > 0) & (diff <= np.ldexp(1.0, e - 8))
    return (diff > TOL_MAXABS) & ~one_ulp & (diff > TOL_MAXABS + np.asarray(bound, dtype=np.float64))


def compare(gpu, ref, bound=None):
    """Max-abs error against the oracle rounded to bf16 (differences of one
    bf16 unit in the last place are counted apart, and so are differences
    within the oracle's P-rounding sensitivity bound), and cosine similarity."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    bound = np.zeros_like(ref) if bound is None else np.asarray(bound, dtype=np.float64)
    ref_bf = bf16_round64(ref)
    diff = np.abs(gpu - ref_bf)
    mag = np.maximum(np.abs(gpu), np.abs(ref_bf))
    _, e = np.frexp(mag)
    ulp = np.ldexp(1.0, e - 8)
    one_ulp = (diff > 0) & (diff <= ulp)
    over = (diff > TOL_MAXABS) & ~one_ulp
    bad = over & (diff > TOL_MAXABS + bound)
    cos = cosine(gpu, ref)
    return dict(maxabs=float(diff.max()) if diff.size else 0.0, n_bad=int(bad.sum()), n_ulp=int(one_ulp.sum()),
                n_tie=int((over & ~bad).sum()), n_cand=int((bound > TOL_MAXABS).sum()), cos=cos, n=int(diff.size))


def cosine(a, b):
    a = np.asarray(a, dtype=np.float64).ravel()
    b = np.asarray(b, dtype=np.float64).ravel()
    return float(np.dot(a, b) / (np.linalg.norm(a) * np.linalg.norm(b) + 1e-300))


def assert_parity(gpu, ref_and_bound, unq=None, what=""):
    """The parity bar.  Against unquantised attention the kernel must reach
    cosine 0.99, or, where the quantised method itself does not (int8 Q/K with
    x20 outlier channels), add no more than 1e-3 of cosine distance to the
    method's own."""
    ref, bound = ref_and_bound
    r = compare(gpu, ref, bound)
    r["tie_cap"] = int(max(TIE_FLOOR, TIE_FRACTION * r["n"], r["n_cand"]))
    RECORDS.append((what, r))
    msg = f"{what}: {r}"
    assert np.all(np.isfinite(gpu)), msg
    if r["n_bad"]:
        idx = [tuple(int(x) for x in i) for i in np.argwhere(bad_mask(gpu, ref, bound))[:5]]
        msg += " failing (index, gpu, oracle, bound): " + str([(i, float(np.asarray(gpu)[i]), float(ref[i]),
                                                                 float(np.asarray(bound)[i])) for i in idx])
    assert r["n_bad"] == 0, msg
    assert r["n_tie"] <= r["tie_cap"], msg
    assert r["cos"] >= TOL_COS_Q, msg
    if unq is not None:
        cu = cosine(gpu, unq)
        cm = cosine(ref, unq)
        r.update(cos_unq=cu, cos_unq_method=cm)
        assert cu >= min(TOL_COS_U, cm - 1e-3), f"{msg} cos_unquantized={cu} (method's own {cm})"
    print(f"parity {what}: {r}")
    return r
