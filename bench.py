"""Throughput of the mixed-precision attention forward on one MI355X.

One step = the whole hot path over one batch of synthetic input already in
HBM: block quantisation of the operands the workload quantises
(fmha_quantize_blocks), then the fused attention forward (fmha_fwd).  The
default workload is the DiT-scale self-attention with bf16 Q/K and E4M3 V/P
(B=1, H=40, S=32760, d=128, non-causal, 2^8 lazy rescale).

Prints one JSON line.  Timing: W untimed warm-up steps, then K steps between
two device synchronisations; per-kernel durations come from HIP events
recorded on the launch stream around every launch of the timed steps.

    python bench.py [--steps K] [--warmup W] [--workload dit] [--no-cpu-baseline]

`--workload nvfp4` measures the per-token NVFP4 quantiser instead (GB/s
against the HBM peak; one step = one launch over a 16384 x 8192 matrix).
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# Published dense peaks of MI355X (TFLOP/s) and HBM bandwidth (GB/s).
PEAK = {"bf16": 2500.0, "f16": 2500.0, "e4m3": 5000.0, "int8": 5000.0}
HBM_PEAK_GBS = 8000.0
METRIC = "fmha_fwd TFLOP/s (4·B·H·Sq·Skv·d, mask-aware) + % of MI355X dtype MFMA peak"


def mixed_peak(qk_fmt, pv_fmt):
    """Dense MFMA peak of a step whose FLOPs split evenly between the QK^T
    product (qk_fmt) and the PV product (pv_fmt): time-weighted harmonic mean."""
    return 1.0 / (0.5 / PEAK[qk_fmt] + 0.5 / PEAK[pv_fmt])


def code_text(path):
    """Source text with comments and blank space removed: what a traffic
    record's hash covers (a comment edit does not change the kernel)."""
    import re
    txt = open(path).read()
    txt = re.sub(r"/\*.*?\*/", " ", txt, flags=re.S)
    txt = re.sub(r"//[^\n]*", " ", txt)
    return " ".join(txt.split()).encode()


def source_hash():
    h = hashlib.sha256()
    for f in ("attention.hip", "device_common.h"):
        h.update(code_text(os.path.join(ROOT, "fmha_fwd_amd", "csrc", f)))
    return h.hexdigest()[:16]


def pair_count(spec, data):
    if spec.masked:
        bm = data["block_mask"].astype(bool)
        S = spec.S
        # active (query block, key block) pairs, clipped to the sequence
        qlen = np.minimum(64, S - 64 * np.arange(bm.shape[2]))
        klen = np.minimum(256, S - 256 * np.arange(bm.shape[3]))
        return int((bm * qlen[None, None, :, None] * klen[None, None, None, :]).sum())
    return spec.pairs()


ESIZE = {"bf16": 2, "e4m3": 1, "int8": 1}


def attention_bytes(spec):
    """Algorithmic HBM bytes of one fmha_fwd launch: every operand byte read
    once (Q, K, V, their 64-token block scales, the block mask and the page
    table where used) and the bf16 output written once."""
    B, Hq, Hkv, S, D, nq = spec.B, spec.Hq, spec.Hkv, spec.S, spec.D, spec.n_q
    nb = lambda n: -(-n // 64)  # noqa: E731
    b = B * Hq * nq * D * ESIZE[spec.q_fmt] + B * Hkv * S * D * (ESIZE[spec.k_fmt] + ESIZE[spec.v_fmt])
    b += B * Hq * nq * D * 2
    b += 4 * ((B * Hq * nb(nq) if spec.q_fmt != "bf16" else 0) + (B * Hkv * nb(S) if spec.k_fmt != "bf16" else 0)
              + (B * Hkv * nb(S) if spec.v_fmt != "bf16" else 0))
    if spec.masked:
        b += B * Hq * nb(nq) * -(-S // 256)
    if spec.paged:
        b += B * -(-S // spec.page_size) * 4
    return b


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return 1


def host_cores():
    """Cores this process may run on (the CPU share of the box)."""
    return len(os.sched_getaffinity(0))


def cpu_baseline(spec, data, budget_s=12.0, n_heads=6):
    """The oracle (as it stands) on a bounded row sample of the workload:
    rows of n_heads (batch, query head) pairs spread over the workload (the
    first and the last head and random ones), each head's first, last and
    tail-block rows first, then random rows, 64 at a time, round robin over
    the heads until the time budget is spent.  Rows are independent, so the
    sample is exact for the rows it covers."""
    from oracle.attention import attention, dequantize
    from oracle.quantize import quantize_blocks
    rng = np.random.default_rng(0)
    nq, group = spec.n_q, spec.Hq // spec.Hkv
    heads = [(0, 0), (spec.B - 1, spec.Hq - 1)]
    while len(heads) < min(n_heads, spec.B * spec.Hq):
        bh = (int(rng.integers(spec.B)), int(rng.integers(spec.Hq)))
        if bh not in heads:
            heads.append(bh)

    def operand(x, fmt, b, hh):
        sub = x[b:b + 1, :, [hh]]
        if fmt == "bf16":
            return sub.astype(np.float64)
        c, s = quantize_blocks(sub, fmt)
        return dequantize(c, fmt, s)

    bm_all = data.get("block_mask")
    first = np.unique(np.clip([0, 1, 63, 64, nq - 1, nq - 2, nq - 57, nq - 64, nq // 2], 0, nq - 1))
    plan = []
    for b, h in heads:
        pool = np.setdiff1d(np.arange(nq), first)
        plan.append([b, h, None, list(first) + list(rng.permutation(pool))])
    t_prep, t_att, rows_done, pairs_done = 0.0, 0.0, 0, 0
    i = 0
    while t_att < budget_s and any(p[3] for p in plan):
        entry = plan[i % len(plan)]
        i += 1
        b, h, ops, todo = entry
        if not todo:
            continue
        if ops is None:
            t0 = time.perf_counter()
            ops = entry[2] = (operand(data["q"], spec.q_fmt, b, h), operand(data["k"], spec.k_fmt, b, h // group),
                              operand(data["v"], spec.v_fmt, b, h // group))
            t_prep += time.perf_counter() - t0
        rows = np.sort(np.array(todo[:64]))
        del todo[:64]
        bm = None if bm_all is None else bm_all[b:b + 1, [h]]
        t0 = time.perf_counter()
        attention(*ops, causal=spec.causal, block_mask=bm, mode="lazy", p_format=spec.p_fmt, rows=rows,
                  heads=[(0, 0)])
        t_att += time.perf_counter() - t0
        rows_done += len(rows)
        if spec.causal:
            pairs_done += int(np.minimum(rows + spec.S - nq + 1, spec.S).sum())
        elif bm is not None:
            klen = np.minimum(256, spec.S - 256 * np.arange(bm.shape[3]))
            pairs_done += int(sum((bm[0, 0, r // 64] != 0).astype(np.int64) @ klen for r in rows))
        else:
            pairs_done += len(rows) * spec.S
    flops = 4.0 * spec.D * pairs_done
    return {"value": flops / t_att / 1e12, "unit": "TFLOP/s", "cores": host_cores(), "blas_threads": blas_threads(),
            "kind": "oracle", "rows_per_s": rows_done / t_att,
            "extrapolated_full_s": 4.0 * spec.D * (pair_count(spec, data) or 0) / (flops / t_att),
            "rows_total": spec.B * spec.Hq * nq,
            "sample": f"{rows_done} query rows of {len(heads)} (batch, head) pairs {heads} (each head's first, last "
                      f"and tail-block rows, then random rows), all their valid keys, lazy {spec.p_fmt}-P oracle "
                      f"in fp64 numpy; operand dequantisation ({t_prep:.1f} s) not counted; {t_att:.1f} s of CPU "
                      f"time",
            "seconds": round(t_att, 2)}


class SclkSampler:
    """Shader (GFX) clock read from the amdgpu sysfs files of the benchmarked
    device while the timed steps run: hwmon's freq1_input (Hz), else the
    level marked current in pp_dpm_sclk (MHz).  A background thread polls it
    every few milliseconds; no subprocess."""

    def __init__(self, torch, period_s=0.003):
        import glob
        import threading
        self.samples, self.period, self.source = [], period_s, None
        dirs = []
        try:
            pr = torch.cuda.get_device_properties(0)
            dom, bus, dev = (getattr(pr, n, None) for n in ("pci_domain_id", "pci_bus_id", "pci_device_id"))
            if bus is not None:
                dirs = [f"/sys/bus/pci/devices/{dom or 0:04x}:{bus:02x}:{dev or 0:02x}.0"]
        except Exception:  # pragma: no cover
            pass
        if not dirs or not os.path.isdir(dirs[0]):
            cands = [d for d in glob.glob("/sys/class/drm/card*/device") if os.path.exists(d + "/pp_dpm_sclk")]
            dirs = cands if len(set(map(os.path.realpath, cands))) == 1 else []
        for d in dirs[:1]:
            hw = sorted(glob.glob(d + "/hwmon/hwmon*/freq1_input"))
            if hw:
                self.source = (hw[0], 1e-9)
            elif os.path.exists(d + "/pp_dpm_sclk"):
                self.source = (d + "/pp_dpm_sclk", None)
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def read(self):
        path, scale = self.source
        txt = open(path).read()
        if scale is not None:
            return float(txt.split()[0]) * scale
        for line in txt.splitlines():
            if line.rstrip().endswith("*"):
                return float(line.split(":")[1].strip().lower().split("mhz")[0]) * 1e-3
        return None

    def _run(self):
        while not self._stop.is_set():
            try:
                v = self.read()
                if v:
                    self.samples.append(v)
            except Exception:  # pragma: no cover
                return
            self._stop.wait(self.period)

    def __enter__(self):
        if self.source is not None:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread.is_alive():
            self._thread.join()

    def summary(self):
        if not self.samples:
            return None
        return {"ghz_median": float(np.median(self.samples)), "ghz_min": float(np.min(self.samples)),
                "ghz_max": float(np.max(self.samples)), "samples": len(self.samples), "source": self.source[0]}


SCLK_MIN_SAMPLES = 10  # sysfs clock readings needed before a median is reported
COPY_BYTES = 1 << 30
NVFP4_METRIC = "per-token NVFP4 quantisation GB/s (algorithmic bytes: 2 read + 0.5 + 1/16 written per element, 4 per token)"


def nvfp4_bytes(M, K):
    return M * K * 2 + M * K // 2 + M * K // 16 + 4 * M


def nvfp4_source_hash():
    h = hashlib.sha256()
    for f in ("nvfp4.hip", "device_common.h"):
        h.update(code_text(os.path.join(ROOT, "fmha_fwd_amd", "csrc", f)))
    return h.hexdigest()[:16]


def nvfp4_cpu_baseline(x_rows_fn, M, K, budget_s=12.0):
    """The NVFP4 oracle (as it stands) on a bounded row sample."""
    from oracle.nvfp4 import quantize_nvfp4
    rng = np.random.default_rng(0)
    rows_done, t = 0, 0.0
    while t < budget_s and rows_done < M:
        g = int(rng.integers(0, max(M // 256, 1)))
        x = x_rows_fn(np.arange(256 * g, min(256 * g + 256, M)))  # one 256-row group
        t0 = time.perf_counter()
        quantize_nvfp4(x)
        t += time.perf_counter() - t0
        rows_done += 256
    return {"value": nvfp4_bytes(rows_done, K) / t / 1e9, "unit": "GB/s", "cores": host_cores(),
            "blas_threads": blas_threads(), "kind": "oracle",
            "rows_per_s": rows_done / t, "extrapolated_full_s": M / (rows_done / t),
            "sample": f"{rows_done} rows (random 256-row groups) of the {M} x {K} matrix, NVFP4 oracle in numpy float32 emulation; "
                      f"{t:.1f} s of CPU time", "seconds": round(t, 2)}


def bench_nvfp4(args, torch, F, W):
    """One step = one fmha_quantize_nvfp4 launch over the whole matrix."""
    idx, M, K = W.NVFP4_SPECS[args.workload]
    x_host = W.nvfp4_activations(M, K, idx)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    F.lib_handle()
    x = torch.from_numpy(x_host).to(torch.bfloat16).to(dev)
    codes = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    sf = torch.empty((M, K // 16), dtype=torch.float8_e4m3fn, device=dev)
    ts = torch.empty((M,), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        F.quantize_nvfp4(x, codes=codes, block_scales=sf, token_scales=ts, stream=stream)
        if ev is not None:
            ev[1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    k_ms = [e[0].elapsed_time(e[1]) for e in events]
    ms_step = wall * 1e3 / args.steps
    nbytes = nvfp4_bytes(M, K)
    achieved = nbytes / (np.mean(k_ms) * 1e-3) / 1e9
    traffic = None
    tfile = os.path.join(ROOT, "profiles", f"{args.workload}_traffic.json")
    if os.path.exists(tfile):
        t = json.load(open(tfile))
        if t.get("source_hash") == nvfp4_source_hash():
            traffic = t.get("bytes_per_launch")
    rec = {
        "metric": NVFP4_METRIC,
        "value": nbytes / (ms_step * 1e-3) / 1e9,
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16-in/e2m1-e4m3-out", "data": "synthetic",
        "config": {"workload": args.workload, "M": M, "K": K, "bytes_per_step": nbytes},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic, "kernel": "quantize_nvfp4"},
        "kernel_ms": float(np.mean(k_ms)), "kernel_ms_min": float(np.min(k_ms)),
        "hbm_copy_gbs": copy_bandwidth(torch),
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = nvfp4_cpu_baseline(lambda r: W.nvfp4_activations(M, K, idx, rows=r), M, K)
    print(json.dumps(rec), flush=True)


def copy_bandwidth(torch, reps=5):
    """GB/s (read + write bytes) of a plain 1 GiB device-to-device copy: the
    practical HBM ceiling next to the 8 TB/s published peak."""
    dev = torch.device("cuda:0")
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    return 2 * COPY_BYTES * reps / (a.elapsed_time(b) * 1e-3) / 1e9


def calibrate_copy(torch, steps):
    """A plain copy of COPY_BYTES (read once, written once) for the byte
    counters: FETCH_SIZE / WRITE_SIZE of this kernel against COPY_BYTES give
    the scale of the counter readings of the attention kernel."""
    dev = torch.device("cuda:0")
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(max(steps, 1)):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "copies": max(steps, 1)}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dit")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy (reference for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the attention of each (batch, head) is independent, so a multi-GPU "
              "run is N copies of this one with a head slice each; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.calibrate_copy:
        calibrate_copy(torch, args.steps)
        return
    import fmha_fwd_amd as F
    from fmha_fwd_amd import workloads as W

    if args.workload in W.NVFP4_SPECS:
        bench_nvfp4(args, torch, F, W)
        return
    spec = W.SPECS[args.workload]
    data = W.generate(spec)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    F.lib_handle()
    q = torch.from_numpy(data["q"]).to(torch.bfloat16).to(dev)
    k = torch.from_numpy(data["k"]).to(torch.bfloat16).to(dev)
    v = torch.from_numpy(data["v"]).to(torch.bfloat16).to(dev)
    stream = torch.cuda.current_stream()

    # Buffers written by the step (allocated once, outside the timed region).
    def codes_like(x, fmt):
        return torch.empty(x.shape, dtype=torch.int8 if fmt == "int8" else torch.float8_e4m3fn, device=dev)

    def scales_like(x):
        return torch.empty((x.shape[0], x.shape[2], (x.shape[1] + 63) // 64), dtype=torch.float32, device=dev)

    quant = []  # (input, fmt, codes, scales)
    for name, x in (("q", q), ("k", k), ("v", v)):
        fmt = getattr(spec, name + "_fmt")
        if fmt != "bf16":
            quant.append((name, x, fmt, codes_like(x, fmt), scales_like(x)))
    ops = {"q": q, "k": k, "v": v}
    sfs = {}
    for name, x, fmt, c, s in quant:
        ops[name] = c
        sfs["sfs_" + name] = s
    fwd_kw = dict(causal=spec.causal)
    if spec.masked:
        fwd_kw["block_mask"] = torch.from_numpy(data["block_mask"]).to(dev)
    if spec.paged:
        # A paged cache is quantised when tokens are written to it, not by the
        # attention step: quantise K/V once here and scatter the codes into the
        # page pool; the timed step quantises the other operands only.
        pt = torch.from_numpy(data["page_table"]).to(dev)
        fwd_kw.update(page_table=pt, page_size=spec.page_size, seq_len_kv=spec.S)
        per_seq, ps = pt.shape[1], spec.page_size
        for name, x, fmt, c, s in [e for e in quant if e[0] in ("k", "v")]:
            F.quantize_blocks(x, fmt, codes=c, scales=s)
            pool = torch.empty((spec.B * per_seq, ps, spec.Hkv, spec.D), dtype=c.dtype, device=dev)
            pool[pt.reshape(-1).long()] = c.reshape(spec.B * per_seq, ps, spec.Hkv, spec.D)
            ops[name] = pool
        quant = [e for e in quant if e[0] not in ("k", "v")]
    out = torch.empty((spec.B, spec.n_q, spec.Hq, spec.D), dtype=torch.bfloat16, device=dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        if len(quant) > 1:  # Q, K and V together: one launch
            F.quantize_blocks_batch([(x, fmt, c, s) for _, x, fmt, c, s in quant], stream=stream)
        for name, x, fmt, c, s in quant[:1] if len(quant) == 1 else ():
            F.quantize_blocks(x, fmt, codes=c, scales=s, stream=stream)
        kk, vv = ops["k"], ops["v"]
        if ev is not None:
            ev[1].record(stream)
        F.fwd(ops["q"], kk, vv, out=out, stream=stream, **sfs, **fwd_kw)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    with SclkSampler(torch) as sclk_sampler:
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(events[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    q_ms = [e[0].elapsed_time(e[1]) for e in events]
    f_ms = [e[1].elapsed_time(e[2]) for e in events]
    ms_step = wall * 1e3 / args.steps
    fwd_ms = float(np.mean(f_ms))
    fwd_median, fwd_min = float(np.median(f_ms)), float(np.min(f_ms))

    copy_gbs = copy_bandwidth(torch)
    pairs = pair_count(spec, data)
    flops = 4.0 * spec.D * pairs
    qk_fmt = "bf16" if spec.q_fmt == "bf16" or spec.k_fmt == "bf16" else spec.q_fmt
    pv_fmt = spec.pv_mfma
    peak = mixed_peak(qk_fmt, pv_fmt)
    achieved = flops / (fwd_ms * 1e-3) / 1e12
    quant_bytes = sum(x.numel() * 3 + s.numel() * 4 for _, x, _, _, s in quant)

    traffic, sclk_counters = None, None
    tfile = os.path.join(ROOT, "profiles", f"fwd_{spec.name}_traffic.json")
    if os.path.exists(tfile):
        t = json.load(open(tfile))
        if t.get("source_hash") == source_hash():
            traffic = t.get("bytes_per_launch")
            sclk_counters = t.get("sclk_ghz")
    sclk_live = sclk_sampler.summary()
    # sysfs reports an average that lags the shader clock: a timed region
    # shorter than SCLK_MIN_SAMPLES readings (or with idle gaps) reads low, so
    # then only the counter-derived clock of the profiles is used
    if sclk_live is not None and sclk_live["samples"] < SCLK_MIN_SAMPLES:
        sclk_live = None
    sclk = sclk_live["ghz_median"] if sclk_live else sclk_counters

    # The binding roofline of the launch: matrix-core time of its FLOPs at the
    # dtype peak against HBM time of its algorithmic bytes at the HBM peak
    # (short query ranges over a long K/V cache are HBM-bound).
    abytes = attention_bytes(spec)
    hbm_bound = abytes / (HBM_PEAK_GBS * 1e9) > flops / (peak * 1e12)
    gbs = abytes / (fwd_ms * 1e-3) / 1e9
    frac = gbs / HBM_PEAK_GBS if hbm_bound else achieved / peak
    rec = {
        "metric": METRIC,
        "value": flops / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"{qk_fmt}-qk/{pv_fmt}-pv",
        "data": "synthetic",
        "config": {"workload": spec.name, "B": spec.B, "Hq": spec.Hq, "Hkv": spec.Hkv, "Sq": spec.n_q, "Skv": spec.S,
                   "d": spec.D, "q": spec.q_fmt, "k": spec.k_fmt, "v": spec.v_fmt, "p": spec.p_fmt,
                   "causal": spec.causal, "block_sparse": spec.masked, "paged": spec.paged,
                   "unmasked_pairs": pairs, "flop_per_step": flops},
        "roofline": {"bound": "hbm" if hbm_bound else "mfma", "achieved": gbs if hbm_bound else achieved,
                     "peak": HBM_PEAK_GBS if hbm_bound else peak, "unit": "GB/s" if hbm_bound else "TFLOP/s",
                     "frac": frac, "traffic": traffic,
                     "kernel": "fmha_fwd", "algorithmic_bytes": abytes,
                     "mfma_tflops": achieved, "mfma_peak": peak, "mfma_frac": achieved / peak,
                     "frac_of_fp8_peak": achieved / PEAK["e4m3"],
                     # shader clock while the timed steps ran (sysfs, median of the samples; else
                     # the counter record's), and the fraction of the peak at that clock (the
                     # published peaks assume 2.4 GHz)
                     "sclk_ghz_measured": sclk,
                     "sclk_sysfs": sclk_live, "sclk_ghz_counters": sclk_counters,
                     "frac_at_measured_sclk": None if sclk is None or hbm_bound
                     else achieved / (peak * min(sclk, 2.4) / 2.4)},
        "fwd_ms": fwd_ms,
        "fwd_ms_median": fwd_median,
        "fwd_ms_min": fwd_min,
        "fwd_tflops_at_min": flops / (fwd_min * 1e-3) / 1e12,
        "quantize_ms": float(np.mean(q_ms)) if quant else 0.0,
        "quantize_gbs": (quant_bytes / (np.mean(q_ms) * 1e-3) / 1e9) if quant else None,
        "quantize_frac_of_hbm_peak": (quant_bytes / (np.mean(q_ms) * 1e-3) / 1e9 / HBM_PEAK_GBS) if quant else None,
        "hbm_copy_gbs": copy_gbs,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(spec, data)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
