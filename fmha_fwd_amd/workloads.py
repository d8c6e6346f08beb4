"""Seeded synthetic inputs shaped like the pages' workloads.

Input generation only: no step of the attention method lives here, so the HIP
path and the CPU oracle can both draw from it.  Every draw comes from numpy's
PCG64 with ``SeedSequence(2711, spawn_key=(config index,))`` spawned into five
child streams used in the order [Q, K, V, structure, mask]; normal draws are
float32 rounded to bf16 (torch's round-to-nearest-even cast).

Configurations (d = 128 throughout; `small_spec` can set d = 192):
  tiny    B=1 H=2  S=256    all bf16, unscaled, non-causal
  dit_i8  B=1 H=24 S=4096   int8 Q/K + E4M3 V with 64-token block scales,
                            2% outlier channels (3 per head) of Q and K x20
  dit     B=1 H=40 S=32760  bf16 Q/K, E4M3 V with 64-token block scales
  gqa     B=2 Hq=64 Hkv=8 S=8192, E4M3 Q/K/V with block scales, causal,
                            per-head standard deviation ~ U(0.5, 2)
  sparse  B=4 H=32 S=16384  bf16 Q, E4M3 K/V in 16-token pages (random page
                            table), Q64 x KV256 block mask with 16 of 64 key
                            blocks active per query block (diagonal always)
  gqa_chunk  the gqa inputs with only the last 256 query positions (a causal
             prefill chunk against 8192 keys)
  sparse_contig  the sparse inputs with K/V contiguous (the cost of paging)
  sparse_dense   the same inputs with contiguous K/V and no mask (the dense
                 attention the block mask thins out)
  dit_i8_d192, gqa_d192, dit_d192, sparse_d192  the dit_i8, gqa, dit and
             sparse shapes and formats at head dim 192 (own spawn keys 9, 10,
             11 and 12)

Per-token NVFP4 quantisation (activation matrices [tokens, hidden], bf16):
  nvfp4   M=16384 tokens x K=8192 channels (a 16k-token prefill batch of an
          8192-wide model), spawn key 8; rows N(0, 1) times a per-token
          magnitude exp(U(-3, 3)), and 0.5% of the channels (41) x20 outliers
          shared by every token, as in LLM activations
"""
from dataclasses import dataclass

import numpy as np

SEED = 2711


@dataclass(frozen=True)
class Spec:
    name: str
    index: int
    B: int
    Hq: int
    Hkv: int
    S: int
    q_fmt: str          # "bf16" | "int8" | "e4m3"
    k_fmt: str
    v_fmt: str
    causal: bool = False
    masked: bool = False
    paged: bool = False
    page_size: int = 16
    D: int = 128
    sq: int = 0         # query rows when fewer than the S keys: the last sq positions (0 = S)

    @property
    def n_q(self):
        return self.sq or self.S

    @property
    def q_scaled(self):
        return self.q_fmt != "bf16"

    @property
    def k_scaled(self):
        return self.k_fmt != "bf16"

    @property
    def v_scaled(self):
        return self.v_fmt != "bf16"

    @property
    def p_fmt(self):
        """Format P is requantized to before the PV product: bf16 for a bf16
        V, E4M3 for an E4M3 or an int8 V."""
        return "bf16" if self.v_fmt == "bf16" else "e4m3"

    @property
    def pv_mfma(self):
        """Operand format of the matrix-core PV product: an int8 V meets the
        E4M3 P in fp16 (both widen exactly), the others use P's format."""
        return "f16" if self.v_fmt == "int8" else self.p_fmt

    def pairs(self):
        """Unmasked (query, key) pairs: the FLOP count is 4 * D * pairs.
        Causal is bottom-right aligned: query i of n_q sees keys <= i + S - n_q."""
        nq = self.n_q
        per_head = nq * self.S
        if self.causal:
            per_head = nq * (self.S - nq) + nq * (nq + 1) // 2
        if self.masked:
            per_head = None
        if per_head is None:
            return None
        return self.B * self.Hq * per_head


SPECS = {
    "tiny": Spec("tiny", 0, 1, 2, 2, 256, "bf16", "bf16", "bf16"),
    "dit_i8": Spec("dit_i8", 1, 1, 24, 24, 4096, "int8", "int8", "e4m3"),
    "dit": Spec("dit", 2, 1, 40, 40, 32760, "bf16", "bf16", "e4m3"),
    "gqa": Spec("gqa", 3, 2, 64, 8, 8192, "e4m3", "e4m3", "e4m3", causal=True),
    "sparse": Spec("sparse", 4, 4, 32, 32, 16384, "bf16", "e4m3", "e4m3", masked=True, paged=True),
    # a prefill chunk: the last 256 positions of the gqa sequence against all of its keys
    "gqa_chunk": Spec("gqa_chunk", 5, 2, 64, 8, 8192, "e4m3", "e4m3", "e4m3", causal=True, sq=256),
    # 16 new positions per sequence (a short prefill step) for 64 sequences
    "gqa_step": Spec("gqa_step", 6, 64, 64, 8, 8192, "e4m3", "e4m3", "e4m3", causal=True, sq=16),
    # the same step with four query heads per KV head (32 / 8)
    "gqa4_step": Spec("gqa4_step", 7, 64, 32, 8, 8192, "e4m3", "e4m3", "e4m3", causal=True, sq=16),
    # head dim 192 (index 8 is the NVFP4 activations' spawn key)
    "dit_i8_d192": Spec("dit_i8_d192", 9, 1, 24, 24, 4096, "int8", "int8", "e4m3", D=192),
    "gqa_d192": Spec("gqa_d192", 10, 2, 64, 8, 8192, "e4m3", "e4m3", "e4m3", causal=True, D=192),
    "dit_d192": Spec("dit_d192", 11, 1, 40, 40, 32760, "bf16", "bf16", "e4m3", D=192),
    "sparse_d192": Spec("sparse_d192", 12, 4, 32, 32, 16384, "bf16", "e4m3", "e4m3", masked=True, paged=True, D=192),
    # the gqa shape with K in E4M3 and V in int8 (per-64-token scales, amax/127)
    "gqa_vi8": Spec("gqa_vi8", 13, 2, 64, 8, 8192, "e4m3", "e4m3", "int8", causal=True),
    # the sparse inputs (same spawn key: same Q, K, V and mask) with K/V contiguous instead of paged
    "sparse_contig": Spec("sparse_contig", 4, 4, 32, 32, 16384, "bf16", "e4m3", "e4m3", masked=True),
    # ... and with no block mask at all: the dense attention the mask thins out
    "sparse_dense": Spec("sparse_dense", 4, 4, 32, 32, 16384, "bf16", "e4m3", "e4m3"),
}


def streams(spec_index):
    ss = np.random.SeedSequence(SEED, spawn_key=(spec_index,))
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(5)]


def to_bf16_values(x):
    """float32 array -> float32 array of the nearest bf16 values (RNE)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def _normal(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32)


def generate(spec):
    """Host inputs of one configuration.

    Returns a dict with q, k, v (float32 arrays holding bf16 values, shapes
    [B, S, H, D], K/V in logical token order) and, where the configuration
    has them, page_table (int32 [B, S/page]) and block_mask (uint8
    [B, Hq, S/64, S/256]).
    """
    rq, rk, rv, rs, rm = streams(spec.index)
    B, S, D = spec.B, spec.S, spec.D
    q = _normal(rq, (B, S, spec.Hq, D))
    k = _normal(rk, (B, S, spec.Hkv, D))
    v = _normal(rv, (B, S, spec.Hkv, D))
    out = {}
    if spec.name.startswith("dit_i8"):
        # 2% of the 128 channels (3 per head) of Q and of K carry x20 outliers
        n_out = int(round(0.02 * D))
        for x, H in ((q, spec.Hq), (k, spec.Hkv)):
            for h in range(H):
                ch = rs.choice(D, size=n_out, replace=False)
                x[:, :, h, ch] *= np.float32(20.0)
    if spec.name.startswith("gqa"):
        sig_q = rs.uniform(0.5, 2.0, spec.Hq).astype(np.float32)
        sig_k = rs.uniform(0.5, 2.0, spec.Hkv).astype(np.float32)
        sig_v = rs.uniform(0.5, 2.0, spec.Hkv).astype(np.float32)
        q *= sig_q[None, None, :, None]
        k *= sig_k[None, None, :, None]
        v *= sig_v[None, None, :, None]
    if spec.paged:
        per_seq = -(-S // spec.page_size)
        perm = rs.permutation(B * per_seq).astype(np.int32)
        out["page_table"] = perm.reshape(B, per_seq)
    if spec.masked:
        nqb, nkb = -(-S // 64), -(-S // 256)
        active = max(1, nkb // 4)
        mask = np.zeros((B, spec.Hq, nqb, nkb), dtype=np.uint8)
        for b in range(B):
            for h in range(spec.Hq):
                for qb in range(nqb):
                    diag = min(qb // 4, nkb - 1)
                    others = np.delete(np.arange(nkb), diag)
                    pick = rm.choice(others, size=active - 1, replace=False)
                    mask[b, h, qb, diag] = 1
                    mask[b, h, qb, pick] = 1
        out["block_mask"] = mask
    if spec.n_q != S:
        q = q[:, S - spec.n_q:]
    out["q"] = to_bf16_values(q)
    out["k"] = to_bf16_values(k)
    out["v"] = to_bf16_values(v)
    return out


def random_block_mask(B, Hq, Sq, Skv, block_kv, density, stream, empty_q_blocks=()):
    """uint8 [B, Hq, ceil(Sq/64), ceil(Skv/block_kv)] block mask with each
    block active with probability `density` (seeded by `stream`); the query
    blocks listed in `empty_q_blocks` see no key at all."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(SEED, spawn_key=(1000 + stream,))))
    nqb, nkb = -(-Sq // 64), -(-Skv // block_kv)
    mask = (rng.random((B, Hq, nqb, nkb)) < density).astype(np.uint8)
    for qb in empty_q_blocks:
        mask[:, :, qb] = 0
    return mask


def small_spec(base, S, B=None, Hq=None, Hkv=None, **kw):
    """A reduced-size variant of a configuration (same formats and options)."""
    s = SPECS[base]
    return Spec(s.name + f"_S{S}", s.index, B or s.B, Hq or s.Hq, Hkv or s.Hkv, S, s.q_fmt, s.k_fmt, s.v_fmt,
                kw.get("causal", s.causal), kw.get("masked", s.masked), kw.get("paged", s.paged),
                kw.get("page_size", s.page_size), D=kw.get("D", s.D), sq=kw.get("sq", 0))


NVFP4_SPECS = {"nvfp4": (8, 16384, 8192)}  # name: (spawn key, M tokens, K channels)


def nvfp4_activations(M, K, index=8, rows=None):
    """bf16 activation values [M, K] (float32 array) for the per-token NVFP4
    quantiser: N(0, 1) rows scaled by exp(U(-3, 3)) per token, 0.5% of the
    channels x20.  Each group of 256 rows draws from a stream of its own, so
    `rows` (an index array) returns those rows of the same matrix while
    drawing only the groups that hold them."""
    _, _, _, rs, _ = streams(index)
    mag = np.exp(rs.uniform(-3.0, 3.0, M)).astype(np.float32)
    n_out = max(1, int(round(0.005 * K)))
    ch = rs.choice(K, size=n_out, replace=False)
    idx = np.arange(M) if rows is None else np.asarray(rows, dtype=np.int64)
    x = np.empty((len(idx), K), dtype=np.float32)
    for grp in np.unique(idx // 256):
        ss = np.random.SeedSequence(SEED, spawn_key=(index, 1, int(grp)))
        n = min(256, M - 256 * int(grp))
        block = np.random.Generator(np.random.PCG64(ss)).standard_normal((n, K), dtype=np.float32)
        sel = np.nonzero(idx // 256 == grp)[0]
        x[sel] = block[idx[sel] - 256 * int(grp)]
    x *= mag[idx][:, None]
    x[:, ch] *= np.float32(20.0)
    return to_bf16_values(x)


SWEEP_BASES = ("tiny", "dit", "dit_i8", "gqa", "sparse")  # the five format combinations


def sweep_case(i):
    """Configuration i of a seeded random sweep: one of the five format
    combinations, head dim 128 or 192, B 1-2, 1-2 KV heads with 1-8 query
    heads each, 1-320 queries against 1-700 keys (ragged, either longer),
    causal or not, and independently a block mask (64-query rows, key blocks
    of 64-512, density 0.2-0.9, sometimes a query block with no key) and paged
    K/V (pages of 16-256 tokens, a random page table over a pool with spare
    pages).  Values are N(0, 1) scaled per head by U(0.5, 2), as bf16.

    Returns (spec, data, mask_block_kv); data as `generate` returns it, with
    q [B, Sq, Hq, D] and k, v [B, Skv, Hkv, D]."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(SEED, spawn_key=(2000 + i,))))
    base = SPECS[SWEEP_BASES[int(rng.integers(len(SWEEP_BASES)))]]
    D = int(rng.choice([128, 192]))
    B = int(rng.integers(1, 3))
    Hkv = int(rng.integers(1, 3))
    group = int(rng.choice([1, 2, 4] if Hkv > 1 else [1, 2, 4, 8]))
    Hq = Hkv * group
    Skv = int(rng.integers(1, 701))
    Sq = Skv if rng.random() < 0.25 else int(rng.integers(1, 321))
    causal = bool(rng.random() < 0.5)
    masked = bool(rng.random() < 0.35)
    paged = bool(rng.random() < 0.35)
    page_size = int(rng.choice([16, 32, 64, 128, 256]))
    kvb = int(rng.choice([64, 128, 256, 512]))
    spec = Spec(f"sweep{i}_{base.name}", 100 + i, B, Hq, Hkv, Skv, base.q_fmt, base.k_fmt, base.v_fmt,
                causal, masked, paged, page_size, D=D, sq=Sq if Sq != Skv else 0)
    sig = [rng.uniform(0.5, 2.0, H).astype(np.float32)[None, None, :, None] for H in (Hq, Hkv, Hkv)]
    q = rng.standard_normal((B, Sq, Hq, D), dtype=np.float32) * sig[0]
    k = rng.standard_normal((B, Skv, Hkv, D), dtype=np.float32) * sig[1]
    v = rng.standard_normal((B, Skv, Hkv, D), dtype=np.float32) * sig[2]
    data = {"q": to_bf16_values(q), "k": to_bf16_values(k), "v": to_bf16_values(v)}
    if paged:
        per_seq = -(-Skv // page_size)
        pool = B * per_seq + int(rng.integers(0, 4))
        data["page_table"] = rng.permutation(pool)[:B * per_seq].astype(np.int32).reshape(B, per_seq)
    if masked:
        nqb, nkb = -(-Sq // 64), -(-Skv // kvb)
        mask = (rng.random((B, Hq, nqb, nkb)) < rng.uniform(0.2, 0.9)).astype(np.uint8)
        if nqb > 1 and rng.random() < 0.5:
            mask[:, :, int(rng.integers(nqb))] = 0
        data["block_mask"] = mask
    return spec, data, kvb

