// Fused attention forward for gfx950: block-scaled int8 / E4M3 / bf16 Q and
// K, E4M3 or bf16 V and P (or an int8 V with an E4M3 P), online softmax with
// lazy rescaling, bf16 output (or E4M3 with a per-head output scale).
//
// Method sources (FlashInfer pull-request write-ups):
//  * #2711 page "FlashInfer의 DiT 최적화: SageAttention과 Int8/FP8 혼합 정밀도
//    커널 도입 분석", 코드 분석 2: per-block Q/K/P/V scale factors that undo
//    the quantisation after BMM1 (QK^T) and BMM2 (PV); 코드 분석 1: Q, K, V
//    formats chosen independently; 왜 이게 좋은 최적화인가? 3: K in fp8 with
//    V in int8 as one such combination.
//  * #5900 page "Blackwell 아키텍처를 위한 FlashInfer의 FP8/BF16 혼합 정밀도
//    Attention 최적화 분석", 코드 분석 3: lazy correction (O is rescaled only
//    when the row maximum grows by 2^8); 코드 분석 1: QK in bf16 or fp8 with an
//    fp8 P, head dim 128, 16-bit output.
//  * #4474 page "FlashInfer의 PrimTS를 활용한 고성능 Block-Sparse Attention
//    최적화", 코드 분석 1-2: Q64 x KV256 block-sparse masks, paged K/V.
//
// Design for CDNA4 (not a translation of the pages' Hopper/Blackwell kernels):
//  * One workgroup = NW wavefronts x 32 queries of one (batch, head), or the
//    same 32 queries of NW query heads that share a KV head (grouped-query
//    head packing).  K and V stream through LDS in 64-key sub-tiles,
//    double-buffered; the Q tile stays in VGPRs for the whole key loop.
//  * The score tile is computed transposed, S^T = K Q^T, on 32x32 MFMA tiles,
//    so every lane owns one query row: the row max / sum are in-register
//    reductions plus one exchange with lane l ^ 32, and the per-row lazy
//    rescale factor multiplies the lane's own O^T registers.
//  * Keys are permuted inside a 32-key MFMA tile (sigma below) so that the
//    S^T accumulator of lane group g holds 16 consecutive keys; those P values
//    are packed in place into the B operand of O^T += V^T P^T, and V^T is read
//    from LDS with the gfx950 transposing loads (ds_read_b64_tr_b8 / _b16).
//  * The lazy decision is per row and per 64-key sub-tile, branch-free: rows
//    that do not trigger take factor 1.
//  * V's per-64-token scale is applied after BMM2: O is kept in units of the
//    current sub-tile's V scale, so one multiply per O element folds the
//    lazy factor and the change of scale, and the PV MFMA accumulates codes
//    x codes into O (or, when the scales span more than 2^64, each partial
//    product is scaled into O).
//  * Row sums of an E4M3 P come from one more MFMA (a 0/1 matrix times the P
//    operand) instead of VALU conversions and additions.
//  * An int8 V meets the E4M3 P on the fp16 MFMA: no 8-bit product takes an
//    int8 and an E4M3 operand, and both code sets are fp16 values, so the
//    widened products are the exact code products.
//  * sfs_p cancels between numerator and denominator, so it enters only the
//    quantisation of P (exp2 argument shifted by log2 sfs_p).
#include <type_traits>

#include "device_common.h"
#include "fmha_internal.h"

namespace fmha {
namespace {

constexpr int kSub = 64;  // keys per sub-tile: lazy-decision and V-scale unit
#ifndef FMHA_DENSE_WAVES
#define FMHA_DENSE_WAVES 4
#endif
constexpr int kDenseWaves = FMHA_DENSE_WAVES;  // wavefronts (x 32 queries) per dense workgroup
// Wavefronts per SIMD the register budget is cut for (512 / n VGPRs per
// lane): three where the loop fits 168 registers (E4M3 or int8 QK, whose Q
// operand takes 16 registers), two otherwise.
#ifndef FMHA_WAVES_PER_EU_8BIT
#define FMHA_WAVES_PER_EU_8BIT 3
#endif
#ifndef FMHA_WAVES_PER_EU_BF16
#define FMHA_WAVES_PER_EU_BF16 2
#endif
#ifndef FMHA_ROW_PACK
#define FMHA_ROW_PACK 1  // 0: at most one head per wave
#endif
#ifndef FMHA_ROW_PACK_NW2
#define FMHA_ROW_PACK_NW2 1  // 0: no two-wave workgroups for small groups
#endif
#ifndef FMHA_HEAD_PACK
#define FMHA_HEAD_PACK 1  // 0: never pack query heads into one workgroup
#endif
// 1: the per-row O factor of the fast V-reference path is applied to one
// d-tile right before that d-tile's PV product is issued, so the multiplies
// of the next d-tile run while the matrix core works on the previous one
// (0: all of O is rescaled in the softmax, before the first PV product).
#ifndef FMHA_PV_INTERLEAVE
#define FMHA_PV_INTERLEAVE 1
#endif
constexpr float kInf = __builtin_huge_valf();

// Key held by row m of a 32-key MFMA tile: lane group g of the S^T result
// then owns keys 16g .. 16g + 15 in its 16 accumulator registers.
__device__ __forceinline__ int sigma(int m) {
  return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3);
}

// A register of no particular value (no instruction): the low half of a
// packed P word is written first and the high half second, so the initial
// contents never reach a result.
__device__ __forceinline__ int any_vgpr() {
  int v;
  asm volatile("" : "=v"(v));
  return v;
}

// f(integral_constant<int, I>) for I = B .. E-1, unrolled at compile time.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Keys per LDS tile of the dense 8-bit-QK instances: 64 (one sub-tile per
// barrier) or 128 (two sub-tiles per barrier, copied one tile ahead; twice
// the LDS, so two wavefronts per SIMD instead of three).
#ifndef FMHA_KV_TILE_8BIT
#define FMHA_KV_TILE_8BIT 64
#endif

template <int QF_, int KF_, int VF_, bool QS_, bool KS_, bool VS_, bool MASKED_, bool PAGED_, int NW_,
          bool RP_ = false, int D_ = 128, int KT_ = 64>
struct Cfg {
  static constexpr int QF = QF_, KF = KF_, VF = VF_, NW = NW_;
  static constexpr int KT = KT_, SUB = KT_ / 64;  // keys per LDS tile, sub-tiles per tile
  static_assert(KT_ == 64 || ((KT_ == 128 || KT_ == 256) && !MASKED_ && !PAGED_ && !RP_), "larger tiles: dense only");
  static constexpr int D = D_, ND = D / 32;  // head dim; 32-row d-tiles of O^T
  static constexpr bool QS = QS_, KS = KS_, VS = VS_, MASKED = MASKED_, PAGED = PAGED_;
  // RP: heads packed inside a wave (fewer than 32 rows per head), so a
  // lane's head, Q scale and P scale are its own (two more live registers)
  static constexpr bool RP = RP_;
  static constexpr int MT = QF;                                  // QK operand format
  // (head dim 192 with a block mask, paged K/V or E4M3 K widened for a bf16
  // Q: one wavefront per SIMD, all 512 registers; their LDS tiles allow no
  // more than four wavefronts per CU anyway)
  static constexpr int WPE = D != 128 && (MASKED || PAGED || (MT == FMT_BF16 && KF == FMT_E4M3))
                                 ? 1
                             : MT == FMT_BF16 || MASKED || PAGED || RP || D != 128 || KT_ != 64
                                 ? FMHA_WAVES_PER_EU_BF16
                                 : FMHA_WAVES_PER_EU_8BIT;
  // E4M3 K under a bf16 Q stays E4M3 in LDS and is widened (exactly) to bf16
  // as each MFMA operand is read.
  static constexpr bool WIDEN = MT == FMT_BF16 && KF == FMT_E4M3;
  // P in E4M3 (row sums on the matrix core, 8-bit V tiles) for an E4M3 or an
  // int8 V; an int8 V meets P on the fp16 product (both widen exactly)
  static constexpr bool P8 = VF != FMT_BF16;
  static constexpr int KROW = KF == FMT_BF16 ? 2 * D : D;        // bytes per K row (HBM and LDS)
  static constexpr int VROW = VF == FMT_BF16 ? 2 * D : D;
  // LDS rows are padded so that every lane reads at a fixed offset from its
  // own base address without bank conflicts (64 banks x 4 bytes = 16 chunks
  // of 16 bytes): K rows advance by an odd number of chunks (17, 9 or 13),
  // so the 16 consecutive rows of one MFMA-operand read land in 16 distinct
  // chunks; 8-bit V rows advance by an even number of chunks not divisible by
  // 4 (10 or 14), so the 8 rows of a transposing read land on 8 distinct even
  // chunks and their neighbours (chunk c + 1) on the odd ones.
  static constexpr int KP = KROW + 16, VP = VF == FMT_BF16 ? VROW + 16 : VROW + 32;
  static constexpr int K_BUF = KT * KP, V_BUF = KT * VP;
  static constexpr int LDS_BYTES = 2 * (K_BUF + V_BUF);
  static constexpr int NT = NW * 64;
  static constexpr int K_CPR = KROW / 16, KP_CPR = KP / 16;      // 16-byte chunks per row
  static constexpr int V_CPR = VROW / 16, VP_CPR = VP / 16;
  static constexpr int K_DMA_OPS = K_BUF / 1024;                 // 1 KB per wave-wide DMA
  static constexpr int V_DMA_OPS = V_BUF / 1024;
  static_assert(K_BUF % 1024 == 0 && V_BUF % 1024 == 0, "DMA granularity");
  static_assert(!(KF == FMT_E4M3 && QF == FMT_INT8), "unsupported");
  static_assert(QF == KF || (QF == FMT_BF16 && KF == FMT_E4M3), "unsupported");
  static_assert(VF != FMT_INT8 || (QF == FMT_E4M3 && D == 128 && VS_), "int8 V: E4M3 Q and K, head dim 128");
};

// Q operand registers of one lane (query l % 32, contraction slice of group g).
template <int MT, int D> struct QRegs;
template <int D> struct QRegs<FMT_BF16, D> { v8bf r[D / 16]; };  // d = (D/2)g + 8t .. +8
template <int D> struct QRegs<FMT_E4M3, D> { v8i r[D / 64]; };   // bytes 64t + 32g .. +32
template <int D> struct QRegs<FMT_INT8, D> { v4i r[D / 32]; };   // bytes 32t + 16g .. +16

template <int MT> struct SAcc { v16f r[2]; };
template <> struct SAcc<FMT_INT8> { v16i r[2]; };

// Workgroup id -> logical tile.  The dispatcher places workgroup i on XCD
// i % 8; each XCD receives a contiguous range of logical tiles, so the
// workgroups resident on one XCD work on the same head at the same time and
// share its K/V stream in that XCD's L2.
__device__ __forceinline__ int xcd_remap(int i, int total) {
  const int r = total % 8, per = total / 8;
  const int x = i % 8, j = i / 8;
  return x * per + min(x, r) + j;
}

// Persistent launch (build option, off by default): a grid of the resident
// workgroup slots, each taking tiles blockIdx.x, blockIdx.x + gridDim.x, ...
// (gridDim.x a multiple of 8, so a workgroup's tiles stay in its XCD's range).
#ifndef FMHA_PERSISTENT
#define FMHA_PERSISTENT 0
#endif
#if FMHA_PERSISTENT
#define FMHA_END_TILE goto tile_end
#else
#define FMHA_END_TILE return
#endif

template <class C>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(C::WPE))) void fwd_kernel(FwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
#if FMHA_PERSISTENT
  for (int it = blockIdx.x; it < a.tiles; it += gridDim.x) {
  const int lin = xcd_remap(it, a.tiles);
#else
  {
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
#endif
  {
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int g = lane >> 5;
  const int m32 = lane & 31;

  // ---- which (batch, head, query tile) this workgroup owns
  // Either NW x 32 consecutive queries of one head, or (head packing, for
  // grouped-query attention with short or causal query ranges) the same R
  // queries of NW * 32 / R query heads that share one KV head, R / 32 of a
  // wave's rows per head: every row then needs the same keys, and K/V tiles
  // serve all those heads at once.  Rows are independent, so a lane's head
  // and query only change where its row is loaded, scaled and stored.
  const int rows = C::MASKED || !a.pack_rows ? 0 : (C::RP ? a.pack_rows : 32);  // R (0: no packing)
  const bool pack = rows > 0;
  const int qtile = pack ? rows : 32 * C::NW;
  const int nqt = (a.Sq + qtile - 1) / qtile;
  int qt = lin % nqt;
  if (a.causal) qt = nqt - 1 - qt;  // longest causal rows first
  const int rest = lin / nqt;
  int hq, b, hk;
  int qi;  // this lane's query row
  if (C::RP) {
    const int hpw = 32 / rows;                 // heads per wave
    const int gpw = a.group / (C::NW * hpw);   // workgroups per KV head and query tile
    const int bhk = rest / gpw;
    hk = bhk % a.Hkv;
    hq = hk * a.group + (rest % gpw) * (C::NW * hpw) + wave * hpw + m32 / rows;
    b = bhk / a.Hkv;
    qi = qt * qtile + m32 % rows;
  } else if (pack) {
    const int gpw = a.group / C::NW;
    const int bhk = rest / gpw;
    hk = bhk % a.Hkv;
    hq = hk * a.group + (rest % gpw) * C::NW + wave;
    b = bhk / a.Hkv;
    qi = qt * qtile + m32;
  } else {
    hq = rest % a.Hq;
    b = rest / a.Hq;
    hk = hq / a.group;
    qi = qt * qtile + 32 * wave + m32;
  }
  const int q0 = qt * qtile;
  const int causal_off = a.Skv - a.Sq;     // key j visible iff j <= i + causal_off

  // ---- key range of the workgroup; sub-tiles needing per-pair masks
  int kv_end = a.Skv;
  if (a.causal) {
    const int qlast = min(q0 + qtile, a.Sq) - 1;
    kv_end = min(kv_end, max(qlast + causal_off + 1, 0));
  }
  const int n_sub = (kv_end + kSub - 1) / kSub;
  // sub-tiles [0, full_end) are valid for every (query, key) pair of the workgroup
  int full_keys = a.Skv;
  if (a.causal) full_keys = min(full_keys, max(q0 + causal_off + 1, 0));
  const int full_end = full_keys / kSub;

  const uint8_t* mask_row = nullptr;
  if (C::MASKED) mask_row = a.mask + (int64_t)b * a.m_sb + (int64_t)hq * a.m_sh + (int64_t)(q0 / 64) * a.m_sqb;
  // Block mask: the active key blocks of this workgroup's query block, 64
  // blocks at a time, as a wave-uniform bit mask (one mask byte per lane,
  // then a ballot), so skipping inactive blocks costs no memory round trip.
  const int kvsub = C::MASKED ? a.mask_kv_sub : 1;  // sub-tiles per mask key block
  const int n_mkb = C::MASKED ? (a.Skv + kSub * kvsub - 1) / (kSub * kvsub) : 0;
  uint64_t mbits = 0;
  int mb_base = -64;  // mbits bit i: mask key block mb_base + i is active
  // First sub-tile at or after t whose mask block is active (n_sub if none).
  auto next_sub = [&](int t) {
    if constexpr (C::MASKED) {
      if (t >= n_sub) return n_sub;
      int mb = a.mask_kv_shift >= 0 ? t >> a.mask_kv_shift : t / kvsub;
      while (mb * kvsub < n_sub) {
        if (mb - mb_base >= 64) {
          mb_base = mb;
          const int i = mb + lane;
          mbits = __ballot(i < n_mkb && mask_row[i] != 0);
        }
        const uint64_t ahead = mbits >> (mb - mb_base);
        if (ahead != 0) {
          mb += __builtin_ctzll(ahead);
          const int r = max(t, mb * kvsub);
          return r < n_sub ? r : n_sub;
        }
        mb = mb_base + 64;
      }
      return n_sub;
    }
    return t;
  };

  // ---- HBM -> LDS staging
  const uint8_t* kbase = a.k + (int64_t)hk * a.k_sh;
  const uint8_t* vbase = a.v + (int64_t)hk * a.v_sh;
  const int32_t* pt_row = C::PAGED ? a.page_table + (int64_t)b * a.pt_sb : nullptr;
  if (!C::PAGED) {
    kbase += (int64_t)b * a.k_sb;
    vbase += (int64_t)b * a.v_sb;
  }
  const int page_shift = C::PAGED ? __builtin_ctz((unsigned)a.page_size) : 0;
  // LDS pointers stay in the LDS address space (no generic-pointer casts).
  lds_u8* const kbuf0 = (lds_u8*)smem;
  lds_u8* const vbuf0 = kbuf0 + 2 * C::K_BUF;
  // Copy j of a sub-tile (1 KB, one wave-wide DMA operation) is issued by
  // wave j % NW as its slot j / NW; contiguous K/V skip the slots past the
  // last copy (a wave-uniform branch), paged K/V repeat the last copy there
  // (identical bytes to the same place).  Per-lane
  // source offsets within a tile are fixed; contiguous K/V go through a
  // buffer resource whose range ends at the last token, so rows past the end
  // of the sequence read as zeros.  K rows are stored in MFMA row order: LDS
  // row 32T + m holds key 32T + sigma(m).
  //
  // Paged K/V (pages of 16 tokens or more, so at most four per sub-tile):
  // the page numbers of a sub-tile are read once, one table entry per lane
  // and a sub-tile ahead; each copy then takes its page from the lane that
  // holds it (ds_bpermute).  Every lane keeps, per slot, its page slot within
  // the sub-tile (2 bits) and its byte offset inside the page.  In the
  // sub-tile that crosses the end of the sequence, rows past the end read
  // the last token instead.
  constexpr int KSL = (C::K_DMA_OPS + C::NW - 1) / C::NW;
  constexpr int VSL = (C::V_DMA_OPS + C::NW - 1) / C::NW;
  static_assert(2 * (KSL + VSL) <= 64, "page-slot bits");
  uint32_t k_src[KSL], v_src[VSL];  // contiguous: byte offset in the tile; paged: in the page
  uint64_t pslot_bits = 0;          // paged: 2-bit page slot of every K and V slot
  const int tshift = min(page_shift, 6);  // rows of one sub-tile per page: 1 << tshift
  const int tmask = (1 << tshift) - 1;
  // Row of the sub-tile (a key offset) and byte column of this lane in copy j.
  auto k_copy_row = [&](int j, int& ch) {
    const int cid = j * 64 + lane;
    const int row = cid / C::KP_CPR;
    ch = cid % C::KP_CPR;
    ch = ch < C::K_CPR ? ch : 0;  // the pad chunk: any valid bytes
    return 32 * (row >> 5) + sigma(row & 31);
  };
  auto v_copy_row = [&](int j, int& ch) {
    const int cid = j * 64 + lane;
    ch = cid % C::VP_CPR;
    ch = ch < C::V_CPR ? ch : 0;
    return cid / C::VP_CPR;
  };
#pragma unroll
  for (int sl = 0; sl < KSL; ++sl) {
    int ch;
    const int row = k_copy_row(min(wave + sl * C::NW, C::K_DMA_OPS - 1), ch);
    if (!C::PAGED) {
      k_src[sl] = (uint32_t)(row * a.k_ss) + ch * 16;
    } else {
      k_src[sl] = (uint32_t)((row & tmask) * a.k_ss) + ch * 16;
      pslot_bits |= (uint64_t)(row >> tshift) << (2 * sl);
    }
  }
#pragma unroll
  for (int sl = 0; sl < VSL; ++sl) {
    int ch;
    const int row = v_copy_row(min(wave + sl * C::NW, C::V_DMA_OPS - 1), ch);
    if (!C::PAGED) {
      v_src[sl] = (uint32_t)(row * a.v_ss) + ch * 16;
    } else {
      v_src[sl] = (uint32_t)((row & tmask) * a.v_ss) + ch * 16;
      pslot_bits |= (uint64_t)(row >> tshift) << (2 * (KSL + sl));
    }
  }
  // Page numbers of sub-tile t: entry i of the sub-tile in lane i (i < 4).
  // The table entry is checked where it is used (page_addr), a sub-tile
  // later: a check here would wait for this load and every copy before it.
  auto load_pages = [&](int t) {
    if constexpr (!C::PAGED) return 0;
    const int first = (t * kSub) >> page_shift, last = (a.Skv - 1) >> page_shift;
    return pt_row[min(first + (lane & 3), last)];
  };
  auto tile_rsrc = [&](const uint8_t* base, int64_t ss, int kv0) {
    const uint64_t rem = (uint64_t)(a.Skv - kv0) * (uint64_t)ss;
    const int nrec = rem > 0x7FFFFFFFull ? 0x7FFFFFFF : (int)rem;
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base + (int64_t)kv0 * ss), 0, nrec, 0x00020000);
  };
  // When the whole sequence of this (batch, KV head) spans under 2^31 bytes,
  // one resource covers it and a tile's start goes into the scalar offset
  // (which the range check counts like the rest of the offset); otherwise
  // every tile gets a resource of its own.
  const bool kv_whole = !C::PAGED && a.kv_whole_rsrc;
  const auto k_rs_all = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, 0, kv_whole ? a.Skv * (int)a.k_ss : 0, 0x00020000);
  const auto v_rs_all = __builtin_amdgcn_make_buffer_rsrc((void*)vbase, 0, kv_whole ? a.Skv * (int)a.v_ss : 0, 0x00020000);
  // Paged: address of the first row of sub-tile t (first key kv0) in page
  // slot lane & 3, whose page number this lane holds; one 64-bit product per
  // sub-tile and tensor, shared by every copy through ds_bpermute.
  auto page_addr = [&](const uint8_t* base, int64_t sb, int64_t ss, int kv0, int page) {
    page = (unsigned)page < (unsigned)a.num_pages ? page : 0;  // outside the pool: page 0
    const int64_t in_page = (int64_t)(kv0 & (a.page_size - 1)) * ss;  // pages longer than a sub-tile
    return (uint64_t)(base + in_page) + (uint64_t)(uint32_t)page * (uint64_t)sb;
  };
  // Source of one paged copy (slot bit field `idx`, in-page offset `off`)
  // from the page addresses `pa`.  In the last sub-tile a row past the end
  // takes the last token's page slot and offset (row `rl` of the sub-tile).
  auto paged_src = [&](uint64_t pa, int64_t ss, int idx, uint32_t off, bool past_end, int rl, int ch) {
    int ps = (int)(pslot_bits >> (2 * idx)) & 3;
    if (past_end) {
      ps = rl >> tshift;
      off = (uint32_t)((rl & tmask) * ss) + ch * 16;
    }
    const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_bpermute(ps << 2, (int)(uint32_t)pa);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute(ps << 2, (int)(uint32_t)(pa >> 32));
    return (const uint8_t*)((((uint64_t)hi << 32) | lo) + off);
  };
  // Pools under 4 GiB: the page offset from the pool base fits 32 bits, so
  // a copy needs one exchange and its address is the (scalar) base plus a
  // 32-bit offset (instances with at most five copies per tensor and wave;
  // the second code path costs the others spills).
  constexpr bool P32 = KSL <= 5 && VSL <= 5;
  auto page_off32 = [&](int64_t sb, int64_t ss, int kv0, int page) {
    page = (unsigned)page < (unsigned)a.num_pages ? page : 0;  // outside the pool: page 0
    return (uint32_t)page * (uint32_t)sb + (uint32_t)((kv0 & (a.page_size - 1)) * ss);
  };
  auto paged_off32 = [&](uint32_t po, int idx, uint32_t off) {
    const int ps = (int)(pslot_bits >> (2 * idx)) & 3;
    return (uint32_t)__builtin_amdgcn_ds_bpermute(ps << 2, (int)po) + off;
  };
  auto dma_k = [&](int t, int buf, int pages) {
    const int kv0 = t * kSub;
    lds_u8* dst = kbuf0 + buf * C::K_BUF;
    if constexpr (!C::PAGED) {
      const auto rs = kv_whole ? k_rs_all : tile_rsrc(kbase, a.k_ss, kv0);
      const int soff = kv_whole ? kv0 * (int)a.k_ss : 0;
#pragma unroll
      for (int sl = 0; sl < KSL; ++sl) {
        const int j = wave + sl * C::NW;
        if (C::K_DMA_OPS % C::NW == 0 || sl + 1 < KSL || j < C::K_DMA_OPS)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, FMHA_LDS(void, dst + j * 1024), 16, (int)k_src[sl], soff, 0, 0);
      }
    } else if (P32 && kv0 + kSub <= a.Skv && a.pool32) {
      const uint32_t po = page_off32(a.k_sb, a.k_ss, kv0, pages);
      uint32_t off[KSL];
#pragma unroll
      for (int sl = 0; sl < KSL; ++sl) off[sl] = paged_off32(po, sl, k_src[sl]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int sl = 0; sl < KSL; ++sl) {
        const int j = min(wave + sl * C::NW, C::K_DMA_OPS - 1);
        __builtin_amdgcn_global_load_lds(kbase + off[sl], FMHA_LDS(void, dst + j * 1024), 16, 0, 0);
      }
    } else if (kv0 + kSub <= a.Skv) {
      // all page exchanges first, so their latencies overlap
      const uint64_t pa = page_addr(kbase, a.k_sb, a.k_ss, kv0, pages);
      const uint8_t* src[KSL];
#pragma unroll
      for (int sl = 0; sl < KSL; ++sl) src[sl] = paged_src(pa, a.k_ss, sl, k_src[sl], false, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int sl = 0; sl < KSL; ++sl) {
        const int j = min(wave + sl * C::NW, C::K_DMA_OPS - 1);
        __builtin_amdgcn_global_load_lds(src[sl], FMHA_LDS(void, dst + j * 1024), 16, 0, 0);
      }
    } else {
      const int rl = a.Skv - 1 - kv0;
      const uint64_t pa = page_addr(kbase, a.k_sb, a.k_ss, kv0, pages);
#pragma unroll
      for (int sl = 0; sl < KSL; ++sl) {
        const int j = min(wave + sl * C::NW, C::K_DMA_OPS - 1);
        int ch;
        const int row = k_copy_row(j, ch);
        const uint8_t* src = paged_src(pa, a.k_ss, sl, k_src[sl], row > rl, rl, ch);
        __builtin_amdgcn_global_load_lds(src, FMHA_LDS(void, dst + j * 1024), 16, 0, 0);
      }
    }
  };
  auto dma_v = [&](int t, int buf, int pages) {
    const int kv0 = t * kSub;
    lds_u8* dst = vbuf0 + buf * C::V_BUF;
    if constexpr (!C::PAGED) {
      const auto rs = kv_whole ? v_rs_all : tile_rsrc(vbase, a.v_ss, kv0);
      const int soff = kv_whole ? kv0 * (int)a.v_ss : 0;
#pragma unroll
      for (int sl = 0; sl < VSL; ++sl) {
        const int j = wave + sl * C::NW;
        if (C::V_DMA_OPS % C::NW == 0 || sl + 1 < VSL || j < C::V_DMA_OPS)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, FMHA_LDS(void, dst + j * 1024), 16, (int)v_src[sl], soff, 0, 0);
      }
    } else if (P32 && kv0 + kSub <= a.Skv && a.pool32) {
      const uint32_t po = page_off32(a.v_sb, a.v_ss, kv0, pages);
      uint32_t off[VSL];
#pragma unroll
      for (int sl = 0; sl < VSL; ++sl) off[sl] = paged_off32(po, KSL + sl, v_src[sl]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int sl = 0; sl < VSL; ++sl) {
        const int j = min(wave + sl * C::NW, C::V_DMA_OPS - 1);
        __builtin_amdgcn_global_load_lds(vbase + off[sl], FMHA_LDS(void, dst + j * 1024), 16, 0, 0);
      }
    } else if (kv0 + kSub <= a.Skv) {
      const uint64_t pa = page_addr(vbase, a.v_sb, a.v_ss, kv0, pages);
      const uint8_t* src[VSL];
#pragma unroll
      for (int sl = 0; sl < VSL; ++sl) src[sl] = paged_src(pa, a.v_ss, KSL + sl, v_src[sl], false, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int sl = 0; sl < VSL; ++sl) {
        const int j = min(wave + sl * C::NW, C::V_DMA_OPS - 1);
        __builtin_amdgcn_global_load_lds(src[sl], FMHA_LDS(void, dst + j * 1024), 16, 0, 0);
      }
    } else {
      const int rl = a.Skv - 1 - kv0;
      const uint64_t pa = page_addr(vbase, a.v_sb, a.v_ss, kv0, pages);
#pragma unroll
      for (int sl = 0; sl < VSL; ++sl) {
        const int j = min(wave + sl * C::NW, C::V_DMA_OPS - 1);
        int ch;
        const int row = v_copy_row(j, ch);
        const uint8_t* src = paged_src(pa, a.v_ss, KSL + sl, v_src[sl], row > rl, rl, ch);
        __builtin_amdgcn_global_load_lds(src, FMHA_LDS(void, dst + j * 1024), 16, 0, 0);
      }
    }
  };
  // ---- Q tile into registers (B operand of S^T = K Q^T)
  QRegs<C::MT, C::D> q;
  {
    const bool ok = qi < a.Sq;
    const uint8_t* qp = a.q + (int64_t)b * a.q_sb + (int64_t)hq * a.q_sh + (int64_t)(ok ? qi : 0) * a.q_ss;
    if constexpr (C::MT == FMT_BF16) {
#pragma unroll
      for (int t = 0; t < C::D / 16; ++t) {
        uint4 u = ok ? *(const uint4*)(qp + C::D * g + 16 * t) : make_uint4(0, 0, 0, 0);
        q.r[t] = __builtin_bit_cast(v8bf, u);
      }
    } else if constexpr (C::MT == FMT_E4M3) {
#pragma unroll
      for (int t = 0; t < C::D / 64; ++t) {
        uint4 u0 = ok ? *(const uint4*)(qp + 64 * t + 32 * g) : make_uint4(0, 0, 0, 0);
        uint4 u1 = ok ? *(const uint4*)(qp + 64 * t + 32 * g + 16) : make_uint4(0, 0, 0, 0);
        q.r[t] = v8i{(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w, (int)u1.x, (int)u1.y, (int)u1.z, (int)u1.w};
      }
    } else {
#pragma unroll
      for (int t = 0; t < C::D / 32; ++t) {
        uint4 u = ok ? *(const uint4*)(qp + 32 * t + 16 * g) : make_uint4(0, 0, 0, 0);
        q.r[t] = v4i{(int)u.x, (int)u.y, (int)u.z, (int)u.w};
      }
    }
  }
  float sq = 1.0f;
  if (C::QS) {
    const int qs = C::RP ? qi : (pack ? q0 : q0 + 32 * wave);  // wave-uniform unless rows hold several heads
    sq = a.sfs_q[((int64_t)b * a.Hq + hq) * a.nblk_q + min(qs, max(a.Sq - 1, 0)) / 64];
  }
  const float log2sp = a.sfs_p ? __log2f(a.sfs_p[hq]) : 0.0f;
  const float* sk_row = C::KS ? a.sfs_k + ((int64_t)b * a.Hkv + hk) * a.nblk_kv : nullptr;
  const float* sv_row = C::VS ? a.sfs_v + ((int64_t)b * a.Hkv + hk) * a.nblk_kv : nullptr;
  // K/V block scales of 64 consecutive sub-tiles live in one VGPR each (lane
  // i holds sub-tile base + i); a sub-tile's scale is read with readlane.
  int sc_base = -(1 << 30);
  float sk_cache = 1.0f, sv_cache = 1.0f;
  float sk_t = 1.0f, sv_t = 1.0f;  // scales of the current sub-tile (uniform)
  auto fetch_scales = [&](int t) {
    if constexpr (C::KS || C::VS) {
      if (t - sc_base >= 64) {
        sc_base = t;
        const int i = min(t + lane, a.nblk_kv - 1);
        if (C::KS) sk_cache = sk_row[i];
        if (C::VS) sv_cache = sv_row[i];
      }
      if (C::KS) sk_t = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sk_cache), t - sc_base));
      if (C::VS) sv_t = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sv_cache), t - sc_base));
    }
  };
  const float c_q = a.scale_log2 * sq;

  // ---- per-lane LDS read bases (stage-relative; every operand read is a
  //      fixed immediate offset from these)
  int kb_lane;
  if constexpr (C::WIDEN) kb_lane = m32 * C::KP + (C::D / 2) * g;
  else if constexpr (C::MT == FMT_BF16) kb_lane = m32 * C::KP + C::D * g;
  else if constexpr (C::MT == FMT_E4M3) kb_lane = m32 * C::KP + 32 * g;
  else kb_lane = m32 * C::KP + 16 * g;
  const int tr_G = lane >> 4;
  int vb_lane;
  if constexpr (C::P8)  // source row 16g + r, column 16(G%2) + 8h
    vb_lane = (16 * (tr_G >> 1) + ((lane & 15) >> 1)) * C::VP + 16 * (tr_G & 1) + 8 * (lane & 1);
  else  // bf16 V: source row 16g + r, byte column 32(G%2) + 8h'
    vb_lane = (16 * (tr_G >> 1) + ((lane & 15) >> 2)) * C::VP + 32 * (tr_G & 1) + 8 * (lane & 3);

  // S^T for one sub-tile from the K buffer `kb`.  The K operand reads of a
  // group (one 32-key tile, or a quarter of one for bf16 at head dim 192;
  // both tiles for E4M3 K widened under a bf16 Q) are issued before its
  // first MFMA, so each MFMA waits only for its own operand and the LDS
  // latency hides behind the MFMAs ahead of it.
  auto qk = [&](const lds_u8* kb, auto fence_tag) {
    constexpr bool FENCE = decltype(fence_tag)::value;
    SAcc<C::MT> acc;
    const lds_u8* kp = kb + kb_lane;
    if constexpr (C::WIDEN && (C::MASKED || C::PAGED)) {
      // E4M3 K beside the block-mask and page state: one 32-key tile of
      // operands in flight at a time (the instance then needs no scratch;
      // +0.8 % on the block-sparse workload)
#pragma unroll
      for (int T = 0; T < 2; ++T) {
        uint4 kr[C::D / 32];
#pragma unroll
        for (int j = 0; j < C::D / 32; ++j) kr[j] = *FMHA_LDS(const uint4, kp + 32 * T * C::KP + 16 * j);
        if constexpr (FENCE) __builtin_amdgcn_sched_barrier(0);
        acc.r[T] = v16f{};
#pragma unroll
        for (int j = 0; j < C::D / 32; ++j) {
          acc.r[T] = mfma_bf16(e4m3x8_to_bf16(kr[j].x, kr[j].y), q.r[2 * j], acc.r[T]);
          acc.r[T] = mfma_bf16(e4m3x8_to_bf16(kr[j].z, kr[j].w), q.r[2 * j + 1], acc.r[T]);
        }
      }
    } else if constexpr (C::WIDEN) {
      // E4M3 K: one 16-byte read holds the operands of two MFMAs (d =
      // (D/2)g + 16j .. +16), widened to bf16 just before use
      uint4 kr[2][C::D / 32];
#pragma unroll
      for (int T = 0; T < 2; ++T)
#pragma unroll
        for (int j = 0; j < C::D / 32; ++j) kr[T][j] = *FMHA_LDS(const uint4, kp + 32 * T * C::KP + 16 * j);
      if constexpr (FENCE) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int T = 0; T < 2; ++T) {
        acc.r[T] = v16f{};
#pragma unroll
        for (int j = 0; j < C::D / 32; ++j) {
          acc.r[T] = mfma_bf16(e4m3x8_to_bf16(kr[T][j].x, kr[T][j].y), q.r[2 * j], acc.r[T]);
          acc.r[T] = mfma_bf16(e4m3x8_to_bf16(kr[T][j].z, kr[T][j].w), q.r[2 * j + 1], acc.r[T]);
        }
      }
    } else if constexpr (C::MT == FMT_BF16 && C::D != 128) {
      // bf16 at head dim 192: a quarter of the K operands in flight at a time
#pragma unroll
      for (int T = 0; T < 2; ++T) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          uint4 kr[C::D / 32];
#pragma unroll
          for (int tt = 0; tt < C::D / 32; ++tt)
            kr[tt] = *FMHA_LDS(const uint4, kp + 32 * T * C::KP + 16 * ((C::D / 32) * h + tt));
          if constexpr (FENCE) __builtin_amdgcn_sched_barrier(0);
          if (h == 0) acc.r[T] = v16f{};
#pragma unroll
          for (int tt = 0; tt < C::D / 32; ++tt)
            acc.r[T] = mfma_bf16(__builtin_bit_cast(v8bf, kr[tt]), q.r[(C::D / 32) * h + tt], acc.r[T]);
        }
      }
    } else if constexpr (C::MT == FMT_BF16) {
      // half the K operands (one 32-key tile) in flight at a time: the
      // fewer live registers schedule slightly better than all of them
      // (measured +0.3-0.8 % on the dense bf16 loop), and masked / paged
      // instances need the room for their copy state
#pragma unroll
      for (int T = 0; T < 2; ++T) {
        uint4 kr[C::D / 16];
#pragma unroll
        for (int tt = 0; tt < C::D / 16; ++tt) kr[tt] = *FMHA_LDS(const uint4, kp + 32 * T * C::KP + 16 * tt);
        if constexpr (FENCE) __builtin_amdgcn_sched_barrier(0);
        acc.r[T] = v16f{};
#pragma unroll
        for (int tt = 0; tt < C::D / 16; ++tt) acc.r[T] = mfma_bf16(__builtin_bit_cast(v8bf, kr[tt]), q.r[tt], acc.r[T]);
      }
    } else if constexpr (C::MT == FMT_E4M3) {
      // 8-bit K: the operands of one 32-key tile in flight at a time (as for
      // bf16; measured neutral to +1.7 %)
#pragma unroll
      for (int T = 0; T < 2; ++T) {
        uint4 kr[C::D / 32];
#pragma unroll
        for (int i = 0; i < C::D / 32; ++i)
          kr[i] = *FMHA_LDS(const uint4, kp + 32 * T * C::KP + 64 * (i >> 1) + 16 * (i & 1));
        if constexpr (FENCE) __builtin_amdgcn_sched_barrier(0);
        acc.r[T] = v16f{};
#pragma unroll
        for (int tt = 0; tt < C::D / 64; ++tt) {
          const uint4 u0 = kr[2 * tt], u1 = kr[2 * tt + 1];
          const v8i av = {(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w, (int)u1.x, (int)u1.y, (int)u1.z, (int)u1.w};
          acc.r[T] = mfma_f8(av, q.r[tt], acc.r[T]);
        }
      }
    } else {
#pragma unroll
      for (int T = 0; T < 2; ++T) {
        uint4 kr[C::D / 32];
#pragma unroll
        for (int tt = 0; tt < C::D / 32; ++tt) kr[tt] = *FMHA_LDS(const uint4, kp + 32 * T * C::KP + 32 * tt);
        if constexpr (FENCE) __builtin_amdgcn_sched_barrier(0);
        acc.r[T] = v16i{};
#pragma unroll
        for (int tt = 0; tt < C::D / 32; ++tt) {
          const uint4 u = kr[tt];
          acc.r[T] = mfma_i8(v4i{(int)u.x, (int)u.y, (int)u.z, (int)u.w}, q.r[tt], acc.r[T]);
        }
      }
    }
    return acc;
  };

  // S^T with the wave's issue priority raised around the K operand reads
  // (+1.5-2 % measured).  The compiler issues the S MFMAs themselves after
  // the priority drop; keeping them inside the raised region measured no
  // different.
  auto qk_raised = [&](const lds_u8* kb) {
    __builtin_amdgcn_s_setprio(1);
    const SAcc<C::MT> acc = qk(kb, std::true_type{});
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    return acc;
  };

  // ---- per-lane state.  O^T (D/32 tiles of 32 d x 32 queries) is kept in units
  // of the reference V scale `sv_ref`: before a sub-tile's PV product is
  // accumulated, O is multiplied by alpha_row * sv_ref / sv_tile (one multiply
  // folds the lazy rescale and the change of V block scale), then the MFMA
  // accumulates codes x codes directly.
  v16f o[C::ND];
#pragma unroll
  for (int d = 0; d < C::ND; ++d) o[d] = v16f{};
  float m_run = -kInf;
  // Row sums of P.  With E4M3 P they come from the matrix core: a 16x16x128
  // product of a 0/1 matrix with the P operand (read as 128 x 16) whose row
  // pattern selects, for the 16 queries of each lane group, the two 32-key
  // slots that belong to that lane's query; register 0 of every lane then
  // holds the sum for its own query.  bf16 P is summed on the VALU.
  float den = 0.0f;
  v4f den_acc = {};
  const v8i ones_a = (((lane >> 2) ^ (lane >> 4)) & 1) ? v8i{} : v8i{0x38383838, 0x38383838, 0x38383838, 0x38383838,
                                                                   0x38383838, 0x38383838, 0x38383838, 0x38383838};
  float sv_ref = 1.0f;

  // V-scale reference (wave-uniform).  The fast path moves the reference to
  // every sub-tile's own scale, so the MFMA accumulates codes x codes straight
  // into O; it is taken when all V block scales of this (batch, KV head) lie
  // within 2^64 of each other, which bounds |O| far below the fp32 range.
  // Otherwise each sub-tile's product goes through a zeroed accumulator and is
  // added with its scale relative to the reference.
  bool v_direct = true;
  if constexpr (C::VS) {
    float lo = kInf, hi = 0.0f;
    for (int i = lane; i < a.nblk_kv; i += 64) {
      const float v = sv_row[i];
      lo = fminf(lo, v);
      hi = fmaxf(hi, v);
    }
    lo = -wave_max(-lo);
    hi = wave_max(hi);
    v_direct = hi <= lo * 0x1p64f;
  }

  // P of one sub-tile in the PV operand format, with the V scale factor the
  // slow V-reference path applies to its product.
  struct PTile {
    v8i pb;            // E4M3 P: B operand of the 32x32x64 MFMA
    v8bf pbf[4];       // bf16 P: B operands of four 32x32x16 MFMAs
    float f;           // product scale (slow path only)
  };

  // Softmax of one sub-tile, written as eight stages of separable work:
  //   0: row max, lazy decision, rescale of den (and of O off the fast path);
  //   1-2: rescale of O, half the d-tiles each (fast V-reference path, E4M3
  //        V excepted: there the PV step rescales each d-tile just before
  //        its product);
  //   3-6: P = 2^(s2 - m) / sp for eight keys each, clamped to the E4M3 range
  //        only where P / sp can reach it (sfs_p given or tau above log2 448);
  //   7: P to the PV operand format (bf16 P: also den += P).
  struct SmState {
    float s[32];
    float c, negm, fo;
    PTile pt;
  };
  auto sm_stage = [&](auto k_tag, SmState& st, const SAcc<C::MT>& acc, int t, auto edge_tag, auto clamp_tag,
                      auto direct_tag) {
    constexpr int K = decltype(k_tag)::value;
    constexpr bool EDGE = decltype(edge_tag)::value;
    constexpr bool CLAMP = decltype(clamp_tag)::value;
    constexpr bool DIRECT = decltype(direct_tag)::value;
    constexpr bool INTERLEAVE = FMHA_PV_INTERLEAVE && C::VF == FMT_E4M3;
    if constexpr (K == 0) {
      st.pt.f = 1.0f;
#pragma unroll
      for (int e = 0; e < 32; ++e) st.s[e] = (float)acc.r[e >> 4][e & 15];
      if constexpr (EDGE) {
        // s[e] is key t*64 + 32(e/16) + 16g + e%16
        const int lim = (a.causal ? min(a.Skv, qi + causal_off + 1) : a.Skv) - t * kSub;
#pragma unroll
        for (int e = 0; e < 32; ++e) {
          const int key = 32 * (e >> 4) + 16 * g + (e & 15);
          st.s[e] = key < lim ? st.s[e] : -kInf;
        }
      }
      // 3-input max tree: 32 -> 11 -> 4 -> 1 (16 v_max3)
      float m1[11];
#pragma unroll
      for (int i = 0; i < 10; ++i) m1[i] = fmaxf(fmaxf(st.s[3 * i], st.s[3 * i + 1]), st.s[3 * i + 2]);
      m1[10] = fmaxf(st.s[30], st.s[31]);
      const float m2a = fmaxf(fmaxf(m1[0], m1[1]), m1[2]), m2b = fmaxf(fmaxf(m1[3], m1[4]), m1[5]);
      const float m2c = fmaxf(fmaxf(m1[6], m1[7]), m1[8]), m2d = fmaxf(m1[9], m1[10]);
      float mx = fmaxf(fmaxf(m2a, m2b), fmaxf(m2c, m2d));
      {
        // lanes l and l ^ 32 hold the two key halves of the same row
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      st.c = C::KS ? c_q * sk_t : c_q;
      const float tmax = mx * st.c;  // c > 0, so the maximum commutes with the scale
      const bool trig = (tmax != -kInf) & ((m_run == -kInf) | (tmax - m_run > a.tau));  // no short-circuit branches
      // 2^(m - t) is 0 for an unset m (m = -inf); rows that do not trigger keep 1
      const float e_mt = __builtin_amdgcn_exp2f(m_run - tmax);
      const float alpha = trig ? e_mt : 1.0f;
      m_run = trig ? tmax : m_run;
      if constexpr (C::P8) den_acc[0] *= alpha;
      else den *= alpha;
      st.negm = m_run == -kInf ? -kInf : -(m_run + log2sp);
      if constexpr (C::VS && DIRECT) {
        // one factor folds the lazy rescale and the change of V reference
        st.fo = alpha * (sv_ref * __builtin_amdgcn_rcpf(sv_t));
        sv_ref = sv_t;
        if constexpr (INTERLEAVE) st.pt.f = st.fo;  // applied by the PV step
      } else {
        if (__ballot(trig) != 0) {
#pragma unroll
          for (int d = 0; d < C::ND; ++d)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[d][r] *= alpha;
        }
        if constexpr (C::VS) st.pt.f = sv_t / sv_ref;  // reference stays at 1
      }
    } else if constexpr (K == 1 || K == 2) {
      if constexpr (C::VS && DIRECT && !INTERLEAVE) {
#pragma unroll
        for (int d = (C::ND / 2) * (K - 1); d < (K == 2 ? C::ND : C::ND / 2); ++d)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[d][r] *= st.fo;
      }
    } else if constexpr (K >= 3 && K <= 6) {
#pragma unroll
      for (int e = 8 * (K - 3); e < 8 * (K - 2); ++e) {
        st.s[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(st.s[e], st.c, st.negm));
        if constexpr (CLAMP) st.s[e] = fminf(st.s[e], 448.0f);
      }
    } else {
      if constexpr (C::P8) {
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          int pk = pack_e4m3<false>(st.s[4 * w], st.s[4 * w + 1], any_vgpr());
          pk = pack_e4m3<true>(st.s[4 * w + 2], st.s[4 * w + 3], pk);
          st.pt.pb[w] = pk;
        }
      } else {
        float dsum = 0.0f;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          uint32_t w[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t lo = f32_to_bf16_bits(st.s[8 * kk + 2 * j]);
            const uint32_t hi = f32_to_bf16_bits(st.s[8 * kk + 2 * j + 1]);
            w[j] = lo | (hi << 16);
            dsum += bf16_bits_to_f32(lo) + bf16_bits_to_f32(hi);
          }
          st.pt.pbf[kk] = __builtin_bit_cast(v8bf, make_uint4(w[0], w[1], w[2], w[3]));
        }
        den += dsum;
      }
    }
  };
  // The whole softmax of sub-tile t: P and the slow-path product scale.
  auto softmax_p = [&](const SAcc<C::MT>& acc, int t, auto edge_tag, auto clamp_tag, auto direct_tag) {
    SmState st;
    static_for<0, 8>([&](auto k) { sm_stage(k, st, acc, t, edge_tag, clamp_tag, direct_tag); });
    return st.pt;
  };

  // V^T operand (E4M3 V) of d-tile d from V buffer `vb`: rows 32(cq/2) +
  // 8(cq%2) further down and columns 32d further right of the lane's base.
  auto read_vop = [&](const lds_u8* vb, int d) {
    v8i v;
    const lds_u8* vp = vb + vb_lane;
#pragma unroll
    for (int cq = 0; cq < 4; ++cq) {
      const v2i r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          FMHA_LDS(v2i, vp + (32 * (cq >> 1) + 8 * (cq & 1)) * C::VP + 32 * d));
      v[2 * cq] = r[0];
      v[2 * cq + 1] = r[1];
    }
    return v;
  };
  // O^T += V^T P^T for one sub-tile from V buffer `vb`; with E4M3 P the row
  // sums of P come from the same operand.
  auto pv_e4m3 = [&](const PTile& pt, const v8i* vop, auto direct_tag) {
    constexpr bool DIRECT = decltype(direct_tag)::value;
    den_acc = mfma_f8_16(ones_a, pt.pb, den_acc);
#pragma unroll
    for (int d = 0; d < C::ND; ++d) {
      if constexpr (C::VS && DIRECT && FMHA_PV_INTERLEAVE) {
        // O factor of this d-tile, then its product; the next d-tile's
        // multiplies are ordered after this product's issue
#pragma unroll
        for (int r = 0; r < 16; ++r) o[d][r] *= pt.f;
        o[d] = mfma_f8(vop[d], pt.pb, o[d]);
        __builtin_amdgcn_sched_barrier(0);
      } else if constexpr (!C::VS || DIRECT) {
        o[d] = mfma_f8(vop[d], pt.pb, o[d]);
      } else {
        const v16f part = mfma_f8(vop[d], pt.pb, v16f{});
#pragma unroll
        for (int r = 0; r < 16; ++r) o[d][r] = __builtin_fmaf(part[r], pt.f, o[d][r]);
      }
    }
  };
  auto pv = [&](const PTile& pt, const lds_u8* vb, auto direct_tag) {
    const lds_u8* vp = vb + vb_lane;
    if constexpr (C::VF == FMT_E4M3) {
      v8i vop[C::ND];
#pragma unroll
      for (int d = 0; d < C::ND; ++d) vop[d] = read_vop(vb, d);
      pv_e4m3(pt, vop, direct_tag);
    } else if constexpr (C::VF == FMT_INT8) {
      // E4M3 P and int8 V on the 32x32x16 fp16 product: both widen to fp16
      // exactly and every product is exact, so O sums the same code products
      // as the 8-bit path would.  MFMA kk takes the eight keys of transposing
      // read kk (rows 32(kk/2) + 8(kk%2) down) and P bytes 8kk .. 8kk+7.
      constexpr bool DIRECT = decltype(direct_tag)::value;
      den_acc = mfma_f8_16(ones_a, pt.pb, den_acc);
      v8h pf[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) pf[kk] = e4m3x8_to_f16(pt.pb[2 * kk], pt.pb[2 * kk + 1]);
#pragma unroll
      for (int d = 0; d < C::ND; ++d) {
        v16f acc = (!C::VS || DIRECT) ? o[d] : v16f{};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const v2i r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              FMHA_LDS(v2i, vp + (32 * (kk >> 1) + 8 * (kk & 1)) * C::VP + 32 * d));
          acc = mfma_f16(int8x8_to_f16(r[0], r[1]), pf[kk], acc);
        }
        if constexpr (!C::VS || DIRECT) {
          o[d] = acc;
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) o[d][r] = __builtin_fmaf(acc[r], pt.f, o[d][r]);
        }
      }
    } else {
      // bf16 P and V (V unscaled).
#pragma unroll
      for (int d = 0; d < C::ND; ++d) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          uint32_t w[4];
#pragma unroll
          for (int cq = 0; cq < 2; ++cq) {
            // rows 32(kk/2) + 8(kk%2) + 4cq further down, columns 64d bytes right
            const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                FMHA_LDS(v4s, vp + (32 * (kk >> 1) + 8 * (kk & 1) + 4 * cq) * C::VP + 64 * d));
            w[2 * cq] = (uint32_t)(uint16_t)r[0] | ((uint32_t)(uint16_t)r[1] << 16);
            w[2 * cq + 1] = (uint32_t)(uint16_t)r[2] | ((uint32_t)(uint16_t)r[3] << 16);
          }
          o[d] = mfma_bf16(__builtin_bit_cast(v8bf, make_uint4(w[0], w[1], w[2], w[3])), pt.pbf[kk], o[d]);
        }
      }
    }
  };


  // ---- main loop over 64-key sub-tiles, K/V double-buffered in LDS.  Per
  // sub-tile a wave runs S^T = K Q^T (MFMA), the softmax (VALU), then
  // O^T += V^T P^T (MFMA); MFMA/VALU overlap comes from the other wave on the
  // SIMD being in another phase.  The copies of the next sub-tile are issued
  // early in the step and land while the current one is processed (paged:
  // its page numbers were read during the previous sub-tile).
  if constexpr (C::SUB > 1) {
    // ---- dense loop over tiles of SUB sub-tiles: the copies of tile T + 1
    // are issued with the first sub-tile of tile T, one barrier per tile.
    const int ntile = (n_sub + C::SUB - 1) / C::SUB;
    if (ntile > 0) {
      dma_k(0, 0, 0);
      dma_v(0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    const bool clamp = C::P8 && a.clamp_p;
    auto sub_step = [&](int t, int T, auto u_tag, auto edge_tag, auto clamp_tag, auto direct_tag) {
      constexpr int u = decltype(u_tag)::value;
      const int bv = T & 1;
      const lds_u8* kb = kbuf0 + bv * C::K_BUF + u * kSub * C::KP;
      const lds_u8* vb = vbuf0 + bv * C::V_BUF + u * kSub * C::VP;
      fetch_scales(t);
      if (u == 0 && T + 1 < ntile) {
        dma_k((T + 1) * C::SUB, bv ^ 1, 0);
        dma_v((T + 1) * C::SUB, bv ^ 1, 0);
      }
      const SAcc<C::MT> acc = qk_raised(kb);
      pv(softmax_p(acc, t, edge_tag, clamp_tag, direct_tag), vb, direct_tag);
    };
    auto run_tiles = [&](auto clamp_tag, auto direct_tag) {
      // whole tiles valid for every pair, then the rest with per-pair masks
      int T = 0;
      for (; (T + 1) * C::SUB <= full_end; ++T) {
        static_for<0, C::SUB>([&](auto u) { sub_step(T * C::SUB + u, T, u, std::false_type{}, clamp_tag, direct_tag); });
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies have landed
        __syncthreads();
      }
      for (; T < ntile; ++T) {
        static_for<0, C::SUB>([&](auto u) {
          if (T * C::SUB + u < n_sub) sub_step(T * C::SUB + u, T, u, std::true_type{}, clamp_tag, direct_tag);
        });
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
      }
    };
    if constexpr (C::VS) {
      if (clamp) {
        if (v_direct) run_tiles(std::true_type{}, std::true_type{});
        else run_tiles(std::true_type{}, std::false_type{});
      } else {
        if (v_direct) run_tiles(std::false_type{}, std::true_type{});
        else run_tiles(std::false_type{}, std::false_type{});
      }
    } else {
      if (clamp) run_tiles(std::true_type{}, std::true_type{});
      else run_tiles(std::false_type{}, std::true_type{});
    }
  } else {
  int tc = next_sub(0);
  int tn = n_sub, pg_n = 0;
  if (tc < n_sub) {
    const int pg_c = load_pages(tc);
    dma_k(tc, 0, pg_c);
    dma_v(tc, 0, pg_c);
    tn = next_sub(tc + 1);
    if (tn < n_sub) pg_n = load_pages(tn);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies have landed
  __syncthreads();
  // Dense two-wave instances with an E4M3 V read their V operands right after
  // issuing the S MFMAs (32 more live registers) and issue the copies of the
  // next sub-tile after that, in the shadow of those MFMAs; the others issue
  // the copies first and read V in the PV step.
  constexpr bool EARLY_V = C::VF == FMT_E4M3 && C::WPE == 2 && !C::MASKED && !C::PAGED && C::D == 128;
  // The buffer holding sub-tile tc: the captured `buf`, toggled by each
  // step, or (unrolled dense loop) a compile-time 0 / 1, so that LDS
  // addresses fold into the instructions.
  int buf = 0;
  auto issue_next = [&](int& tnn, int bv) {
    if (tn < n_sub) {
      dma_k(tn, bv ^ 1, pg_n);
      dma_v(tn, bv ^ 1, pg_n);
      tnn = next_sub(tn + 1);
      if (C::PAGED && tnn < n_sub) pg_n = load_pages(tnn);
    }
  };
  auto step = [&](auto edge_tag, auto clamp_tag, auto direct_tag, auto buf_tag) {
    constexpr int FIXED = decltype(buf_tag)::value;  // -1: the captured buf
    const int bv = FIXED >= 0 ? FIXED : buf;
    fetch_scales(tc);
    int tnn = n_sub;
    if constexpr (EARLY_V) {
      const SAcc<C::MT> acc = qk_raised(kbuf0 + bv * C::K_BUF);
      v8i vop[C::ND];
#pragma unroll
      for (int d = 0; d < C::ND; ++d) vop[d] = read_vop(vbuf0 + bv * C::V_BUF, d);
      issue_next(tnn, bv);
      __builtin_amdgcn_sched_barrier(0);
      pv_e4m3(softmax_p(acc, tc, edge_tag, clamp_tag, direct_tag), vop, direct_tag);
    } else {
      issue_next(tnn, bv);
      const SAcc<C::MT> acc = qk_raised(kbuf0 + bv * C::K_BUF);
      pv(softmax_p(acc, tc, edge_tag, clamp_tag, direct_tag), vbuf0 + bv * C::V_BUF, direct_tag);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies have landed
    __syncthreads();
    if (FIXED < 0) buf ^= 1;
    tc = tn;
    tn = tnn;
  };
  using BufRt = std::integral_constant<int, -1>;
  auto run = [&](auto clamp_tag, auto direct_tag) {
    // sub-tiles valid for every pair of the workgroup first (a block mask
    // only skips whole sub-tiles), then the edge ones; dense contiguous
    // instances at head dim 128 take the first kind two per trip with the
    // buffers fixed (the others have no registers to spare for the longer
    // loop)
    if constexpr (!C::MASKED && !C::PAGED && C::D == 128) {
      while (tc < n_sub && tc < full_end) {
        [[clang::always_inline]] step(std::false_type{}, clamp_tag, direct_tag, std::integral_constant<int, 0>{});
        if (!(tc < n_sub && tc < full_end)) {
          buf = 1;
          break;
        }
        [[clang::always_inline]] step(std::false_type{}, clamp_tag, direct_tag, std::integral_constant<int, 1>{});
      }
    } else {
      while (tc < n_sub && tc < full_end) step(std::false_type{}, clamp_tag, direct_tag, BufRt{});
    }
    while (tc < n_sub) step(std::true_type{}, clamp_tag, direct_tag, BufRt{});
  };
  const bool clamp = C::P8 && a.clamp_p;
  if constexpr (C::VS) {
    if (clamp) {
      if (v_direct) run(std::true_type{}, std::true_type{});
      else run(std::true_type{}, std::false_type{});
    } else {
      if (v_direct) run(std::false_type{}, std::true_type{});
      else run(std::false_type{}, std::false_type{});
    }
  } else {
    if (clamp) run(std::true_type{}, std::true_type{});
    else run(std::false_type{}, std::true_type{});
  }

  }  // SUB == 1

  // ---- epilogue: O = num / den in bf16 (or E4M3); rows without a valid key give 0
  float dt;
  if constexpr (C::P8) dt = den_acc[0];
  else dt = den + __shfl_xor(den, 32, 64);
  const float inv = dt > 0.0f ? sv_ref / dt : 0.0f;
  if (qi >= a.Sq) FMHA_END_TILE;
  uint8_t* op = a.o + (int64_t)b * a.o_sb + (int64_t)hq * a.o_sh + (int64_t)qi * a.o_ss;
  if (a.o_fp8) {
    // E4M3 output: encode(O / sfs_o), nearest-even, saturating at +-448
    const float f = a.sfs_o ? inv / a.sfs_o[hq] : inv;
#pragma unroll
    for (int d = 0; d < C::ND; ++d) {
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = fminf(fmaxf(o[d][4 * a4 + i] * f, -448.0f), 448.0f);
        int pk = pack_e4m3<false>(x[0], x[1], 0);
        pk = pack_e4m3<true>(x[2], x[3], pk);
        *(int*)(op + 32 * d + 8 * a4 + 4 * g) = pk;
      }
    }
    FMHA_END_TILE;
  }
#pragma unroll
  for (int d = 0; d < C::ND; ++d) {
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int dd = 32 * d + 8 * a4 + 4 * g;
      uint32_t h0 = f32_to_bf16_bits(o[d][4 * a4 + 0] * inv);
      uint32_t h1 = f32_to_bf16_bits(o[d][4 * a4 + 1] * inv);
      uint32_t h2 = f32_to_bf16_bits(o[d][4 * a4 + 2] * inv);
      uint32_t h3 = f32_to_bf16_bits(o[d][4 * a4 + 3] * inv);
      *(uint2*)(op + 2 * dd) = make_uint2(h0 | (h1 << 16), h2 | (h3 << 16));
    }
  }
  }  // tile
#if FMHA_PERSISTENT
  tile_end:
  __syncthreads();
#endif
  }
#endif
}
#undef FMHA_END_TILE

// Rows per head of a packed workgroup (0: no packing).  Heads are packed
// when the query range is causal or shorter than a workgroup tile; query
// ranges shorter than 16 also pack heads inside a wave: R rows per head, R
// the smallest power of two >= Sq that the group size still allows.
int pack_rows(const FwdArgs& a, int nw) {
  const bool pack = FMHA_HEAD_PACK && a.mask == nullptr && a.group % nw == 0 && (a.causal || a.Sq < 32 * nw);
  if (!pack) return 0;
  int rows = 32;
  while (FMHA_ROW_PACK && rows > 1 && rows / 2 >= a.Sq && (a.group / nw) % (64 / rows) == 0) rows /= 2;
  return rows;
}

template <class C>
hipError_t launch(const FwdArgs& args, hipStream_t stream) {
  // Head packing where K/V reuse across the heads of a group pays: a query
  // range shorter than one workgroup tile, or a causal one (the waves then
  // share one diagonal instead of staggering along it).
  FwdArgs a = args;
  a.pack_rows = pack_rows(a, C::NW);
  if (!C::RP && a.pack_rows) a.pack_rows = 32;
  const bool pack = a.pack_rows > 0;
  const int rows = pack ? a.pack_rows : 32;
  const int qtile = pack ? rows : 32 * C::NW;
  const int64_t tiles = (int64_t)((a.Sq + qtile - 1) / qtile) * a.Hq * a.B / (pack ? C::NW * (32 / rows) : 1);
  if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  a.tiles = (int)tiles;
  dim3 grid((unsigned)tiles);
  const size_t lds = (size_t)C::LDS_BYTES;
  static bool configured = false;  // benign race: the attribute is idempotent
  static int slots = 0;            // persistent launch: resident workgroups per device
  if (!configured) {
    hipError_t e = hipFuncSetAttribute((const void*)fwd_kernel<C>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    if (FMHA_PERSISTENT) {
      int dev = 0, cus = 0, per_cu = 0;
      if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
      if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
      if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fwd_kernel<C>, C::NT, lds)) != hipSuccess) return e;
      slots = max(8, (cus * per_cu) / 8 * 8);
    }
    configured = true;
  }
  if (FMHA_PERSISTENT && tiles > slots) grid.x = (unsigned)slots;
  hipLaunchKernelGGL(fwd_kernel<C>, grid, dim3(C::NT), lds, stream, a);
  return hipGetLastError();
}

}  // namespace

bool fwd_supported(const FwdKey& k) {
  if (k.D == 192) {
    // head dim 192: 8-bit Q and K, bf16 Q and K with a scaled E4M3 V (the
    // DiT formats), all bf16, and bf16 Q with scaled E4M3 K and V (the
    // block-sparse format); dense, causal, block-masked or paged.  bf16 Q and
    // K read a quarter of the K operands at a time so that Q, O and the reads
    // fit two wavefronts per SIMD (all-bf16 K and V tiles take 100 KB of LDS:
    // one workgroup per CU); masked, paged and widened-K instances run one
    // wavefront per SIMD
    if (k.qf == FMT_INT8 && k.kf == FMT_INT8 && k.vf == FMT_E4M3) return k.q_scaled && k.k_scaled && k.v_scaled;
    if (k.qf == FMT_E4M3 && k.kf == FMT_E4M3 && k.vf == FMT_E4M3) return k.q_scaled && k.k_scaled && k.v_scaled;
    if (k.qf == FMT_BF16 && k.kf == FMT_BF16 && k.vf == FMT_E4M3) return !k.q_scaled && !k.k_scaled && k.v_scaled;
    if (k.qf == FMT_BF16 && k.kf == FMT_BF16 && k.vf == FMT_BF16) return !k.q_scaled && !k.k_scaled && !k.v_scaled;
    if (k.qf == FMT_BF16 && k.kf == FMT_E4M3 && k.vf == FMT_E4M3) return !k.q_scaled && k.k_scaled && k.v_scaled;
    return false;
  }
  if (k.D != 128) return false;
  if (k.qf == FMT_BF16 && k.kf == FMT_BF16 && k.vf == FMT_BF16)
    return !k.q_scaled && !k.k_scaled && !k.v_scaled;
  if (k.qf == FMT_INT8 && k.kf == FMT_INT8 && k.vf == FMT_E4M3) return k.q_scaled && k.k_scaled && k.v_scaled;
  if (k.qf == FMT_BF16 && k.kf == FMT_BF16 && k.vf == FMT_E4M3) return !k.q_scaled && !k.k_scaled;
  if (k.qf == FMT_E4M3 && k.kf == FMT_E4M3 && k.vf == FMT_E4M3) return k.q_scaled && k.k_scaled && k.v_scaled;
  if (k.qf == FMT_BF16 && k.kf == FMT_E4M3 && k.vf == FMT_E4M3) return !k.q_scaled && k.k_scaled && k.v_scaled;
  if (k.qf == FMT_E4M3 && k.kf == FMT_E4M3 && k.vf == FMT_INT8) return k.q_scaled && k.k_scaled && k.v_scaled;
  return false;
}

template <int QF, int KF, int VF, bool QS, bool KS, bool VS>
static hipError_t dispatch_layout(const FwdKey& k, const FwdArgs& a, hipStream_t s) {
  if (k.masked) {
    if (k.paged) return launch<Cfg<QF, KF, VF, QS, KS, VS, true, true, 2>>(a, s);
    return launch<Cfg<QF, KF, VF, QS, KS, VS, true, false, 2>>(a, s);
  }
  const int rows = pack_rows(a, kDenseWaves);
  if (rows > 0 && rows < 32) {
    if (k.paged) return launch<Cfg<QF, KF, VF, QS, KS, VS, false, true, kDenseWaves, true>>(a, s);
    return launch<Cfg<QF, KF, VF, QS, KS, VS, false, false, kDenseWaves, true>>(a, s);
  }
  // Groups too small to fill four waves with several heads each (e.g. four
  // query heads per KV head) use two-wave workgroups; with 8-bit K in LDS
  // four of them still fit a CU.
  if constexpr (KF != FMT_BF16) {
    const int rows2 = pack_rows(a, 2);
    if (FMHA_ROW_PACK_NW2 && rows2 > 0 && rows2 < 32) {
      if (k.paged) return launch<Cfg<QF, KF, VF, QS, KS, VS, false, true, 2, true>>(a, s);
      return launch<Cfg<QF, KF, VF, QS, KS, VS, false, false, 2, true>>(a, s);
    }
  }
  if (k.paged) return launch<Cfg<QF, KF, VF, QS, KS, VS, false, true, kDenseWaves>>(a, s);
  constexpr int KT = QF != FMT_BF16 ? FMHA_KV_TILE_8BIT : 64;
  return launch<Cfg<QF, KF, VF, QS, KS, VS, false, false, kDenseWaves, false, 128, KT>>(a, s);
}

// Head dim 192: dense / causal (with whole-wave head packing as a run-time
// choice), block-masked, paged, or both; no heads packed inside a wave (that
// needs the RP instances).
template <int QF, int KF, int VF, bool QS, bool KS, bool VS>
static hipError_t dispatch_d192(const FwdKey& k, const FwdArgs& a, hipStream_t s) {
  if (k.masked) {
    if (k.paged) return launch<Cfg<QF, KF, VF, QS, KS, VS, true, true, 2, false, 192>>(a, s);
    return launch<Cfg<QF, KF, VF, QS, KS, VS, true, false, 2, false, 192>>(a, s);
  }
  if (k.paged) return launch<Cfg<QF, KF, VF, QS, KS, VS, false, true, kDenseWaves, false, 192>>(a, s);
  return launch<Cfg<QF, KF, VF, QS, KS, VS, false, false, kDenseWaves, false, 192>>(a, s);
}

hipError_t launch_fwd(const FwdKey& k, const FwdArgs& a, hipStream_t s) {
  if (!fwd_supported(k)) return hipErrorInvalidValue;
  if (k.D == 192) {
    if (k.qf == FMT_BF16 && k.vf == FMT_BF16)
      return dispatch_d192<FMT_BF16, FMT_BF16, FMT_BF16, false, false, false>(k, a, s);
    if (k.qf == FMT_BF16 && k.kf == FMT_BF16)
      return dispatch_d192<FMT_BF16, FMT_BF16, FMT_E4M3, false, false, true>(k, a, s);
    if (k.qf == FMT_BF16)
      return dispatch_d192<FMT_BF16, FMT_E4M3, FMT_E4M3, false, true, true>(k, a, s);
    if (k.qf == FMT_INT8)
      return dispatch_d192<FMT_INT8, FMT_INT8, FMT_E4M3, true, true, true>(k, a, s);
    return dispatch_d192<FMT_E4M3, FMT_E4M3, FMT_E4M3, true, true, true>(k, a, s);
  }
  if (k.qf == FMT_BF16 && k.kf == FMT_BF16 && k.vf == FMT_BF16)
    return dispatch_layout<FMT_BF16, FMT_BF16, FMT_BF16, false, false, false>(k, a, s);
  if (k.qf == FMT_INT8)
    return dispatch_layout<FMT_INT8, FMT_INT8, FMT_E4M3, true, true, true>(k, a, s);
  if (k.qf == FMT_BF16 && k.kf == FMT_BF16) {
    if (k.v_scaled) return dispatch_layout<FMT_BF16, FMT_BF16, FMT_E4M3, false, false, true>(k, a, s);
    return dispatch_layout<FMT_BF16, FMT_BF16, FMT_E4M3, false, false, false>(k, a, s);
  }
  if (k.qf == FMT_E4M3 && k.vf == FMT_INT8)
    return dispatch_layout<FMT_E4M3, FMT_E4M3, FMT_INT8, true, true, true>(k, a, s);
  if (k.qf == FMT_E4M3)
    return dispatch_layout<FMT_E4M3, FMT_E4M3, FMT_E4M3, true, true, true>(k, a, s);
  return dispatch_layout<FMT_BF16, FMT_E4M3, FMT_E4M3, false, true, true>(k, a, s);
}

}  // namespace fmha
