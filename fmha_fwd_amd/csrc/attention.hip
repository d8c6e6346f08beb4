// Fused attention forward for gfx950: block-scaled int8 / E4M3 / bf16 Q and
// K, E4M3 or bf16 V and P, online softmax with lazy rescaling, bf16 output.
//
// Method sources (FlashInfer pull-request write-ups):
//  * #2711 page "FlashInfer의 DiT 최적화: SageAttention과 Int8/FP8 혼합 정밀도
//    커널 도입 분석", 코드 분석 2: per-block Q/K/P/V scale factors that undo
//    the quantisation after BMM1 (QK^T) and BMM2 (PV); 코드 분석 1: Q, K, V
//    formats chosen independently.
//  * #5900 page "Blackwell 아키텍처를 위한 FlashInfer의 FP8/BF16 혼합 정밀도
//    Attention 최적화 분석", 코드 분석 3: lazy correction (O is rescaled only
//    when the row maximum grows by 2^8); 코드 분석 1: QK in bf16 or fp8 with an
//    fp8 P, head dim 128, 16-bit output.
//  * #4474 page "FlashInfer의 PrimTS를 활용한 고성능 Block-Sparse Attention
//    최적화", 코드 분석 1-2: Q64 x KV256 block-sparse masks, paged K/V.
//
// Design for CDNA4 (not a translation of the pages' Hopper/Blackwell kernels):
//  * One workgroup = NW wavefronts x 32 queries of one (batch, head).  K and V
//    stream through LDS in 64-key sub-tiles, double-buffered; the Q tile stays
//    in VGPRs for the whole key loop.
//  * The score tile is computed transposed, S^T = K Q^T, on 32x32 MFMA tiles,
//    so every lane owns one query row: the row max / sum are in-register
//    reductions plus one exchange with lane l ^ 32, and the per-row lazy
//    rescale factor multiplies the lane's own O^T registers.
//  * Keys are permuted inside a 32-key MFMA tile (sigma below) so that the
//    S^T accumulator of lane group g holds 16 consecutive keys; those P values
//    are packed in place into the B operand of O^T += V^T P^T, and V^T is read
//    from LDS with the gfx950 transposing loads (ds_read_b64_tr_b8 / _b16).
//  * The lazy decision is per row and per 64-key sub-tile; the branch is taken
//    by the whole wave when any row triggers, with factor 1 for the others.
//  * V's per-64-token scale multiplies each sub-tile's PV partial product
//    before it is added to O (scales applied after BMM2).
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
#ifndef FMHA_WAVES_PER_EU
#define FMHA_WAVES_PER_EU 2  // register budget: 512 / 2 VGPRs per lane
#endif
constexpr float kInf = __builtin_huge_valf();

// Key held by row m of a 32-key MFMA tile: lane group g of the S^T result
// then owns keys 16g .. 16g + 15 in its 16 accumulator registers.
__device__ __forceinline__ int sigma(int m) {
  return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3);
}

template <int QF_, int KF_, int VF_, bool QS_, bool KS_, bool VS_, bool MASKED_, bool PAGED_, int NW_>
struct Cfg {
  static constexpr int QF = QF_, KF = KF_, VF = VF_, NW = NW_;
  static constexpr bool QS = QS_, KS = KS_, VS = VS_, MASKED = MASKED_, PAGED = PAGED_;
  static constexpr int MT = QF;                                  // QK operand format
  static constexpr int KROW = MT == FMT_BF16 ? 256 : 128;        // bytes per K row (LDS format)
  static constexpr int VROW = VF == FMT_BF16 ? 256 : 128;
  static constexpr int KGROW = KF == FMT_BF16 ? 256 : 128;       // bytes per K row in HBM
  // LDS rows are padded by one 16-byte chunk: consecutive rows start one
  // chunk apart in the 64 x 4-byte banks, so the 16 rows an MFMA operand read
  // touches at a time, and the 8 rows of a transposing read, hit distinct banks
  // while every lane reads at a fixed offset from its own base address.
  static constexpr int KP = KROW + 16, VP = VROW + 16;
  static constexpr int K_BUF = kSub * KP, V_BUF = kSub * VP;
  static constexpr int LDS_BYTES = 2 * (K_BUF + V_BUF);
  static constexpr bool K_DMA = KROW == KGROW;                   // HBM -> LDS without conversion
  static constexpr int NT = NW * 64;
  static constexpr int K_CPR = KROW / 16, KP_CPR = KP / 16;      // 16-byte chunks per row
  static constexpr int V_CPR = VROW / 16, VP_CPR = VP / 16;
  static constexpr int K_DMA_OPS = K_BUF / 1024;                 // 1 KB per wave-wide DMA
  static constexpr int V_DMA_OPS = V_BUF / 1024;
  static_assert(K_BUF % 1024 == 0 && V_BUF % 1024 == 0, "DMA granularity");
  static constexpr int KG_CPR = KGROW / 16;                      // register path (widening K)
  static constexpr int K_REG_LOADS = K_DMA ? 0 : kSub * KG_CPR / NT;
  static_assert(K_DMA || kSub * KG_CPR % NT == 0, "tile / thread mismatch");
  static_assert(!(KF == FMT_E4M3 && QF == FMT_INT8), "unsupported");
  static_assert(QF == KF || (QF == FMT_BF16 && KF == FMT_E4M3), "unsupported");
};

// Q operand registers of one lane (query l % 32, contraction slice of group g).
template <int MT> struct QRegs;
template <> struct QRegs<FMT_BF16> { v8bf r[8]; };  // d = 64g + 8t .. +8, t = 0..7
template <> struct QRegs<FMT_E4M3> { v8i r[2]; };   // bytes 64t + 32g .. +32
template <> struct QRegs<FMT_INT8> { v4i r[4]; };   // bytes 32t + 16g .. +16

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

template <class C>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(FMHA_WAVES_PER_EU))) void fwd_kernel(FwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int g = lane >> 5;
  const int m32 = lane & 31;

  // ---- which (batch, head, query tile) this workgroup owns
  const int qtile = 32 * C::NW;
  const int nqt = (a.Sq + qtile - 1) / qtile;
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  int qt = lin % nqt;
  if (a.causal) qt = nqt - 1 - qt;  // longest causal rows first
  const int bh = lin / nqt;
  const int hq = bh % a.Hq;
  const int b = bh / a.Hq;
  const int hk = hq / a.group;
  const int q0 = qt * qtile;
  const int q0w = q0 + 32 * wave;
  const int qi = q0w + m32;                // this lane's query row
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
  auto next_sub = [&](int t) {
    if (C::MASKED) {
      while (t < n_sub && mask_row[t / a.mask_kv_sub] == 0) ++t;
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
  // Byte offset of token `key`, clamped into the sequence (rows past the end
  // load the last token, whose pairs are masked); a page-table entry outside
  // the pool reads page 0.
  auto token_off = [&](int key, const int64_t sb, const int64_t ss) -> int64_t {
    key = min(key, a.Skv - 1);
    if (!C::PAGED) return (int64_t)key * ss;
    int page = pt_row[key >> page_shift];
    page = (unsigned)page < (unsigned)a.num_pages ? page : 0;
    return (int64_t)page * sb + (int64_t)(key & (a.page_size - 1)) * ss;
  };
  uint8_t* const kbuf0 = smem;
  uint8_t* const vbuf0 = smem + 2 * C::K_BUF;
  // Every wave issues the same number of wave-wide DMA operations per
  // sub-tile (slots past the tile repeat its last operation: identical bytes
  // to the same place), so the loop body has no per-wave branches.  Per-lane
  // source offsets within a tile are fixed; contiguous K/V go through a
  // buffer resource whose range ends at the last token, so rows past the end
  // of the sequence read as zeros.  K rows are stored in MFMA row order: LDS
  // row 32T + m holds key 32T + sigma(m).
  constexpr int KSL = C::K_DMA ? (C::K_DMA_OPS + C::NW - 1) / C::NW : 0;
  constexpr int VSL = (C::V_DMA_OPS + C::NW - 1) / C::NW;
  uint32_t k_src[KSL > 0 ? KSL : 1], v_src[VSL];
  int k_row[KSL > 0 ? KSL : 1], v_row[VSL];  // key within the tile (paged path)
#pragma unroll
  for (int sl = 0; sl < KSL; ++sl) {
    const int j = min(wave + sl * C::NW, C::K_DMA_OPS - 1);
    const int cid = j * 64 + lane;
    const int row = cid / C::KP_CPR;
    int ch = cid % C::KP_CPR;
    ch = ch < C::K_CPR ? ch : 0;  // the pad chunk: any valid bytes
    k_row[sl] = 32 * (row >> 5) + sigma(row & 31);
    k_src[sl] = (uint32_t)(k_row[sl] * a.k_ss) + ch * 16;
    if (C::PAGED) k_src[sl] = ch * 16;
  }
#pragma unroll
  for (int sl = 0; sl < VSL; ++sl) {
    const int j = min(wave + sl * C::NW, C::V_DMA_OPS - 1);
    const int cid = j * 64 + lane;
    const int row = cid / C::VP_CPR;
    int ch = cid % C::VP_CPR;
    ch = ch < C::V_CPR ? ch : 0;
    v_row[sl] = row;
    v_src[sl] = (uint32_t)(row * a.v_ss) + ch * 16;
    if (C::PAGED) v_src[sl] = ch * 16;
  }
  auto tile_rsrc = [&](const uint8_t* base, int64_t ss, int kv0) {
    const uint64_t rem = (uint64_t)(a.Skv - kv0) * (uint64_t)ss;
    const int nrec = rem > 0x7FFFFFFFull ? 0x7FFFFFFF : (int)rem;
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base + (int64_t)kv0 * ss), 0, nrec, 0x00020000);
  };
  auto dma_k = [&](int t, int buf) {
    if constexpr (C::K_DMA) {
      const int kv0 = t * kSub;
      uint8_t* dst = kbuf0 + buf * C::K_BUF;
      if constexpr (!C::PAGED) {
        const auto rs = tile_rsrc(kbase, a.k_ss, kv0);
#pragma unroll
        for (int sl = 0; sl < KSL; ++sl) {
          const int j = min(wave + sl * C::NW, C::K_DMA_OPS - 1);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, FMHA_LDS(void, dst + j * 1024), 16, (int)k_src[sl], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int sl = 0; sl < KSL; ++sl) {
          const int j = min(wave + sl * C::NW, C::K_DMA_OPS - 1);
          const uint8_t* src = kbase + token_off(kv0 + k_row[sl], a.k_sb, a.k_ss) + k_src[sl];
          __builtin_amdgcn_global_load_lds(src, FMHA_LDS(void, dst + j * 1024), 16, 0, 0);
        }
      }
    }
  };
  auto dma_v = [&](int t, int buf) {
    const int kv0 = t * kSub;
    uint8_t* dst = vbuf0 + buf * C::V_BUF;
    if constexpr (!C::PAGED) {
      const auto rs = tile_rsrc(vbase, a.v_ss, kv0);
#pragma unroll
      for (int sl = 0; sl < VSL; ++sl) {
        const int j = min(wave + sl * C::NW, C::V_DMA_OPS - 1);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, FMHA_LDS(void, dst + j * 1024), 16, (int)v_src[sl], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int sl = 0; sl < VSL; ++sl) {
        const int j = min(wave + sl * C::NW, C::V_DMA_OPS - 1);
        const uint8_t* src = vbase + token_off(kv0 + v_row[sl], a.v_sb, a.v_ss) + v_src[sl];
        __builtin_amdgcn_global_load_lds(src, FMHA_LDS(void, dst + j * 1024), 16, 0, 0);
      }
    }
  };
  // Register path for K when its LDS format differs (E4M3 widened to bf16).
  uint4 kreg[C::K_REG_LOADS > 0 ? C::K_REG_LOADS : 1];
  auto load_k_regs = [&](int t) {
    const int kv0 = t * kSub;
#pragma unroll
    for (int i = 0; i < C::K_REG_LOADS; ++i) {
      const int id = tid + i * C::NT;
      const int row = id / C::KG_CPR, cc = id % C::KG_CPR;
      const int key = kv0 + 32 * (row >> 5) + sigma(row & 31);
      kreg[i] = *(const uint4*)(kbase + token_off(key, a.k_sb, a.k_ss) + cc * 16);
    }
  };
  auto store_k_regs = [&](int buf) {
    uint8_t* dst = kbuf0 + buf * C::K_BUF;
#pragma unroll
    for (int i = 0; i < C::K_REG_LOADS; ++i) {
      const int id = tid + i * C::NT;
      const int row = id / C::KG_CPR, cc = id % C::KG_CPR;
      // E4M3 codes widened to bf16 (exact: 4 significant bits).
      uint32_t w[4] = {kreg[i].x, kreg[i].y, kreg[i].z, kreg[i].w};
      uint32_t o[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v2f lo = unpack_e4m3<false>((int)w[j]);
        v2f hi = unpack_e4m3<true>((int)w[j]);
        o[2 * j] = (__float_as_uint(lo.x) >> 16) | (__float_as_uint(lo.y) & 0xFFFF0000u);
        o[2 * j + 1] = (__float_as_uint(hi.x) >> 16) | (__float_as_uint(hi.y) & 0xFFFF0000u);
      }
      uint8_t* rp = dst + row * C::KP + 32 * cc;
      *(uint4*)(rp) = make_uint4(o[0], o[1], o[2], o[3]);
      *(uint4*)(rp + 16) = make_uint4(o[4], o[5], o[6], o[7]);
    }
  };

  // ---- Q tile into registers (B operand of S^T = K Q^T)
  QRegs<C::MT> q;
  {
    const bool ok = qi < a.Sq;
    const uint8_t* qp = a.q + (int64_t)b * a.q_sb + (int64_t)hq * a.q_sh + (int64_t)(ok ? qi : 0) * a.q_ss;
    if constexpr (C::MT == FMT_BF16) {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        uint4 u = ok ? *(const uint4*)(qp + 128 * g + 16 * t) : make_uint4(0, 0, 0, 0);
        q.r[t] = __builtin_bit_cast(v8bf, u);
      }
    } else if constexpr (C::MT == FMT_E4M3) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        uint4 u0 = ok ? *(const uint4*)(qp + 64 * t + 32 * g) : make_uint4(0, 0, 0, 0);
        uint4 u1 = ok ? *(const uint4*)(qp + 64 * t + 32 * g + 16) : make_uint4(0, 0, 0, 0);
        q.r[t] = v8i{(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w, (int)u1.x, (int)u1.y, (int)u1.z, (int)u1.w};
      }
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        uint4 u = ok ? *(const uint4*)(qp + 32 * t + 16 * g) : make_uint4(0, 0, 0, 0);
        q.r[t] = v4i{(int)u.x, (int)u.y, (int)u.z, (int)u.w};
      }
    }
  }
  float sq = 1.0f;
  if (C::QS) sq = a.sfs_q[((int64_t)b * a.Hq + hq) * a.nblk_q + min(q0w, max(a.Sq - 1, 0)) / 64];
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
  if constexpr (C::MT == FMT_BF16) kb_lane = m32 * C::KP + 128 * g;
  else if constexpr (C::MT == FMT_E4M3) kb_lane = m32 * C::KP + 32 * g;
  else kb_lane = m32 * C::KP + 16 * g;
  const int tr_G = lane >> 4;
  int vb_lane;
  if constexpr (C::VF == FMT_E4M3)  // source row 16g + r, column 16(G%2) + 8h
    vb_lane = (16 * (tr_G >> 1) + ((lane & 15) >> 1)) * C::VP + 16 * (tr_G & 1) + 8 * (lane & 1);
  else  // bf16 V: source row 16g + r, byte column 32(G%2) + 8h'
    vb_lane = (16 * (tr_G >> 1) + ((lane & 15) >> 2)) * C::VP + 32 * (tr_G & 1) + 8 * (lane & 3);

  // S^T for one sub-tile from the K buffer `kb`.  All K operand reads are
  // issued before the first MFMA, so each MFMA waits only for its own operand
  // and the LDS latency hides behind the MFMAs ahead of it.
  auto qk = [&](const uint8_t* kb) {
    SAcc<C::MT> acc;
    const uint8_t* kp = kb + kb_lane;
    if constexpr (C::MT == FMT_BF16 && C::PAGED) {
      // (register-lean variant for the paged path, whose address state
      // already takes more registers)
#pragma unroll
      for (int T = 0; T < 2; ++T) {
        acc.r[T] = v16f{};
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) {
          const uint4 u = *(const uint4*)(kp + 32 * T * C::KP + 16 * tt);
          acc.r[T] = mfma_bf16(__builtin_bit_cast(v8bf, u), q.r[tt], acc.r[T]);
        }
      }
    } else if constexpr (C::MT == FMT_BF16) {
      uint4 kr[2][8];
#pragma unroll
      for (int T = 0; T < 2; ++T)
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) kr[T][tt] = *(const uint4*)(kp + 32 * T * C::KP + 16 * tt);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int T = 0; T < 2; ++T) {
        acc.r[T] = v16f{};
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) acc.r[T] = mfma_bf16(__builtin_bit_cast(v8bf, kr[T][tt]), q.r[tt], acc.r[T]);
      }
    } else if constexpr (C::MT == FMT_E4M3) {
      uint4 kr[2][4];
#pragma unroll
      for (int T = 0; T < 2; ++T)
#pragma unroll
        for (int i = 0; i < 4; ++i) kr[T][i] = *(const uint4*)(kp + 32 * T * C::KP + 64 * (i >> 1) + 16 * (i & 1));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int T = 0; T < 2; ++T) {
        acc.r[T] = v16f{};
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const uint4 u0 = kr[T][2 * tt], u1 = kr[T][2 * tt + 1];
          const v8i av = {(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w, (int)u1.x, (int)u1.y, (int)u1.z, (int)u1.w};
          acc.r[T] = mfma_f8(av, q.r[tt], acc.r[T]);
        }
      }
    } else {
      uint4 kr[2][4];
#pragma unroll
      for (int T = 0; T < 2; ++T)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) kr[T][tt] = *(const uint4*)(kp + 32 * T * C::KP + 32 * tt);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int T = 0; T < 2; ++T) {
        acc.r[T] = v16i{};
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const uint4 u = kr[T][tt];
          acc.r[T] = mfma_i8(v4i{(int)u.x, (int)u.y, (int)u.z, (int)u.w}, q.r[tt], acc.r[T]);
        }
      }
    }
    return acc;
  };

  // ---- per-lane state.  O^T (4 tiles of 32 d x 32 queries) is kept in units
  // of the reference V scale `sv_ref`: before a sub-tile's PV product is
  // accumulated, O is multiplied by alpha_row * sv_ref / sv_tile (one multiply
  // folds the lazy rescale and the change of V block scale), then the MFMA
  // accumulates codes x codes directly.
  v16f o[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) o[d] = v16f{};
  float m_run = -kInf;
  float den = 0.0f;
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

  // softmax + P requantisation + PV for sub-tile t from S^T `acc` and V buffer `vb`
  auto softmax_pv = [&](const SAcc<C::MT>& acc, int t, const uint8_t* vb, auto edge_tag, auto clamp_tag,
                        auto direct_tag) {
    constexpr bool EDGE = decltype(edge_tag)::value;
    constexpr bool CLAMP = decltype(clamp_tag)::value;
    constexpr bool DIRECT = decltype(direct_tag)::value;
    const int kv0 = t * kSub;
    // V^T operands of the four d-tiles, read before the softmax so their LDS
    // latency hides behind it: rows 32(cq/2) + 8(cq%2) further down and
    // columns 32d further right of the lane's base
    // (hoisted only where registers allow it: the bf16-QK contiguous path)
    constexpr bool HOIST_V = C::VF == FMT_E4M3 && C::MT == FMT_BF16 && !C::PAGED;
    v8i vop[4];
    auto read_v = [&]() {
      const uint8_t* vp = vb + vb_lane;
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int cq = 0; cq < 4; ++cq) {
          const v2i r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              FMHA_LDS(v2i, vp + (32 * (cq >> 1) + 8 * (cq & 1)) * C::VP + 32 * d));
          vop[d][2 * cq] = r[0];
          vop[d][2 * cq + 1] = r[1];
        }
    };
    if constexpr (HOIST_V) read_v();
    float s[32];
#pragma unroll
    for (int e = 0; e < 32; ++e) s[e] = (float)acc.r[e >> 4][e & 15];
    if constexpr (EDGE) {
      // s[e] is key kv0 + 32(e/16) + 16g + e%16
      const int lim = a.causal ? min(a.Skv, qi + causal_off + 1) : a.Skv;
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const int key = kv0 + 32 * (e >> 4) + 16 * g + (e & 15);
        s[e] = key < lim ? s[e] : -kInf;
      }
    }
    float mx = fmaxf(s[0], s[1]);
#pragma unroll
    for (int e = 2; e < 32; e += 2) mx = fmaxf(mx, fmaxf(s[e], s[e + 1]));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float c = C::KS ? c_q * sk_t : c_q;
    const float tmax = mx * c;  // c > 0, so the maximum commutes with the scale
    const bool trig = (tmax != -kInf) && (m_run == -kInf || tmax - m_run > a.tau);
    // 2^(m - t) is 0 for an unset m (m = -inf); rows that do not trigger keep 1
    const float e_mt = __builtin_amdgcn_exp2f(m_run - tmax);
    const float alpha = trig ? e_mt : 1.0f;
    m_run = trig ? tmax : m_run;
    den *= alpha;
    const float negm = m_run == -kInf ? -kInf : -(m_run + log2sp);
    // Rescale O: lazy factor and (fast path) change of V reference scale.
    if constexpr (C::VS && DIRECT) {
      const float fo = alpha * (sv_ref / sv_t);
      sv_ref = sv_t;
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[d][r] *= fo;
    } else {
      if (__ballot(trig) != 0) {
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[d][r] *= alpha;
      }
    }
    // P = 2^(s2 - m) / sp, clamped to the E4M3 range only where P / sp can
    // reach it (sfs_p given or tau above log2(448))
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      s[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e], c, negm));
      if constexpr (CLAMP) s[e] = fminf(s[e], 448.0f);
    }
    if constexpr (C::VF == FMT_E4M3) {
      v8i pb;
      float dsum = 0.0f;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        int pk = pack_e4m3<false>(s[4 * w], s[4 * w + 1], 0);
        pk = pack_e4m3<true>(s[4 * w + 2], s[4 * w + 3], pk);
        pb[w] = pk;
        const v2f lo = unpack_e4m3<false>(pk);
        const v2f hi = unpack_e4m3<true>(pk);
        dsum += (lo.x + lo.y) + (hi.x + hi.y);
      }
      den += dsum;
      if constexpr (!HOIST_V) read_v();
      if constexpr (!C::VS || DIRECT) {
#pragma unroll
        for (int d = 0; d < 4; ++d) o[d] = mfma_f8(vop[d], pb, o[d]);
      } else {
        const float f = sv_t / sv_ref;  // reference stays at 1
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const v16f part = mfma_f8(vop[d], pb, v16f{});
#pragma unroll
          for (int r = 0; r < 16; ++r) o[d][r] = __builtin_fmaf(part[r], f, o[d][r]);
        }
      }
    } else {
      // bf16 P and V (V unscaled).
      v8bf pbf[4];
      float dsum = 0.0f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t lo = f32_to_bf16_bits(s[8 * kk + 2 * j]);
          const uint32_t hi = f32_to_bf16_bits(s[8 * kk + 2 * j + 1]);
          w[j] = lo | (hi << 16);
          dsum += bf16_bits_to_f32(lo) + bf16_bits_to_f32(hi);
        }
        pbf[kk] = __builtin_bit_cast(v8bf, make_uint4(w[0], w[1], w[2], w[3]));
      }
      den += dsum;
      const uint8_t* vp = vb + vb_lane;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
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
          o[d] = mfma_bf16(__builtin_bit_cast(v8bf, make_uint4(w[0], w[1], w[2], w[3])), pbf[kk], o[d]);
        }
      }
    }
  };

  // ---- main loop over 64-key sub-tiles, K/V double-buffered in LDS.  Per
  // sub-tile a wave runs S^T = K Q^T (MFMA), the softmax (VALU), then
  // O^T += V^T P^T (MFMA); an MFMA holds its wave's issue for its whole
  // duration on this hardware, so MFMA/VALU overlap comes from the second
  // wave on the SIMD (another workgroup) being in the opposite phase.
  int tc = next_sub(0);
  if (tc < n_sub) {
    dma_k(tc, 0);
    dma_v(tc, 0);
    if constexpr (!C::K_DMA) {
      load_k_regs(tc);
      store_k_regs(0);
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's DMA has landed
  __syncthreads();
  int buf = 0;
  auto step = [&](auto edge_tag, auto clamp_tag, auto direct_tag) {
    fetch_scales(tc);
    const int tn = next_sub(tc + 1);
    if (tn < n_sub) {
      dma_k(tn, buf ^ 1);
      dma_v(tn, buf ^ 1);
      if constexpr (!C::K_DMA) load_k_regs(tn);
    }
    const SAcc<C::MT> acc = qk(kbuf0 + buf * C::K_BUF);
    softmax_pv(acc, tc, vbuf0 + buf * C::V_BUF, edge_tag, clamp_tag, direct_tag);
    if constexpr (!C::K_DMA) {
      if (tn < n_sub) store_k_regs(buf ^ 1);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's DMA has landed
    __syncthreads();
    buf ^= 1;
    tc = tn;
  };
  auto run = [&](auto clamp_tag, auto direct_tag) {
    // sub-tiles valid for every pair of the workgroup first, then the edge ones
    if constexpr (!C::MASKED) {
      while (tc < n_sub && tc < full_end) step(std::false_type{}, clamp_tag, direct_tag);
    }
    while (tc < n_sub) step(std::true_type{}, clamp_tag, direct_tag);
  };
  const bool clamp = C::VF == FMT_E4M3 && a.clamp_p;
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

  // ---- epilogue: O = num / den in bf16; rows without a valid key give 0
  const float dt = den + __shfl_xor(den, 32, 64);
  const float inv = dt > 0.0f ? sv_ref / dt : 0.0f;
  if (qi >= a.Sq) return;
  uint8_t* op = a.o + (int64_t)b * a.o_sb + (int64_t)hq * a.o_sh + (int64_t)qi * a.o_ss;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
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
#endif
}

template <class C>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  const int qtile = 32 * C::NW;
  const int64_t tiles = (int64_t)((a.Sq + qtile - 1) / qtile) * a.Hq * a.B;
  if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  dim3 grid((unsigned)tiles);
  const size_t lds = (size_t)C::LDS_BYTES;
  static bool configured = false;  // benign race: the attribute is idempotent
  if (!configured) {
    hipError_t e = hipFuncSetAttribute((const void*)fwd_kernel<C>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    configured = true;
  }
  hipLaunchKernelGGL(fwd_kernel<C>, grid, dim3(C::NT), lds, stream, a);
  return hipGetLastError();
}

}  // namespace

bool fwd_supported(const FwdKey& k) {
  if (k.qf == FMT_BF16 && k.kf == FMT_BF16 && k.vf == FMT_BF16)
    return !k.q_scaled && !k.k_scaled && !k.v_scaled;
  if (k.qf == FMT_INT8 && k.kf == FMT_INT8 && k.vf == FMT_E4M3) return k.q_scaled && k.k_scaled && k.v_scaled;
  if (k.qf == FMT_BF16 && k.kf == FMT_BF16 && k.vf == FMT_E4M3) return !k.q_scaled && !k.k_scaled;
  if (k.qf == FMT_E4M3 && k.kf == FMT_E4M3 && k.vf == FMT_E4M3) return k.q_scaled && k.k_scaled && k.v_scaled;
  if (k.qf == FMT_BF16 && k.kf == FMT_E4M3 && k.vf == FMT_E4M3) return !k.q_scaled && k.k_scaled && k.v_scaled;
  return false;
}

template <int QF, int KF, int VF, bool QS, bool KS, bool VS>
static hipError_t dispatch_layout(const FwdKey& k, const FwdArgs& a, hipStream_t s) {
  if (k.masked) {
    if (k.paged) return launch<Cfg<QF, KF, VF, QS, KS, VS, true, true, 2>>(a, s);
    return launch<Cfg<QF, KF, VF, QS, KS, VS, true, false, 2>>(a, s);
  }
  if (k.paged) return launch<Cfg<QF, KF, VF, QS, KS, VS, false, true, kDenseWaves>>(a, s);
  return launch<Cfg<QF, KF, VF, QS, KS, VS, false, false, kDenseWaves>>(a, s);
}

hipError_t launch_fwd(const FwdKey& k, const FwdArgs& a, hipStream_t s) {
  if (!fwd_supported(k)) return hipErrorInvalidValue;
  if (k.qf == FMT_BF16 && k.kf == FMT_BF16 && k.vf == FMT_BF16)
    return dispatch_layout<FMT_BF16, FMT_BF16, FMT_BF16, false, false, false>(k, a, s);
  if (k.qf == FMT_INT8)
    return dispatch_layout<FMT_INT8, FMT_INT8, FMT_E4M3, true, true, true>(k, a, s);
  if (k.qf == FMT_BF16 && k.kf == FMT_BF16) {
    if (k.v_scaled) return dispatch_layout<FMT_BF16, FMT_BF16, FMT_E4M3, false, false, true>(k, a, s);
    return dispatch_layout<FMT_BF16, FMT_BF16, FMT_E4M3, false, false, false>(k, a, s);
  }
  if (k.qf == FMT_E4M3)
    return dispatch_layout<FMT_E4M3, FMT_E4M3, FMT_E4M3, true, true, true>(k, a, s);
  return dispatch_layout<FMT_BF16, FMT_E4M3, FMT_E4M3, false, true, true>(k, a, s);
}

}  // namespace fmha
