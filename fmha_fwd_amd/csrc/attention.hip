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
#include "device_common.h"
#include "fmha_internal.h"

namespace fmha {
namespace {

constexpr int kSub = 64;  // keys per sub-tile: lazy-decision and V-scale unit
constexpr float kInf = __builtin_huge_valf();

// Key held by row m of a 32-key MFMA tile: lane group g of the S^T result
// then owns keys 16g .. 16g + 15 in its 16 accumulator registers.
__device__ __forceinline__ int sigma(int m) {
  return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3);
}
// XOR swizzles of 16-byte chunks inside an LDS row (row index = key in tile),
// chosen so that the 16 rows one MFMA-operand read touches at a time, and the
// 8 consecutive rows of a transposing read, fall in distinct banks.
__device__ __forceinline__ int swz256(int key) { return (key & 7) | ((key & 16) >> 1); }
__device__ __forceinline__ int swz128(int key) { return ((key >> 1) & 3) | ((key >> 2) & 4); }

template <int KROW>
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * KROW + ((chunk ^ (KROW == 256 ? swz256(row) : swz128(row))) << 4);
}

template <int QF_, int KF_, int VF_, bool QS_, bool KS_, bool VS_, bool MASKED_, bool PAGED_, int NW_>
struct Cfg {
  static constexpr int QF = QF_, KF = KF_, VF = VF_, NW = NW_;
  static constexpr bool QS = QS_, KS = KS_, VS = VS_, MASKED = MASKED_, PAGED = PAGED_;
  static constexpr int MT = QF;                                  // QK operand format
  static constexpr int KROW = MT == FMT_BF16 ? 256 : 128;        // LDS bytes per K row
  static constexpr int VROW = VF == FMT_BF16 ? 256 : 128;
  static constexpr int KGROW = KF == FMT_BF16 ? 256 : 128;       // HBM bytes per K row
  static constexpr int K_TILE = kSub * KROW;
  static constexpr int V_TILE = kSub * VROW;
  static constexpr int STAGE = K_TILE + V_TILE;
  static constexpr int NT = NW * 64;
  static constexpr int K_CPR = KGROW / 16;                       // 16-byte chunks per row
  static constexpr int V_CPR = VROW / 16;
  static constexpr int K_LOADS = kSub * K_CPR / NT;
  static constexpr int V_LOADS = kSub * V_CPR / NT;
  static_assert(kSub * K_CPR % NT == 0 && kSub * V_CPR % NT == 0, "tile / thread mismatch");
  static_assert(!(KF == FMT_E4M3 && QF == FMT_INT8), "unsupported");
  static_assert(QF == KF || (QF == FMT_BF16 && KF == FMT_E4M3), "unsupported");
};

// Q operand registers of one lane (query l % 32, contraction slice of group g).
template <int MT> struct QRegs;
template <> struct QRegs<FMT_BF16> { v8bf r[8]; };  // d = 64g + 8t .. +8, t = 0..7
template <> struct QRegs<FMT_E4M3> { v8i r[2]; };   // bytes 64t + 32g .. +32
template <> struct QRegs<FMT_INT8> { v4i r[4]; };   // bytes 32t + 16g .. +16

template <class C>
__global__ __launch_bounds__(C::NT) void fwd_kernel(FwdArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;
  const int m32 = lane & 31;

  const int b = blockIdx.z;
  const int hq = blockIdx.y;
  const int hk = hq / a.group;
  const int q0 = blockIdx.x * (32 * C::NW);
  const int q0w = q0 + 32 * wave;
  const int qi = q0w + m32;                // this lane's query row
  const int causal_off = a.Skv - a.Sq;     // key j visible iff j <= i + causal_off

  // ---- key range of the workgroup and of this wave
  int kv_end = a.Skv;
  if (a.causal) {
    const int qlast = min(q0 + 32 * C::NW, a.Sq) - 1;
    kv_end = min(kv_end, max(qlast + causal_off + 1, 0));
  }
  const int n_sub = (kv_end + kSub - 1) / kSub;
  int kv_end_w = a.Skv;
  if (a.causal) kv_end_w = min(kv_end_w, max(min(q0w + 31, a.Sq - 1) + causal_off + 1, 0));
  const bool wave_live = q0w < a.Sq;

  const uint8_t* mask_row = nullptr;
  if (C::MASKED) mask_row = a.mask + (int64_t)b * a.m_sb + (int64_t)hq * a.m_sh + (int64_t)(q0 / 64) * a.m_sqb;
  auto next_sub = [&](int t) {
    if (C::MASKED) {
      while (t < n_sub && mask_row[t / a.mask_kv_sub] == 0) ++t;
    }
    return t;
  };

  // ---- global -> register staging of one sub-tile of K and V
  const uint8_t* kbase = a.k + (int64_t)hk * a.k_sh;
  const uint8_t* vbase = a.v + (int64_t)hk * a.v_sh;
  const int32_t* pt_row = C::PAGED ? a.page_table + (int64_t)b * a.pt_sb : nullptr;
  if (!C::PAGED) {
    kbase += (int64_t)b * a.k_sb;
    vbase += (int64_t)b * a.v_sb;
  }
  const int page_shift = C::PAGED ? __builtin_ctz((unsigned)a.page_size) : 0;
  auto token_off = [&](int key, const int64_t sb, const int64_t ss, bool& ok) -> int64_t {
    if (!C::PAGED) {
      ok = key < a.Skv;
      return (int64_t)key * ss;
    }
    ok = false;
    if (key >= a.Skv) return 0;
    const int page = pt_row[key >> page_shift];
    ok = (unsigned)page < (unsigned)a.num_pages;
    return ok ? (int64_t)page * sb + (int64_t)(key & (a.page_size - 1)) * ss : 0;
  };

  uint4 kreg[C::K_LOADS];
  uint4 vreg[C::V_LOADS];
  auto load_tile = [&](int t) {
    const int kv0 = t * kSub;
#pragma unroll
    for (int i = 0; i < C::K_LOADS; ++i) {
      const int id = tid + i * C::NT;
      const int row = id / C::K_CPR, cc = id % C::K_CPR;
      bool ok;
      const int64_t off = token_off(kv0 + row, a.k_sb, a.k_ss, ok);
      kreg[i] = ok ? *(const uint4*)(kbase + off + cc * 16) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < C::V_LOADS; ++i) {
      const int id = tid + i * C::NT;
      const int row = id / C::V_CPR, cc = id % C::V_CPR;
      bool ok;
      const int64_t off = token_off(kv0 + row, a.v_sb, a.v_ss, ok);
      vreg[i] = ok ? *(const uint4*)(vbase + off + cc * 16) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_tile = [&](int stage) {
    uint8_t* ks = smem + stage * C::STAGE;
    uint8_t* vs = ks + C::K_TILE;
#pragma unroll
    for (int i = 0; i < C::K_LOADS; ++i) {
      const int id = tid + i * C::NT;
      const int row = id / C::K_CPR, cc = id % C::K_CPR;
      if (C::KF == C::MT) {
        *(uint4*)(ks + lds_off<C::KROW>(row, cc)) = kreg[i];
      } else {
        // E4M3 codes widened to bf16 (exact: 4 significant bits) for the
        // bf16 x bf16 product with a bf16 Q.
        uint32_t w[4] = {kreg[i].x, kreg[i].y, kreg[i].z, kreg[i].w};
        uint32_t o[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v2f lo = unpack_e4m3<false>((int)w[j]);
          v2f hi = unpack_e4m3<true>((int)w[j]);
          o[2 * j] = (__float_as_uint(lo.x) >> 16) | (__float_as_uint(lo.y) & 0xFFFF0000u);
          o[2 * j + 1] = (__float_as_uint(hi.x) >> 16) | (__float_as_uint(hi.y) & 0xFFFF0000u);
        }
        *(uint4*)(ks + lds_off<C::KROW>(row, 2 * cc)) = make_uint4(o[0], o[1], o[2], o[3]);
        *(uint4*)(ks + lds_off<C::KROW>(row, 2 * cc + 1)) = make_uint4(o[4], o[5], o[6], o[7]);
      }
    }
#pragma unroll
    for (int i = 0; i < C::V_LOADS; ++i) {
      const int id = tid + i * C::NT;
      const int row = id / C::V_CPR, cc = id % C::V_CPR;
      *(uint4*)(vs + lds_off<C::VROW>(row, cc)) = vreg[i];
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

  // ---- per-lane state: O^T (4 tiles of 32 d x 32 queries), row max, denominator
  v16f o[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) o[d] = v16f{};
  float m_run = -kInf;
  float den = 0.0f;

  // Per-lane LDS offsets of the MFMA operands (stage-relative).
  const int krow0 = sigma(m32);  // K row of this lane in tile T = 0 (T = 1 adds 32 rows)
  // V^T transposing reads: source lane supplies row key(c, r) and column block.
  const int tr_G = lane >> 4;
  const int tr_g = tr_G >> 1;

  // ---- main loop over 64-key sub-tiles
  int t = next_sub(0);
  if (t < n_sub) {
    load_tile(t);
    store_tile(0);
  }
  __syncthreads();
  int stage = 0;
  while (t < n_sub) {
    const int tn = next_sub(t + 1);
    if (tn < n_sub) load_tile(tn);
    const int kv0 = t * kSub;
    if (wave_live && kv0 < kv_end_w) {
      const uint8_t* ks = smem + stage * C::STAGE;
      const uint8_t* vs = ks + C::K_TILE;
      // -- S^T = K Q^T for the two 32-key tiles
      float s[32];
      if constexpr (C::MT == FMT_INT8) {
        v16i acc[2] = {v16i{}, v16i{}};
#pragma unroll
        for (int T = 0; T < 2; ++T) {
          const int row = 32 * T + krow0;
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
            uint4 u = *(const uint4*)(ks + lds_off<C::KROW>(row, 2 * tt + g));
            acc[T] = mfma_i8(v4i{(int)u.x, (int)u.y, (int)u.z, (int)u.w}, q.r[tt], acc[T]);
          }
        }
#pragma unroll
        for (int e = 0; e < 32; ++e) s[e] = (float)acc[e >> 4][e & 15];
      } else {
        v16f acc[2] = {v16f{}, v16f{}};
#pragma unroll
        for (int T = 0; T < 2; ++T) {
          const int row = 32 * T + krow0;
          if constexpr (C::MT == FMT_BF16) {
#pragma unroll
            for (int tt = 0; tt < 8; ++tt) {
              uint4 u = *(const uint4*)(ks + lds_off<C::KROW>(row, 8 * g + tt));
              acc[T] = mfma_bf16(__builtin_bit_cast(v8bf, u), q.r[tt], acc[T]);
            }
          } else {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
              uint4 u0 = *(const uint4*)(ks + lds_off<C::KROW>(row, 4 * tt + 2 * g));
              uint4 u1 = *(const uint4*)(ks + lds_off<C::KROW>(row, 4 * tt + 2 * g + 1));
              v8i av = {(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w, (int)u1.x, (int)u1.y, (int)u1.z, (int)u1.w};
              acc[T] = mfma_f8(av, q.r[tt], acc[T]);
            }
          }
        }
#pragma unroll
        for (int e = 0; e < 32; ++e) s[e] = acc[e >> 4][e & 15];
      }
      // -- validity of (query, key) pairs on edge sub-tiles: s[e] is key
      //    kv0 + 32*(e/16) + 16*g + e%16
      const bool edge = (kv0 + kSub > a.Skv) || (a.causal && kv0 + kSub - 1 > q0w + causal_off);
      if (edge) {
        const int lim = a.causal ? min(a.Skv, qi + causal_off + 1) : a.Skv;
#pragma unroll
        for (int e = 0; e < 32; ++e) {
          const int key = kv0 + 32 * (e >> 4) + 16 * g + (e & 15);
          if (key >= lim) s[e] = -kInf;
        }
      }
      // -- row maximum (raw units), lazy decision (log2 units)
      float mx = s[0];
#pragma unroll
      for (int e = 1; e < 32; ++e) mx = fmaxf(mx, s[e]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      float c = a.scale_log2 * sq;
      if (C::KS) c *= sk_row[t];
      const float tmax = mx * c;  // c > 0, so the maximum commutes with the scale
      const bool trig = (tmax != -kInf) && (m_run == -kInf || tmax - m_run > a.tau);
      if (__ballot(trig) != 0) {
        const float alpha = trig ? (m_run == -kInf ? 0.0f : __builtin_amdgcn_exp2f(m_run - tmax)) : 1.0f;
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[d][r] *= alpha;
        den *= alpha;
        if (trig) m_run = tmax;
      }
      const float negm = m_run == -kInf ? -kInf : -(m_run + log2sp);
      float p[32];
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e], c, negm));
        if (C::VF == FMT_E4M3 && a.clamp_p) p[e] = fminf(p[e], 448.0f);
      }
      // -- P to the PV operand format, denominator from the quantised values,
      //    then O^T += V^T P^T
      if constexpr (C::VF == FMT_E4M3) {
        v8i pb;
        float dsum = 0.0f;
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          int pk = pack_e4m3<false>(p[4 * w], p[4 * w + 1], 0);
          pk = pack_e4m3<true>(p[4 * w + 2], p[4 * w + 3], pk);
          pb[w] = pk;
          const v2f lo = unpack_e4m3<false>(pk);
          const v2f hi = unpack_e4m3<true>(pk);
          dsum += (lo.x + lo.y) + (hi.x + hi.y);
        }
        den += dsum;
        const float svv = C::VS ? sv_row[t] : 1.0f;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          v8i av;
#pragma unroll
          for (int cq = 0; cq < 4; ++cq) {
            // source row: key 32(cq/2) + 16 g + 8(cq%2) + r, column 32d + 16(G%2) + 8h
            const int row = 32 * (cq >> 1) + 16 * tr_g + 8 * (cq & 1) + ((lane & 15) >> 1);
            const int off = lds_off<128>(row, 2 * d + (tr_G & 1)) + 8 * (lane & 1);
            const v2i r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(FMHA_LDS(v2i, vs + off));
            av[2 * cq] = r[0];
            av[2 * cq + 1] = r[1];
          }
          if (C::VS) {
            const v16f part = mfma_f8(av, pb, v16f{});
#pragma unroll
            for (int r = 0; r < 16; ++r) o[d][r] = __builtin_fmaf(part[r], svv, o[d][r]);
          } else {
            o[d] = mfma_f8(av, pb, o[d]);
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
            const uint32_t lo = f32_to_bf16_bits(p[8 * kk + 2 * j]);
            const uint32_t hi = f32_to_bf16_bits(p[8 * kk + 2 * j + 1]);
            w[j] = lo | (hi << 16);
            dsum += bf16_bits_to_f32(lo) + bf16_bits_to_f32(hi);
          }
          pbf[kk] = __builtin_bit_cast(v8bf, make_uint4(w[0], w[1], w[2], w[3]));
        }
        den += dsum;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            uint32_t w[4];
#pragma unroll
            for (int cq = 0; cq < 2; ++cq) {
              // source row: key 32(kk/2) + 16 g + 8(kk%2) + 4 cq + r, halfword
              // column 32d + 16(G%2) + 4h'
              const int row = 32 * (kk >> 1) + 16 * tr_g + 8 * (kk & 1) + 4 * cq + ((lane & 15) >> 2);
              const int hp = lane & 3;
              const int off = lds_off<256>(row, 4 * d + 2 * (tr_G & 1) + (hp >> 1)) + 8 * (hp & 1);
              const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(FMHA_LDS(v4s, vs + off));
              w[2 * cq] = (uint32_t)(uint16_t)r[0] | ((uint32_t)(uint16_t)r[1] << 16);
              w[2 * cq + 1] = (uint32_t)(uint16_t)r[2] | ((uint32_t)(uint16_t)r[3] << 16);
            }
            o[d] = mfma_bf16(__builtin_bit_cast(v8bf, make_uint4(w[0], w[1], w[2], w[3])), pbf[kk], o[d]);
          }
        }
      }
    }
    if (tn < n_sub) store_tile(stage ^ 1);
    __syncthreads();
    stage ^= 1;
    t = tn;
  }

  // ---- epilogue: O = num / den in bf16; rows without a valid key give 0
  if (!wave_live) return;
  const float dt = den + __shfl_xor(den, 32, 64);
  const float inv = dt > 0.0f ? 1.0f / dt : 0.0f;
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
}

template <class C>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  const int qtile = 32 * C::NW;
  dim3 grid((unsigned)((a.Sq + qtile - 1) / qtile), (unsigned)a.Hq, (unsigned)a.B);
  const size_t lds = 2 * (size_t)C::STAGE;
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
  if (k.paged) return launch<Cfg<QF, KF, VF, QS, KS, VS, false, true, 4>>(a, s);
  return launch<Cfg<QF, KF, VF, QS, KS, VS, false, false, 4>>(a, s);
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
