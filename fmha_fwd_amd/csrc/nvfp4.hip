// Per-token NVFP4 quantisation of a bf16 activation matrix [M tokens, K]:
// E2M1 codes (two per byte), one E4M3 scale per 16 consecutive elements of a
// row (linear layout) and one fp32 scale per token (#3237 page "FlashInfer의
// Per-token NVFP4 Quantization 커널 최적화 분석", 코드 분석 1-2).
//
// Per row: amax = max |x|; ts = amax / 2688; per 16-element block sf =
// E4M3(min(bmax * (448 / amax), 448)), bs = dec(sf) * ts, es = 1 / bs
// (0 when bs is 0, at most FLT_MAX), code = E2M1(x * es).  Rows with amax
// below 2^-116 take ts = 1 and zero block scales.  fp32 throughout, divisions
// correctly rounded, nearest-even everywhere.
//
// HBM-bound (2 bytes read, 0.5 + 1/16 bytes written per element).  One
// wavefront owns one row; lane l owns blocks l, l + 64, ...  Rows up to 16384
// elements stay in registers between the amax pass and the encode pass, so
// the input is read once (the page's input caching, here in VGPRs instead of
// shared memory); longer rows are read twice, the second time mostly from
// the caches.  The E2M1 encoding is the gfx950 converter
// v_cvt_scalef32_pk_fp4_f32 with a unit scale (nearest-even, saturating at
// +-6, sign of zero kept).
#include <cfloat>

#include "device_common.h"
#include "fmha_internal.h"

namespace fmha {
namespace {

constexpr int kRowsPerGroup = 4;  // wavefronts (rows) per workgroup

struct RowScales {
  float ts, g6;
};

__device__ __forceinline__ uint32_t bf16x16_max_bits(const uint4& a, const uint4& b) {
  // |x| of a bf16 orders like its magnitude bits
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  v2us m2 = {0, 0};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t mag = w[j] & 0x7FFF7FFFu;
    const v2us m = {(unsigned short)(mag & 0xFFFF), (unsigned short)(mag >> 16)};
    m2 = __builtin_elementwise_max(m2, m);
  }
  return m2.x > m2.y ? m2.x : m2.y;
}

__device__ __forceinline__ RowScales row_scales(uint32_t amax_bits) {
  const float amax = bf16_bits_to_f32(amax_bits);
  const bool live = amax_bits >= 0x0580u;  // amax >= 2^-116
  return {live ? amax / 2688.0f : 1.0f, live ? 448.0f / amax : 0.0f};
}

// Block scale byte and the 16 codes (8 bytes) of one block.
__device__ __forceinline__ void encode_block(const uint4& a, const uint4& b, uint32_t bmax_bits, RowScales rs,
                                             uint8_t& sf, uint2& codes) {
  const float sfv = fminf(bf16_bits_to_f32(bmax_bits) * rs.g6, 448.0f);
  const int sfc = pack_e4m3<false>(sfv, 0.0f, 0) & 0xFF;
  const float bs = unpack_e4m3<false>(sfc)[0] * rs.ts;
  const float es = bs > 0.0f ? fminf(1.0f / bs, FLT_MAX) : 0.0f;
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t out[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float lo = bf16_bits_to_f32(w[j] & 0xFFFFu) * es;  // element 2j
    const float hi = __uint_as_float(w[j] & 0xFFFF0000u) * es;
    // byte j % 4 of word j / 4: element 2j in the low nibble
    uint32_t& o = out[j >> 2];
    switch (j & 3) {
      case 0: o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, lo, hi, 1.0f, 0); break;
      case 1: o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, lo, hi, 1.0f, 1); break;
      case 2: o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, lo, hi, 1.0f, 2); break;
      default: o = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(o, lo, hi, 1.0f, 3); break;
    }
  }
  sf = (uint8_t)sfc;
  codes = make_uint2(out[0], out[1]);
}

// NB > 0: the row in registers, at most NB blocks per lane.  NB == 0: rows
// of any length, read twice in chunks of four blocks per lane.
template <int NB>
__global__ __launch_bounds__(kRowsPerGroup * 64) void quantize_nvfp4_kernel(Nvfp4Args a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerGroup + (threadIdx.x >> 6);
  if (row >= a.M) return;  // uniform per wave
  const int nb = a.K / 16;
  const uint8_t* xr = a.x + row * a.x_rs;
  uint8_t* cr = a.codes + row * a.c_rs;
  uint8_t* sr = a.sf + row * a.sf_rs;

  if constexpr (NB > 0) {
    uint4 v[NB][2];
    uint32_t bm[NB];
    uint32_t amax_bits = 0;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int j = lane + 64 * i;
      if (j < nb) {
        v[i][0] = *(const uint4*)(xr + 32 * j);
        v[i][1] = *(const uint4*)(xr + 32 * j + 16);
      } else {
        v[i][0] = v[i][1] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      bm[i] = bf16x16_max_bits(v[i][0], v[i][1]);
      amax_bits = bm[i] > amax_bits ? bm[i] : amax_bits;
    }
    const RowScales rs = row_scales(wave_max_u32(amax_bits));
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int j = lane + 64 * i;
      if (j < nb) {
        uint8_t sf;
        uint2 c;
        encode_block(v[i][0], v[i][1], bm[i], rs, sf, c);
        *(uint2*)(cr + 8 * j) = c;
        sr[j] = sf;
      }
    }
    if (lane == 0) a.ts[row] = rs.ts;
  } else {
    constexpr int CH = 4;
    uint32_t amax_bits = 0;
    for (int j0 = 0; j0 < nb; j0 += 64 * CH) {
      uint4 v[CH][2];
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const int j = j0 + lane + 64 * i;
        if (j < nb) {
          v[i][0] = *(const uint4*)(xr + 32 * j);
          v[i][1] = *(const uint4*)(xr + 32 * j + 16);
        } else {
          v[i][0] = v[i][1] = make_uint4(0, 0, 0, 0);
        }
      }
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const uint32_t m = bf16x16_max_bits(v[i][0], v[i][1]);
        amax_bits = m > amax_bits ? m : amax_bits;
      }
    }
    const RowScales rs = row_scales(wave_max_u32(amax_bits));
    for (int j0 = 0; j0 < nb; j0 += 64 * CH) {
      uint4 v[CH][2];
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const int j = j0 + lane + 64 * i;
        if (j < nb) {
          v[i][0] = *(const uint4*)(xr + 32 * j);
          v[i][1] = *(const uint4*)(xr + 32 * j + 16);
        } else {
          v[i][0] = v[i][1] = make_uint4(0, 0, 0, 0);
        }
      }
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const int j = j0 + lane + 64 * i;
        if (j < nb) {
          uint8_t sf;
          uint2 c;
          encode_block(v[i][0], v[i][1], bf16x16_max_bits(v[i][0], v[i][1]), rs, sf, c);
          *(uint2*)(cr + 8 * j) = c;
          sr[j] = sf;
        }
      }
    }
    if (lane == 0) a.ts[row] = rs.ts;
  }
}

template <int NB>
hipError_t launch(const Nvfp4Args& a, hipStream_t stream) {
  const int64_t grid = (a.M + kRowsPerGroup - 1) / kRowsPerGroup;
  hipLaunchKernelGGL(quantize_nvfp4_kernel<NB>, dim3((unsigned)grid), dim3(kRowsPerGroup * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_nvfp4(const Nvfp4Args& a, hipStream_t stream) {
  if (a.M == 0) return hipSuccess;
  const int per_lane = (a.K / 16 + 63) / 64;  // blocks per lane
  if (per_lane <= 2) return launch<2>(a, stream);
  if (per_lane <= 4) return launch<4>(a, stream);
  if (per_lane <= 8) return launch<8>(a, stream);
  if (per_lane <= 16) return launch<16>(a, stream);
  return launch<0>(a, stream);
}

}  // namespace fmha
