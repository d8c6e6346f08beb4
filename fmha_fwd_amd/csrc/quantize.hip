// Per-(batch, head, 64-token block) quantisation to int8 or E4M3 with one
// fp32 scale per block (#2711 page "FlashInfer의 DiT 최적화: SageAttention과
// Int8/FP8 혼합 정밀도 커널 도입 분석", 코드 분석 2: block scale factors).
//
// HBM-bound: 2 bytes read and 1 byte written per element.  One wavefront owns
// one 64 x D block and keeps it in registers between the amax pass and the
// encode pass, so the input is read from HBM exactly once (the input-caching
// lesson of the #3237 page "FlashInfer의 Per-token NVFP4 Quantization 커널
// 최적화 분석", 코드 분석 2).  Lanes read 16-byte chunks (8 channels): for
// D = 128 sixteen lanes cover one 256-byte token row and a wave instruction
// covers four rows; for D = 192 the block's 64 x 24 chunks are dealt to the
// lanes in order (24 per lane).
#include "device_common.h"
#include "fmha_internal.h"

namespace fmha {
namespace {

constexpr int kWaves = 4;

// Eight bf16 values (one 16-byte chunk) -> eight codes (8 bytes).
template <int OUT>
__device__ __forceinline__ uint2 encode8(const uint4& v, float inv) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float y[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    y[2 * j] = __uint_as_float(w[j] << 16) * inv;
    y[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u) * inv;
  }
  if (OUT == FMT_E4M3) {
    int p0 = pack_e4m3<false>(y[0], y[1], 0);
    p0 = pack_e4m3<true>(y[2], y[3], p0);
    int p1 = pack_e4m3<false>(y[4], y[5], 0);
    p1 = pack_e4m3<true>(y[6], y[7], p1);
    return make_uint2((uint32_t)p0, (uint32_t)p1);
  }
  uint32_t p[2] = {0, 0};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    int c = (int)__builtin_rintf(y[j]);
    c = c > 127 ? 127 : (c < -127 ? -127 : c);
    p[j >> 2] |= ((uint32_t)c & 0xFFu) << (8 * (j & 3));
  }
  return make_uint2(p[0], p[1]);
}

// 64 x 192 blocks: chunk c = lane + 64 i of the block is token c / 24,
// channels 8 (c % 24) .. +8.
template <int OUT>
__device__ __forceinline__ void quantize_block_d192(const QuantArgs& a, const int64_t unit, const int lane) {
  constexpr int CPR = 24, PER_LANE = CPR;  // 64 rows x 24 chunks over 64 lanes
  const int blk = (int)(unit % a.nblk);
  const int64_t bh = unit / a.nblk;
  const int h = (int)(bh % a.H);
  const int b = (int)(bh / a.H);
  const int tok0 = blk * 64;
  const uint8_t* xb = a.x + (int64_t)b * a.x_sb + (int64_t)h * a.x_sh;
  uint4 v[PER_LANE];
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) {
    const int c = lane + 64 * i;
    const int tok = tok0 + c / CPR;
    v[i] = tok < a.S ? *(const uint4*)(xb + (int64_t)tok * a.x_ss + 16 * (c % CPR)) : make_uint4(0, 0, 0, 0);
  }
  // |x| of a bf16 orders like its magnitude bits: exact amax with 16-bit max.
  v2us m2 = {0, 0};
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) {
    const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t mag = w[j] & 0x7FFF7FFFu;
      const v2us m = {(unsigned short)(mag & 0xFFFF), (unsigned short)(mag >> 16)};
      m2 = __builtin_elementwise_max(m2, m);
    }
  }
  uint32_t amax_bits = m2.x > m2.y ? m2.x : m2.y;
  amax_bits = wave_max_u32(amax_bits);
  const float amax = bf16_bits_to_f32(amax_bits);
  const float qmax = OUT == FMT_INT8 ? 127.0f : 448.0f;
  const bool live = amax_bits >= 0x0080u;  // amax >= 2^-126
  const float scale = live ? amax / qmax : 1.0f;   // correctly rounded division
  // A dead block (amax below 2^-126) takes scale 1 and all-zero codes: code
  // 0x00 also for negative zeros and negative subnormals, whose product with
  // any multiplier would keep the sign (E4M3 0x80).
  const float inv = live ? qmax / amax : 0.0f;
  uint8_t* cb = a.codes + (int64_t)b * a.c_sb + (int64_t)h * a.c_sh;
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) {
    const int c = lane + 64 * i;
    const int tok = tok0 + c / CPR;
    const uint2 out = live ? encode8<OUT>(v[i], inv) : make_uint2(0, 0);
    if (tok < a.S) *(uint2*)(cb + (int64_t)tok * a.c_ss + 8 * (c % CPR)) = out;
  }
  if (lane == 0) a.scales[bh * a.nblk + blk] = scale;
}

template <int OUT>
__global__ __launch_bounds__(kWaves * 64) void quantize_blocks_kernel_d192(QuantArgs a) {
  const int64_t unit = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (unit >= (int64_t)a.B * a.H * a.nblk) return;  // uniform per wave
  quantize_block_d192<OUT>(a, unit, threadIdx.x & 63);
}

template <int OUT>  // FMT_INT8 or FMT_E4M3
__device__ __forceinline__ void quantize_block_d128(const QuantArgs& a, const int64_t unit, const int lane) {
  const int blk = (int)(unit % a.nblk);
  const int64_t bh = unit / a.nblk;
  const int h = (int)(bh % a.H);
  const int b = (int)(bh / a.H);

  const int row0 = lane >> 4;          // rows row0 + 4*i, i = 0..15
  const int col_bytes = (lane & 15) * 16;  // 8 bf16 channels
  const int tok0 = blk * 64;
  const uint8_t* xb = a.x + (int64_t)b * a.x_sb + (int64_t)h * a.x_sh + col_bytes;

  uint4 v[16];
  v2us m2 = {0, 0};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int tok = tok0 + row0 + 4 * i;
    if (tok < a.S) {
      v[i] = *(const uint4*)(xb + (int64_t)tok * a.x_ss);
    } else {
      v[i] = make_uint4(0, 0, 0, 0);
    }
  }
  // |x| of a bf16 orders like its magnitude bits: exact amax with 16-bit max.
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t mag = w[j] & 0x7FFF7FFFu;
      v2us m = {(unsigned short)(mag & 0xFFFF), (unsigned short)(mag >> 16)};
      m2 = __builtin_elementwise_max(m2, m);
    }
  }
  uint32_t amax_bits = m2.x > m2.y ? m2.x : m2.y;
  amax_bits = wave_max_u32(amax_bits);
  const float amax = bf16_bits_to_f32(amax_bits);
  const float qmax = OUT == FMT_INT8 ? 127.0f : 448.0f;
  const bool live = amax_bits >= 0x0080u;  // amax >= 2^-126
  const float scale = live ? amax / qmax : 1.0f;   // correctly rounded division
  const float inv = live ? qmax / amax : 0.0f;  // dead blocks: all-zero codes (as above)

  uint8_t* cb = a.codes + (int64_t)b * a.c_sb + (int64_t)h * a.c_sh + (lane & 15) * 8;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int tok = tok0 + row0 + 4 * i;
    const uint2 out = live ? encode8<OUT>(v[i], inv) : make_uint2(0, 0);
    if (tok < a.S) *(uint2*)(cb + (int64_t)tok * a.c_ss) = out;
  }
  if (lane == 0) a.scales[bh * a.nblk + blk] = scale;
}

template <int OUT>
__global__ __launch_bounds__(kWaves * 64) void quantize_blocks_kernel(QuantArgs a) {
  const int64_t unit = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (unit >= (int64_t)a.B * a.H * a.nblk) return;  // uniform per wave
  quantize_block_d128<OUT>(a, unit, threadIdx.x & 63);
}

// Several tensors of one head dim in one launch: wave w of the grid takes
// block w - first[j] of job j, first[j] <= w < first[j + 1] (the blocks of
// each job in the order of a single launch).
template <int D>
__global__ __launch_bounds__(kWaves * 64) void quantize_blocks_batch_kernel(QuantBatch jb) {
  const int64_t unit = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (unit >= jb.first[jb.n]) return;  // uniform per wave
  int j = 0;
  while (unit >= jb.first[j + 1]) ++j;
  const QuantArgs& a = jb.job[j];
  const int lane = threadIdx.x & 63;
  if constexpr (D == 192) {
    if (a.out_fmt == FMT_INT8) quantize_block_d192<FMT_INT8>(a, unit - jb.first[j], lane);
    else quantize_block_d192<FMT_E4M3>(a, unit - jb.first[j], lane);
  } else {
    if (a.out_fmt == FMT_INT8) quantize_block_d128<FMT_INT8>(a, unit - jb.first[j], lane);
    else quantize_block_d128<FMT_E4M3>(a, unit - jb.first[j], lane);
  }
}

}  // namespace

hipError_t launch_quantize_blocks_batch(const QuantArgs* jobs, int n, hipStream_t stream) {
  if (n < 1 || n > kMaxQuantJobs) return hipErrorInvalidValue;
  QuantBatch jb{};
  jb.n = n;
  jb.first[0] = 0;
  for (int j = 0; j < n; ++j) {
    if (jobs[j].D != jobs[0].D) return hipErrorInvalidValue;
    jb.job[j] = jobs[j];
    jb.first[j + 1] = jb.first[j] + (int64_t)jobs[j].B * jobs[j].H * jobs[j].nblk;
  }
  const int64_t units = jb.first[n];
  if (units == 0) return hipSuccess;
  const int64_t grid = (units + kWaves - 1) / kWaves;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (jobs[0].D == 192)
    hipLaunchKernelGGL(quantize_blocks_batch_kernel<192>, dim3((unsigned)grid), dim3(kWaves * 64), 0, stream, jb);
  else
    hipLaunchKernelGGL(quantize_blocks_batch_kernel<128>, dim3((unsigned)grid), dim3(kWaves * 64), 0, stream, jb);
  return hipGetLastError();
}

hipError_t launch_quantize_blocks(const QuantArgs& a, hipStream_t stream) {
  const int64_t units = (int64_t)a.B * a.H * a.nblk;
  if (units == 0) return hipSuccess;
  const int64_t grid = (units + kWaves - 1) / kWaves;
  if (a.D == 192) {
    if (a.out_fmt == FMT_INT8)
      hipLaunchKernelGGL(quantize_blocks_kernel_d192<FMT_INT8>, dim3((unsigned)grid), dim3(kWaves * 64), 0, stream, a);
    else
      hipLaunchKernelGGL(quantize_blocks_kernel_d192<FMT_E4M3>, dim3((unsigned)grid), dim3(kWaves * 64), 0, stream, a);
    return hipGetLastError();
  }
  if (a.out_fmt == FMT_INT8)
    hipLaunchKernelGGL(quantize_blocks_kernel<FMT_INT8>, dim3((unsigned)grid), dim3(kWaves * 64), 0, stream, a);
  else
    hipLaunchKernelGGL(quantize_blocks_kernel<FMT_E4M3>, dim3((unsigned)grid), dim3(kWaves * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace fmha
