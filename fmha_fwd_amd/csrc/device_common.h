// Device-side helpers shared by the gfx950 kernels: vector types, MFMA
// wrappers, number-format conversions and wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fmha {

typedef __attribute__((ext_vector_type(2))) int v2i;
typedef __attribute__((ext_vector_type(4))) int v4i;
typedef __attribute__((ext_vector_type(8))) int v8i;
typedef __attribute__((ext_vector_type(16))) int v16i;
typedef __attribute__((ext_vector_type(2))) float v2f;
typedef __attribute__((ext_vector_type(4))) float v4f;
typedef __attribute__((ext_vector_type(16))) float v16f;
typedef __attribute__((ext_vector_type(8))) __bf16 v8bf;
typedef __attribute__((ext_vector_type(8))) _Float16 v8h;
typedef __attribute__((ext_vector_type(2))) _Float16 v2h;
typedef __attribute__((ext_vector_type(4))) short v4s;
typedef __attribute__((ext_vector_type(2))) unsigned short v2us;

#define FMHA_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))
typedef __attribute__((address_space(3))) uint8_t lds_u8;  // byte in LDS

// ---------------------------------------------------------------- MFMA
// 32x32 output tiles.  Operand layout (checked on gfx950): lane l supplies row
// (A) / column (B) l % 32 and the contraction slots of lane group l / 32;
// result register r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l % 32.
__device__ __forceinline__ v16f mfma_bf16(v8bf a, v8bf b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v16f mfma_f16(v8h a, v8h b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v16i mfma_i8(v4i a, v4i b, v16i c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}
// E4M3 x E4M3 with unit block scales (E8M0 exponent 127 = 2^0).
__device__ __forceinline__ v16f mfma_f8(v8i a, v8i b, v16f c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// 16x16x128 E4M3 product: lane l supplies row (A) / column (B) l % 16 and
// contraction slots 32*(l/16) .. +32 (byte i of the 8 registers = slot +i);
// result register r of lane l is row 4*(l/16) + r, column l % 16.
__device__ __forceinline__ v4f mfma_f8_16(v8i a, v8i b, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// ---------------------------------------------------------------- formats
// Two floats -> two E4M3 codes in byte pair `hi` of `old` (round to nearest
// even; the hardware returns NaN instead of saturating at |x| >= 464, so
// callers clamp first where that range can be reached).
template <bool HI>
__device__ __forceinline__ int pack_e4m3(float a, float b, int old) {
  return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
}
template <bool HI>
__device__ __forceinline__ v2f unpack_e4m3(int packed) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(packed, HI);
}
// Eight E4M3 codes (byte i of w0:w1 = element i) -> eight bf16, exactly
// (every E4M3 value, subnormals included, is a bf16 value).
__device__ __forceinline__ v8bf e4m3x8_to_bf16(uint32_t w0, uint32_t w1) {
  typedef __attribute__((ext_vector_type(2))) __bf16 v2bf;
  const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  return v8bf{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}
// Eight E4M3 codes (byte i of w0:w1 = element i) -> eight fp16, exactly
// (E4M3's exponents -9 .. 8 and three fraction bits lie inside fp16's).
__device__ __forceinline__ v8h e4m3x8_to_f16(uint32_t w0, uint32_t w1) {
  const v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
  const v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
  const v2h c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
  const v2h d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
  return v8h{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}
// Eight int8 codes (byte i of w0:w1 = element i) -> eight fp16, exactly.
// With its sign bit flipped a code c reads as the unsigned byte c + 128;
// placed under the fp16 pattern 0x64 (1024, unit spacing up to 2048) it is
// the half 1152 + c, and one packed subtraction of 1152 leaves c.
__device__ __forceinline__ v8h int8x8_to_f16(uint32_t w0, uint32_t w1) {
  const uint32_t u0 = w0 ^ 0x80808080u, u1 = w1 ^ 0x80808080u;
  // v_perm byte selectors: 0-3 pick bytes of the second source, 4 byte 0 of
  // the first (0x64)
  const uint32_t h[4] = {__builtin_amdgcn_perm(0x64646464u, u0, 0x04010400u),
                         __builtin_amdgcn_perm(0x64646464u, u0, 0x04030402u),
                         __builtin_amdgcn_perm(0x64646464u, u1, 0x04010400u),
                         __builtin_amdgcn_perm(0x64646464u, u1, 0x04030402u)};
  const v2h off = {(_Float16)1152.0f, (_Float16)1152.0f};
  v8h r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const v2h x = __builtin_bit_cast(v2h, h[i]) - off;
    r[2 * i] = x[0];
    r[2 * i + 1] = x[1];
  }
  return r;
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}
// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    uint32_t w = (uint32_t)__shfl_xor((int)v, o, 64);
    v = v > w ? v : w;
  }
  return v;
}

}  // namespace fmha
