// Internal interface between the C-ABI layer (api.cpp) and the kernels.
// All strides here are in BYTES; every pointer is a device pointer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fmha {

enum Fmt : int { FMT_BF16 = 0, FMT_E4M3 = 1, FMT_INT8 = 2 };

struct QuantArgs {
  const uint8_t* x;
  int64_t x_sb, x_ss, x_sh;
  uint8_t* codes;
  int64_t c_sb, c_ss, c_sh;
  float* scales;
  int B, S, H, nblk;
  int D;        // 128 or 192
  int out_fmt;  // FMT_INT8 or FMT_E4M3
};

hipError_t launch_quantize_blocks(const QuantArgs& a, hipStream_t stream);

// Up to kMaxQuantJobs quantisations of one head dim in a single launch.
constexpr int kMaxQuantJobs = 8;
struct QuantBatch {
  QuantArgs job[kMaxQuantJobs];
  int64_t first[kMaxQuantJobs + 1];  // first grid block (wave) of each job; first[n] = total
  int n;
};
hipError_t launch_quantize_blocks_batch(const QuantArgs* jobs, int n, hipStream_t stream);

struct Nvfp4Args {
  const uint8_t* x; int64_t x_rs;   // bf16 [M, K], row stride in bytes
  uint8_t* codes; int64_t c_rs;     // [M, K/2], two E2M1 codes per byte
  uint8_t* sf; int64_t sf_rs;       // [M, K/16] E4M3 block scales
  float* ts;                        // [M] token scales
  int M, K;                         // K a multiple of 16
};

hipError_t launch_quantize_nvfp4(const Nvfp4Args& a, hipStream_t stream);

struct FwdArgs {
  const uint8_t* q; int64_t q_sb, q_ss, q_sh;
  const uint8_t* k; int64_t k_sb, k_ss, k_sh;   // paged: sb = page stride, ss = slot stride
  const uint8_t* v; int64_t v_sb, v_ss, v_sh;
  uint8_t* o; int64_t o_sb, o_ss, o_sh;
  const float* sfs_q;   // [B, Hq, nblk_q] or null
  const float* sfs_k;   // [B, Hkv, nblk_kv] or null
  const float* sfs_v;   // [B, Hkv, nblk_kv] or null
  int B, Sq, Skv, Hq, Hkv, group;
  int nblk_q, nblk_kv;
  float scale_log2;     // softmax_scale * log2(e)
  float tau;
  int causal;
  const uint8_t* mask;  // null = dense
  int64_t m_sb, m_sh, m_sqb;
  int mask_kv_sub;      // 64-key sub-tiles per mask key block
  int mask_kv_shift;    // log2(mask_kv_sub) when it is a power of two, else -1
  const int32_t* page_table;  // null = contiguous
  int64_t pt_sb;
  int page_size, num_pages;
  int pool32;           // paged K/V pools span < 4 GiB from their (head-offset) base
  const float* sfs_p;   // [Hq] or null
  int clamp_p;          // P / sp may reach the E4M3 overflow range
  int pack_rows;        // set by the launcher: 0, or R: a workgroup takes R queries of NW * 32 / R heads sharing a KV head
  int kv_whole_rsrc;    // contiguous K/V of one (batch, head) span < 2^31 bytes: one buffer resource each
  int o_fp8;            // o is E4M3: encode(O / sfs_o[h])
  const float* sfs_o;   // [Hq] or null (= 1)
  int tiles;            // set by the launcher: logical workgroup tiles of the launch
};

struct FwdKey {
  int D;                // head dim: 128, or 192 for some keys
  int qf, kf, vf;
  bool q_scaled, k_scaled, v_scaled;
  bool masked, paged;
};

// Returns hipErrorInvalidValue (without launching) when no kernel instance
// exists for the key; the caller validates that beforehand.
bool fwd_supported(const FwdKey& key);
hipError_t launch_fwd(const FwdKey& key, const FwdArgs& a, hipStream_t stream);

}  // namespace fmha
