// C ABI of the attention library: argument validation (before any HIP call),
// selection of the kernel instance from the per-tensor formats and scale-block
// sizes (the dispatch key of the #2711 page "FlashInfer의 DiT 최적화:
// SageAttention과 Int8/FP8 혼합 정밀도 커널 도입 분석", 코드 분석 1: Q, K, V, O
// dtypes plus the number of elements per Q/K/P/V scale factor), and launch on
// the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstddef>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/fmha.h"
#include "fmha_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return FMHA_OK;
}

int elem_size(int32_t dt) { return dt == FMHA_DT_BF16 ? 2 : 1; }

bool known_dtype(int32_t dt) { return dt == FMHA_DT_BF16 || dt == FMHA_DT_E4M3 || dt == FMHA_DT_INT8; }

int to_fmt(int32_t dt) {
  return dt == FMHA_DT_BF16 ? fmha::FMT_BF16 : dt == FMHA_DT_E4M3 ? fmha::FMT_E4M3 : fmha::FMT_INT8;
}

// Checks pointer and strides of a [*, *, *, D] tensor with contiguous D.
int check_tensor(const char* name, const fmha_tensor& t, bool needed) {
  if (!known_dtype(t.dtype)) return fail(FMHA_ERR_INVALID, "%s: unknown dtype %d", name, (int)t.dtype);
  if (!needed) return FMHA_OK;
  if (t.ptr == nullptr) return fail(FMHA_ERR_INVALID, "%s: null pointer", name);
  if (reinterpret_cast<uintptr_t>(t.ptr) % 16 != 0) return fail(FMHA_ERR_INVALID, "%s: pointer not 16-byte aligned", name);
  const int es = elem_size(t.dtype);
  const int64_t st[3] = {t.stride_b, t.stride_s, t.stride_h};
  const char* nm[3] = {"stride_b", "stride_s", "stride_h"};
  for (int i = 0; i < 3; ++i) {
    if (st[i] < 0) return fail(FMHA_ERR_INVALID, "%s: negative %s", name, nm[i]);
    if ((st[i] * es) % 16 != 0) return fail(FMHA_ERR_INVALID, "%s: %s * element size is not a multiple of 16 bytes", name, nm[i]);
  }
  return FMHA_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(FMHA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" {

uint32_t fmha_abi_version(void) { return 0x000400u; }

const char* fmha_last_error(void) { return g_last_error.c_str(); }

namespace {

// Validates one block quantisation (messages prefixed with `who`) and fills
// its kernel arguments; *empty is set for a no-op (B, S or H equal to 0).
int quant_args(const char* who, const fmha_tensor* x, const fmha_tensor* codes, float* scales, int32_t B,
               int32_t S, int32_t H, int32_t D, int32_t block_tokens, fmha::QuantArgs* a, bool* empty) {
  if (!x || !codes) return fail(FMHA_ERR_INVALID, "%s: null tensor descriptor", who);
  if (B < 0 || S < 0 || H < 0) return fail(FMHA_ERR_INVALID, "%s: negative size (B=%d S=%d H=%d)", who, B, S, H);
  if (D != 128 && D != 192) return fail(FMHA_ERR_UNSUPPORTED, "%s: D=%d (128 or 192 are supported)", who, D);
  if (block_tokens != 64)
    return fail(FMHA_ERR_UNSUPPORTED, "%s: block_tokens=%d (only 64 is supported)", who, block_tokens);
  if (x->dtype != FMHA_DT_BF16) return fail(FMHA_ERR_INVALID, "%s: x must be bf16", who);
  if (codes->dtype != FMHA_DT_INT8 && codes->dtype != FMHA_DT_E4M3)
    return fail(FMHA_ERR_INVALID, "%s: codes must be int8 or e4m3", who);
  *empty = (int64_t)B * S * H == 0;
  char name[64];
  int r;
  snprintf(name, sizeof name, "%s x", who);
  if ((r = check_tensor(name, *x, !*empty)) != FMHA_OK) return r;
  snprintf(name, sizeof name, "%s codes", who);
  if ((r = check_tensor(name, *codes, !*empty)) != FMHA_OK) return r;
  if (*empty) return FMHA_OK;
  if (!scales) return fail(FMHA_ERR_INVALID, "%s: null scales", who);
  if (reinterpret_cast<uintptr_t>(scales) % 4 != 0) return fail(FMHA_ERR_INVALID, "%s: scales not 4-byte aligned", who);
  *a = fmha::QuantArgs{};
  a->x = static_cast<const uint8_t*>(x->ptr);
  a->x_sb = x->stride_b * 2;
  a->x_ss = x->stride_s * 2;
  a->x_sh = x->stride_h * 2;
  a->codes = static_cast<uint8_t*>(codes->ptr);
  a->c_sb = codes->stride_b;
  a->c_ss = codes->stride_s;
  a->c_sh = codes->stride_h;
  a->scales = scales;
  a->B = B;
  a->S = S;
  a->H = H;
  a->nblk = (S + 63) / 64;
  a->D = D;
  a->out_fmt = codes->dtype == FMHA_DT_INT8 ? fmha::FMT_INT8 : fmha::FMT_E4M3;
  return FMHA_OK;
}

}  // namespace

int fmha_quantize_blocks(const fmha_tensor* x, const fmha_tensor* codes, float* scales, int32_t B, int32_t S,
                         int32_t H, int32_t D, int32_t block_tokens, fmha_stream_t stream) {
  fmha::QuantArgs a;
  bool empty = false;
  const int r = quant_args("quantize", x, codes, scales, B, S, H, D, block_tokens, &a, &empty);
  if (r != FMHA_OK) return r;
  if (empty) return ok();
  return hip_status(fmha::launch_quantize_blocks(a, static_cast<hipStream_t>(stream)), "quantize launch");
}

int fmha_quantize_blocks_batch(const fmha_quantize_job* jobs, int32_t n_jobs, fmha_stream_t stream) {
  if (n_jobs < 0 || n_jobs > FMHA_MAX_QUANTIZE_JOBS)
    return fail(FMHA_ERR_INVALID, "quantize batch: n_jobs=%d (0 to %d)", n_jobs, FMHA_MAX_QUANTIZE_JOBS);
  if (n_jobs == 0) return ok();
  if (!jobs) return fail(FMHA_ERR_INVALID, "quantize batch: null jobs");
  fmha::QuantArgs a[FMHA_MAX_QUANTIZE_JOBS];
  int n = 0;
  for (int j = 0; j < n_jobs; ++j) {
    const fmha_quantize_job& q = jobs[j];
    char who[32];
    snprintf(who, sizeof who, "quantize job %d", j);
    bool empty = false;
    const int r = quant_args(who, &q.x, &q.codes, q.scales, q.B, q.S, q.H, q.D, q.block_tokens, &a[n], &empty);
    if (r != FMHA_OK) return r;
    if (q.D != jobs[0].D)
      return fail(FMHA_ERR_UNSUPPORTED, "quantize batch: job %d has D=%d, job 0 D=%d (one head dim per batch)", j,
                  q.D, jobs[0].D);
    if (!empty) ++n;
  }
  if (n == 0) return ok();
  return hip_status(fmha::launch_quantize_blocks_batch(a, n, static_cast<hipStream_t>(stream)), "quantize batch launch");
}

int fmha_quantize_nvfp4(const void* x, int64_t x_row_stride, int32_t M, int32_t K, uint8_t* codes,
                        int64_t codes_row_stride, uint8_t* block_scales, int64_t scales_row_stride,
                        float* token_scales, fmha_stream_t stream) {
  if (M < 0) return fail(FMHA_ERR_INVALID, "nvfp4: negative M=%d", M);
  if (K <= 0 || K % 16 != 0) return fail(FMHA_ERR_INVALID, "nvfp4: K=%d is not a positive multiple of 16", K);
  if (K > (1 << 28)) return fail(FMHA_ERR_UNSUPPORTED, "nvfp4: K=%d above 2^28 (32-bit in-row offsets)", K);
  if (M == 0) return ok();
  if (!x || !codes || !block_scales || !token_scales) return fail(FMHA_ERR_INVALID, "nvfp4: null pointer");
  if (reinterpret_cast<uintptr_t>(x) % 16 != 0) return fail(FMHA_ERR_INVALID, "nvfp4: x not 16-byte aligned");
  if (x_row_stride < K || x_row_stride % 8 != 0)
    return fail(FMHA_ERR_INVALID, "nvfp4: x_row_stride=%lld must be >= K and a multiple of 8", (long long)x_row_stride);
  if (reinterpret_cast<uintptr_t>(codes) % 8 != 0) return fail(FMHA_ERR_INVALID, "nvfp4: codes not 8-byte aligned");
  if (codes_row_stride < K / 2 || codes_row_stride % 8 != 0)
    return fail(FMHA_ERR_INVALID, "nvfp4: codes_row_stride=%lld must be >= K/2 and a multiple of 8",
                (long long)codes_row_stride);
  if (scales_row_stride < K / 16)
    return fail(FMHA_ERR_INVALID, "nvfp4: scales_row_stride=%lld must be >= K/16", (long long)scales_row_stride);
  if (reinterpret_cast<uintptr_t>(token_scales) % 4 != 0)
    return fail(FMHA_ERR_INVALID, "nvfp4: token_scales not 4-byte aligned");
  fmha::Nvfp4Args a{};
  a.x = static_cast<const uint8_t*>(x);
  a.x_rs = x_row_stride * 2;
  a.codes = codes;
  a.c_rs = codes_row_stride;
  a.sf = block_scales;
  a.sf_rs = scales_row_stride;
  a.ts = token_scales;
  a.M = M;
  a.K = K;
  return hip_status(fmha::launch_quantize_nvfp4(a, static_cast<hipStream_t>(stream)), "nvfp4 launch");
}

int fmha_fwd(const fmha_fwd_params* p, fmha_stream_t stream) {
  if (!p) return fail(FMHA_ERR_INVALID, "fwd: null params");
  // this layout, or the previous one (which ends before sfs_o)
  const size_t prev_size = offsetof(fmha_fwd_params, sfs_o);
  if (p->struct_size != sizeof(fmha_fwd_params) && p->struct_size != prev_size)
    return fail(FMHA_ERR_INVALID, "fwd: struct_size %u does not match this library (%zu or %zu)", p->struct_size,
                sizeof(fmha_fwd_params), prev_size);
  const float* sfs_o = p->struct_size == sizeof(fmha_fwd_params) ? p->sfs_o : nullptr;
  if (p->B < 0 || p->Sq < 0 || p->Skv < 0) return fail(FMHA_ERR_INVALID, "fwd: negative size");
  if (p->Hq < 1 || p->Hkv < 1) return fail(FMHA_ERR_INVALID, "fwd: Hq and Hkv must be >= 1");
  if (p->Hq % p->Hkv != 0) return fail(FMHA_ERR_INVALID, "fwd: Hq=%d is not a multiple of Hkv=%d", p->Hq, p->Hkv);
  if (p->D != 128 && p->D != 192) return fail(FMHA_ERR_UNSUPPORTED, "fwd: D=%d (128 or 192 are supported)", p->D);
  if (p->o.dtype != FMHA_DT_BF16 && p->o.dtype != FMHA_DT_E4M3)
    return fail(FMHA_ERR_UNSUPPORTED, "fwd: o must be bf16 or e4m3");
  if (sfs_o && p->o.dtype != FMHA_DT_E4M3) return fail(FMHA_ERR_INVALID, "fwd: sfs_o given for a bf16 o");
  if (sfs_o && reinterpret_cast<uintptr_t>(sfs_o) % 4) return fail(FMHA_ERR_INVALID, "fwd: sfs_o misaligned");
  const bool empty = (int64_t)p->B * p->Sq == 0;
  const bool paged = p->page_table != nullptr;
  const bool need_kv = !empty && p->Skv > 0;
  int r;
  if ((r = check_tensor("q", p->q, !empty)) != FMHA_OK) return r;
  if ((r = check_tensor("k", p->k, need_kv)) != FMHA_OK) return r;
  if ((r = check_tensor("v", p->v, need_kv)) != FMHA_OK) return r;
  if ((r = check_tensor("o", p->o, !empty)) != FMHA_OK) return r;
  // K/V token rows must not overlap: the copies bound a tile's bytes by
  // (tokens x token stride), so a token stride below one row (a broadcast
  // view with stride 0, say) would read zeros instead of the rows.
  if (need_kv && (p->k.stride_s < p->D || p->v.stride_s < p->D))
    return fail(FMHA_ERR_INVALID, "fwd: k/v stride_s (%lld, %lld elements) is below one token row (D=%d)",
                (long long)p->k.stride_s, (long long)p->v.stride_s, p->D);

  const int sb[3] = {p->sage_block_q, p->sage_block_k, p->sage_block_v};
  const void* sp[3] = {p->sfs_q, p->sfs_k, p->sfs_v};
  const char* sn[3] = {"q", "k", "v"};
  for (int i = 0; i < 3; ++i) {
    if (sb[i] != 0 && sb[i] != 64) return fail(FMHA_ERR_UNSUPPORTED, "fwd: sage_block_%s=%d (0 or 64)", sn[i], sb[i]);
    const bool has_blocks = i == 0 ? p->Sq > 0 : p->Skv > 0;  // an empty sequence has no scales to point at
    if (sb[i] == 64 && !sp[i] && has_blocks)
      return fail(FMHA_ERR_INVALID, "fwd: sage_block_%s=64 but sfs_%s is null", sn[i], sn[i]);
    if (sb[i] == 0 && sp[i]) return fail(FMHA_ERR_INVALID, "fwd: sfs_%s given but sage_block_%s=0", sn[i], sn[i]);
    if (sp[i] && reinterpret_cast<uintptr_t>(sp[i]) % 4) return fail(FMHA_ERR_INVALID, "fwd: sfs_%s misaligned", sn[i]);
  }
  if (!std::isfinite(p->softmax_scale)) return fail(FMHA_ERR_INVALID, "fwd: softmax_scale is not finite");
  if (!(p->lazy_rescale_log2 >= 0.0f && p->lazy_rescale_log2 <= 16.0f))
    return fail(FMHA_ERR_INVALID, "fwd: lazy_rescale_log2 must be in [0, 16]");
  if (p->causal != 0 && p->causal != 1) return fail(FMHA_ERR_INVALID, "fwd: causal must be 0 or 1");
  if (p->block_mask) {
    if (p->mask_block_q != 64) return fail(FMHA_ERR_UNSUPPORTED, "fwd: mask_block_q=%d (only 64)", p->mask_block_q);
    if (p->mask_block_kv <= 0 || p->mask_block_kv % 64)
      return fail(FMHA_ERR_UNSUPPORTED, "fwd: mask_block_kv=%d (a positive multiple of 64)", p->mask_block_kv);
    if (p->mask_stride_b < 0 || p->mask_stride_h < 0 || p->mask_stride_qb < 0)
      return fail(FMHA_ERR_INVALID, "fwd: negative mask stride");
  }
  if (paged) {
    const int ps = p->page_size;
    if (ps < 16 || ps > (1 << 20) || (ps & (ps - 1)))
      return fail(FMHA_ERR_UNSUPPORTED, "fwd: page_size=%d (a power of two, at least 16)", ps);
    if (p->num_pages < 1) return fail(FMHA_ERR_INVALID, "fwd: num_pages=%d", p->num_pages);
    if (p->page_table_stride_b < 0) return fail(FMHA_ERR_INVALID, "fwd: negative page_table_stride_b");
  }
  if (p->sfs_p && reinterpret_cast<uintptr_t>(p->sfs_p) % 4) return fail(FMHA_ERR_INVALID, "fwd: sfs_p misaligned");
  // one 64-token tile of K or V must span less than 2 GiB (32-bit in-tile offsets)
  if (p->k.stride_s * elem_size(p->k.dtype) >= (int64_t(1) << 25) ||
      p->v.stride_s * elem_size(p->v.dtype) >= (int64_t(1) << 25))
    return fail(FMHA_ERR_UNSUPPORTED, "fwd: K/V token stride of 32 MiB or more");

  fmha::FwdKey key{};
  key.D = p->D;
  key.qf = to_fmt(p->q.dtype);
  key.kf = to_fmt(p->k.dtype);
  key.vf = to_fmt(p->v.dtype);
  key.q_scaled = p->sage_block_q == 64;
  key.k_scaled = p->sage_block_k == 64;
  key.v_scaled = p->sage_block_v == 64;
  key.masked = p->block_mask != nullptr;
  key.paged = paged;
  if (!fmha::fwd_supported(key))
    return fail(FMHA_ERR_UNSUPPORTED,
                "fwd: no kernel for (q, k, v) = (%d, %d, %d) with scales (q %d, k %d, v %d); supported: "
                "bf16/bf16/bf16 unscaled, int8/int8/e4m3 [q,k,v], bf16/bf16/e4m3 [v or none], "
                "e4m3/e4m3/e4m3 [q,k,v], bf16/e4m3/e4m3 [k,v], e4m3/e4m3/int8 [q,k,v]; with D=192 the first "
                "five except bf16/bf16/e4m3 without a V scale",
                (int)p->q.dtype, (int)p->k.dtype, (int)p->v.dtype, sb[0], sb[1], sb[2]);
  if (empty) return ok();

  fmha::FwdArgs a{};
  const int qe = elem_size(p->q.dtype), ke = elem_size(p->k.dtype), ve = elem_size(p->v.dtype);
  a.q = static_cast<const uint8_t*>(p->q.ptr);
  a.q_sb = p->q.stride_b * qe; a.q_ss = p->q.stride_s * qe; a.q_sh = p->q.stride_h * qe;
  a.k = static_cast<const uint8_t*>(p->k.ptr);
  a.k_sb = p->k.stride_b * ke; a.k_ss = p->k.stride_s * ke; a.k_sh = p->k.stride_h * ke;
  a.v = static_cast<const uint8_t*>(p->v.ptr);
  a.v_sb = p->v.stride_b * ve; a.v_ss = p->v.stride_s * ve; a.v_sh = p->v.stride_h * ve;
  a.o = static_cast<uint8_t*>(p->o.ptr);
  const int oe = elem_size(p->o.dtype);
  a.o_sb = p->o.stride_b * oe; a.o_ss = p->o.stride_s * oe; a.o_sh = p->o.stride_h * oe;
  a.o_fp8 = p->o.dtype == FMHA_DT_E4M3;
  a.sfs_o = sfs_o;
  a.sfs_q = p->sfs_q; a.sfs_k = p->sfs_k; a.sfs_v = p->sfs_v; a.sfs_p = p->sfs_p;
  a.B = p->B; a.Sq = p->Sq; a.Skv = p->Skv; a.Hq = p->Hq; a.Hkv = p->Hkv; a.group = p->Hq / p->Hkv;
  a.nblk_q = (p->Sq + 63) / 64;
  a.nblk_kv = (p->Skv + 63) / 64;
  const double scale = p->softmax_scale > 0.0f ? (double)p->softmax_scale : 1.0 / std::sqrt((double)p->D);
  a.scale_log2 = (float)(scale / std::log(2.0));
  a.tau = p->lazy_rescale_log2;
  a.causal = p->causal;
  a.mask = p->block_mask;
  a.m_sb = p->mask_stride_b; a.m_sh = p->mask_stride_h; a.m_sqb = p->mask_stride_qb;
  a.mask_kv_sub = p->block_mask ? p->mask_block_kv / 64 : 1;
  a.mask_kv_shift = (a.mask_kv_sub & (a.mask_kv_sub - 1)) == 0 ? __builtin_ctz((unsigned)a.mask_kv_sub) : -1;
  a.page_table = p->page_table;
  a.pt_sb = p->page_table_stride_b;
  a.page_size = paged ? p->page_size : 1;
  a.num_pages = paged ? p->num_pages : 0;
  // every offset inside a pool is below num_pages * page stride (a page holds
  // its page_size slots): 32-bit page offsets when that is under 4 GiB
  a.pool32 = paged && (int64_t)p->num_pages * std::max(a.k_sb, a.v_sb) < ((int64_t)1 << 32) &&
             (int64_t)p->page_size * std::max(a.k_ss, a.v_ss) <= std::max(a.k_sb, a.v_sb);
  // P <= 2^tau / sfs_p; E4M3 conversion needs a clamp once that can reach 464.
  a.clamp_p = (p->sfs_p != nullptr) || (p->lazy_rescale_log2 > 8.5f);
  // Contiguous K/V: with positive token strides and a sequence (plus one
  // sub-tile of overrun) under 2^31 bytes, every tile offset fits the
  // buffer's 32-bit offset, so one resource per workgroup serves all tiles.
  a.kv_whole_rsrc = !paged && a.k_ss > 0 && a.v_ss > 0 &&
                    (int64_t)(p->Skv + 64) * std::max(a.k_ss, a.v_ss) < ((int64_t)1 << 31);
  return hip_status(fmha::launch_fwd(key, a, static_cast<hipStream_t>(stream)), "fwd launch");
}

}  // extern "C"
