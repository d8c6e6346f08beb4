/*
 * fmha.h -- C ABI of the MI355X (gfx950) mixed-precision attention forward.
 *
 * Three operations, each enqueued on a caller-supplied HIP stream:
 *
 *   fmha_quantize_blocks  per-(batch, head, 64-token block) quantisation of a
 *                         bf16 tensor to int8 or E4M3 codes plus one fp32
 *                         scale per block (SageAttention-style block scale
 *                         factors); fmha_quantize_blocks_batch does several
 *                         in one launch.
 *   fmha_fwd              fused attention forward over int8 / E4M3 / bf16
 *                         Q, K, V with per-block scale factors, online softmax
 *                         with lazy rescaling, P requantised to the V format,
 *                         causal / GQA / block-sparse / paged-KV options, and
 *                         a bf16 output.
 *   fmha_quantize_nvfp4   per-token NVFP4 quantisation of a bf16 activation
 *                         matrix (E2M1 codes, E4M3 16-element block scales,
 *                         one fp32 scale per token).
 *
 * Sources (FlashInfer pull-request write-ups):
 *   #2711 page "FlashInfer의 DiT 최적화: SageAttention과 Int8/FP8 혼합 정밀도
 *     커널 도입 분석": 코드 분석 1 (kernel choice keyed by the Q, K, V, O dtypes
 *     and the number of elements per Q/K/P/V scale factor), 코드 분석 2 (four
 *     scale-factor pointers for Q, K, P, V, applied after BMM1/BMM2).
 *   #5900 page "Blackwell 아키텍처를 위한 FlashInfer의 FP8/BF16 혼합 정밀도
 *     Attention 최적화 분석": title and 코드 분석 1 (QK in bf16 or fp8, PV in
 *     fp8, 16-bit output, head dim 128), 코드 분석 3 (lazy correction: O is
 *     rescaled only when the row maximum grows by 2^8), 리뷰어 피드백 반영
 *     (head dim 192 and an FP8 output as configurations of the family).
 *   #4474 page "FlashInfer의 PrimTS를 활용한 고성능 Block-Sparse Attention
 *     최적화": 코드 분석 1 (Q64 x KV256 tiles; query heads per KV head),
 *     코드 분석 2 (block-sparse attention over contiguous or paged K/V taking
 *     q, the paged cache and a page table).
 *   #3237 page "FlashInfer의 Per-token NVFP4 Quantization 커널 최적화 분석":
 *     코드 분석 1-2 (per-token NVFP4 quantisation kernel, linear scale-factor
 *     layout, the input read once for the row maximum and the encoding).
 *
 * Conventions common to every call:
 *   - Every data pointer (an argument, or inside a tensor or params struct)
 *     is a DEVICE pointer; the structs themselves live in host memory and are
 *     read during the call only.  The caller owns every buffer; the library allocates nothing and
 *     keeps no pointer after returning.
 *   - Arguments are validated before any HIP call.  On a validation failure
 *     nothing is enqueued and the call returns FMHA_ERR_INVALID or
 *     FMHA_ERR_UNSUPPORTED; fmha_last_error() describes the problem.
 *   - Work is enqueued asynchronously; faults surface at the caller's next
 *     synchronisation.  A launch error returns FMHA_ERR_HIP.
 *   - Results are deterministic: identical inputs give identical bits.
 *   - Calls on different streams may overlap; the library has no global
 *     mutable state other than the thread-local error string and a per-kernel
 *     flag recording that its LDS-size attribute was set (setting it twice
 *     is harmless).
 */
#ifndef FMHA_H_
#define FMHA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element formats.  E4M3 is the OCP 8-bit float "e4m3fn" (bias 7, max 448,
 * no infinities, NaN = S.1111.111), the format NVIDIA calls E4M3. */
typedef enum {
  FMHA_DT_BF16 = 1,
  FMHA_DT_E4M3 = 2,
  FMHA_DT_INT8 = 3
} fmha_dtype;

enum {
  FMHA_OK = 0,
  FMHA_ERR_INVALID = -1,     /* bad pointer, size, stride or alignment */
  FMHA_ERR_UNSUPPORTED = -2, /* valid request, no kernel for this combination */
  FMHA_ERR_HIP = -3          /* the HIP runtime reported an error */
};

/* A strided 4-D tensor [B, S, H, D] whose channel (D) dimension is
 * contiguous.  Strides are in ELEMENTS.  ptr and every stride times the
 * element size must be multiples of 16 bytes. */
typedef struct {
  void* ptr;
  int32_t dtype;             /* fmha_dtype */
  int64_t stride_b;
  int64_t stride_s;
  int64_t stride_h;
} fmha_tensor;

/* hipStream_t passed as an opaque pointer (NULL = the default stream). */
typedef void* fmha_stream_t;

/*
 * fmha_quantize_blocks -- block scale factors and codes (#2711 page, 코드 분석 2).
 *
 * For every (b, h) and every block of block_tokens consecutive tokens
 * [64*k, min(64*k + 64, S)) (the last block may be partial):
 *   amax  = max |x| over the block's tokens and all D channels (fp32);
 *   if amax < 2^-126 (including 0): scale = 1.0f and every code = 0;
 *   else scale = amax / Qmax, inv = Qmax / amax (both correctly rounded fp32),
 *        code  = encode(x * inv) (fp32 product, round to nearest even),
 * with Qmax = 127 for FMHA_DT_INT8 (codes in [-127, 127]) and 448 for
 * FMHA_DT_E4M3 (round to nearest even code, saturating).
 *
 *   x       [B, S, H, D] bf16 (x->dtype == FMHA_DT_BF16); read only.
 *   codes   [B, S, H, D] int8 or E4M3 (codes->dtype); written.  May not
 *           overlap x.
 *   scales  fp32 [B, H, ceil(S / block_tokens)], contiguous; written.
 *   D must be 128 or 192 and block_tokens 64.  B, S or H equal to 0 is a
 *   no-op.
 */
int fmha_quantize_blocks(const fmha_tensor* x, const fmha_tensor* codes,
                         float* scales, int32_t B, int32_t S, int32_t H,
                         int32_t D, int32_t block_tokens, fmha_stream_t stream);

/*
 * fmha_quantize_blocks_batch -- up to FMHA_MAX_QUANTIZE_JOBS block
 * quantisations in one launch (the Q, K and V of one attention call: the
 * #2711 page quantises all three with their own scale factors, 코드 분석 2).
 * Each job is exactly one fmha_quantize_blocks call (same arguments, same
 * results bit for bit); jobs may mix int8 and E4M3 codes and shapes, but not
 * head dims (every job's D must equal job 0's, else FMHA_ERR_UNSUPPORTED).
 * No job's codes or scales may overlap another job's input or output.
 * Every job is validated before any HIP call; an error names the job.
 * n_jobs == 0 is a no-op; n_jobs outside [0, FMHA_MAX_QUANTIZE_JOBS] is
 * FMHA_ERR_INVALID.
 */
#define FMHA_MAX_QUANTIZE_JOBS 8
typedef struct {
  fmha_tensor x;          /* bf16 [B, S, H, D]; read only */
  fmha_tensor codes;      /* int8 or E4M3 [B, S, H, D]; written */
  float* scales;          /* fp32 [B, H, ceil(S / block_tokens)], contiguous */
  int32_t B, S, H, D;
  int32_t block_tokens;   /* 64 */
} fmha_quantize_job;

int fmha_quantize_blocks_batch(const fmha_quantize_job* jobs, int32_t n_jobs,
                               fmha_stream_t stream);

/*
 * Parameters of fmha_fwd.  Zero-initialise, then set struct_size =
 * sizeof(fmha_fwd_params) and the fields used.
 */
typedef struct {
  uint32_t struct_size;
  int32_t B, Sq, Skv, Hq, Hkv, D;  /* D == 128 or 192 (at 192, bf16/bf16/e4m3
                                      needs the V scale); Hq % Hkv == 0; query
                                      head h reads key/value head
                                      h / (Hq / Hkv) */
  /* q: [B, Sq, Hq, D]; o: [B, Sq, Hq, D] bf16 or E4M3 (written).
   * k, v contiguous-cache case: [B, Skv, Hkv, D].
   * k, v paged case (page_table != NULL): pools [num_pages, page_size, Hkv, D]
   * where stride_b is the stride between pages and stride_s the stride
   * between the slots of one page.  The token (slot) stride of k and v must
   * be at least D elements (FMHA_ERR_INVALID otherwise: no broadcast or
   * overlapping key/value rows). */
  fmha_tensor q, k, v, o;
  /* Per-block scale factors, fp32 [B, H, ceil(S / 64)] contiguous (H = Hq for
   * sfs_q, Hkv for sfs_k / sfs_v; S = Sq or Skv, counted in logical tokens),
   * or NULL for an unscaled operand.  An int8 / E4M3 Q or K needs its scale
   * (sage_block = 64); V may be E4M3 with (64) or without (0) a scale, and
   * an int8 V needs its scale. */
  const float* sfs_q;
  const float* sfs_k;
  const float* sfs_v;
  int32_t sage_block_q, sage_block_k, sage_block_v; /* 0 (unscaled) or 64 */
  /* Static per-query-head dequantisation scale of P, fp32 [Hq], or NULL
   * (= 1.0): P is quantised as encode(P / sfs_p[h]) before BMM2. */
  const float* sfs_p;
  float softmax_scale;       /* <= 0 selects 1 / sqrt(D) */
  float lazy_rescale_log2;   /* tau: rescale O only when the row maximum of
                                the log2-domain scores grows by more than tau;
                                0 rescales on every increase.  Must be in
                                [0, 16]; the usual value is 8. */
  int32_t causal;            /* key j visible from query i iff j <= i + Skv - Sq */
  /* Block-sparse mask, uint8 [B, Hq, ceil(Sq / mask_block_q),
   * ceil(Skv / mask_block_kv)] with the given element strides (0 broadcasts),
   * last dimension contiguous; non-zero = the (query block, key block) pair
   * takes part.  NULL = dense. */
  const uint8_t* block_mask;
  int64_t mask_stride_b, mask_stride_h, mask_stride_qb;
  int32_t mask_block_q, mask_block_kv;   /* 64, 256 */
  /* Paged K/V: int32 [B, ceil(Skv / page_size)] with row stride
   * page_table_stride_b; entry p of row b is the pool page holding logical
   * tokens [p * page_size, (p + 1) * page_size).  An entry outside
   * [0, num_pages) is read as page 0 (no access outside the pool; the
   * output for such tokens is unspecified).  NULL = contiguous K/V. */
  const int32_t* page_table;
  int64_t page_table_stride_b;
  int32_t page_size;         /* tokens per page: a power of two >= 16 (16 in the block-sparse workload) */
  int32_t num_pages;
  /* Static per-query-head output scale, fp32 [Hq], for an E4M3 o, or NULL
   * (= 1.0): o = encode(O / sfs_o[h]), E4M3 nearest-even, saturating at
   * +-448.  Must be NULL for a bf16 o.  A caller built against the previous
   * layout (struct_size = offsetof(fmha_fwd_params, sfs_o)) gets NULL. */
  const float* sfs_o;
} fmha_fwd_params;

/*
 * fmha_fwd -- o = attention(q, k, v) with block-scaled operands.
 *
 * Per (b, query head h, query row i), with scores in log2 units
 *   s2[j] = (Q[i] . K[j]) * sfs_q * sfs_k * softmax_scale * log2(e)
 * over the valid keys j (tail, causal, block mask), keys are visited in
 * ascending 64-key sub-tiles; the reference maximum m moves to a sub-tile's
 * maximum t only when m is unset or t - m > tau, and only then are the
 * running numerator and denominator multiplied by 2^(m - t).
 *   P = 2^(s2 - m);  w = Qp(P / sp) * sp  (Qp = E4M3 for an E4M3 or an
 *   int8 V, bf16 for a bf16 V; sp = sfs_p[h] or 1);  num += w V[j] * sfs_v;
 *   den += w.
 *   o[i] = bf16(num / den), or 0 for a row without a valid key; an E4M3 o
 *   holds encode(num / den / so) instead (so = sfs_o[h] or 1).
 *
 * Supported (q, k, v) formats, with the scaled operands in brackets:
 *   (bf16, bf16, bf16)          unscaled
 *   (int8, int8, e4m3)          [q, k, v]
 *   (bf16, bf16, e4m3)          [v] or none
 *   (e4m3, e4m3, e4m3)          [q, k, v]
 *   (bf16, e4m3, e4m3)          [k, v]
 *   (e4m3, e4m3, int8)          [q, k, v], head dim 128: the #2711 page's
 *                               K-fp8 / V-int8 example of separate K and V
 *                               types (왜 이게 좋은 최적화인가? 3); V codes
 *                               are amax/127 block codes as fmha_quantize_blocks
 *                               writes them
 * o is bf16 or E4M3 for each of them.  Other combinations return
 * FMHA_ERR_UNSUPPORTED.
 */
int fmha_fwd(const fmha_fwd_params* p, fmha_stream_t stream);

/*
 * fmha_quantize_nvfp4 -- per-token NVFP4 quantisation (#3237 page, 코드 분석
 * 1-2).  The page names the kernel but not the format; the public NVFP4
 * definition is used: E2M1 elements (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6),
 * one E4M3 scale per 16 consecutive elements, one fp32 scale per token.
 *
 * For every row r of x [M, K] (fp32 arithmetic, correctly rounded, nearest
 * even, no flush to zero):
 *   amax = max |x[r, :]|;
 *   if amax < 2^-116 (zero rows included): ts = 1, g6 = 0;
 *   else ts = amax / 2688, g6 = 448 / amax              (2688 = 6 * 448);
 *   for each block j of 16 elements (bmax = max |x| over the block):
 *     sf  = E4M3(min(bmax * g6, 448));
 *     bs  = dec(sf) * ts;
 *     es  = bs > 0 ? min(1 / bs, FLT_MAX) : 0;
 *     code[k] = E2M1(x[r, 16j + k] * es)  (saturating at +-6, sign of zero kept);
 * so x ~ E2M1 value * dec(sf) * ts, and the largest element of a row maps to
 * +-6 in a block whose scale is 448.
 *
 *   x             bf16 [M, K]; row stride x_row_stride in ELEMENTS (>= K, a
 *                 multiple of 8); 16-byte aligned; read only.
 *   codes         uint8 [M, K/2]: element 2i in the low nibble of byte i;
 *                 row stride codes_row_stride in BYTES (>= K/2, a multiple
 *                 of 8); 8-byte aligned; written.
 *   block_scales  uint8 [M, K/16] E4M3 bit patterns, linear (row-major);
 *                 row stride scales_row_stride in BYTES (>= K/16); written.
 *   token_scales  fp32 [M], contiguous, 4-byte aligned; written.
 *   K must be a positive multiple of 16 (at most 2^28, else
 *   FMHA_ERR_UNSUPPORTED); M == 0 is a no-op.  Outputs may not
 *   overlap x or each other.  Inputs are finite.
 */
int fmha_quantize_nvfp4(const void* x, int64_t x_row_stride, int32_t M, int32_t K,
                        uint8_t* codes, int64_t codes_row_stride,
                        uint8_t* block_scales, int64_t scales_row_stride,
                        float* token_scales, fmha_stream_t stream);

/* Description of the last error on the calling thread ("" after success);
 * valid until the next fmha_* call on that thread. */
const char* fmha_last_error(void);

/* ABI version: 0xMMmmpp (0x000300: fmha_quantize_nvfp4 added; 0x000400:
 * fmha_quantize_blocks_batch added). */
uint32_t fmha_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FMHA_H_ */
