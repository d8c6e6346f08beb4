"""Slow, plain CPU oracle for the mixed-precision attention forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only the test-suite, the smoke check in ``__graft_entry__`` and the CPU-baseline
leg of ``bench.py`` may call it.  It shares no code with the HIP library.

Sources (web pages, each a write-up of one merged FlashInfer pull request;
cited below by PR number, section and, where useful, bullet):

* #2711 page -- "FlashInfer의 DiT 최적화: SageAttention과 Int8/FP8 혼합 정밀도
  커널 도입 분석" (DiT kernels: SageAttention block scale factors, separate
  Q/K/V/O dtypes).
* #5900 page -- "Blackwell 아키텍처를 위한 FlashInfer의 FP8/BF16 혼합 정밀도
  Attention 최적화 분석" (QK-BF16/PV-FP8 and all-FP8 dense context FMHA, lazy
  correction).
* #4474 page -- "FlashInfer의 PrimTS를 활용한 고성능 Block-Sparse Attention
  최적화" (Q64xKV256 profile, block-sparse attention over contiguous or paged
  K/V).
* #3237 page -- "FlashInfer의 Per-token NVFP4 Quantization 커널 최적화 분석"
  (per-token NVFP4 quantisation of activations).

Modules:
  codecs     -- bf16 / OCP-E4M3 / int8 encoders and decoders (closed form).
  quantize   -- per-(batch, head, 64-token block) quantisation.
  attention  -- attention over dequantised tensors, emulating P quantisation
                and the lazy rescale; also exact and unquantised variants.
  nvfp4      -- per-token NVFP4 (E2M1 elements, E4M3 16-element block scales,
                fp32 token scale) quantisation.

Every function states the passage it follows; where the pages are silent the
reading taken is stated at the point of use.
"""
from . import codecs, quantize, attention, nvfp4  # noqa: F401
