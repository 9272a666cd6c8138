"""fp64 CPU oracle for DiT attention, int8-QK attention and the first-block-cache reduction.

TEST INFRASTRUCTURE ONLY.  This package is the slow, plain, obviously-correct definition the
HIP library is checked against.  Only the test suite, the smoke check and the benchmark's CPU
baseline leg may import or run it; the library and its Python binding never do, and this
package imports nothing from them (the two share no code; inputs come from ``datagen``).

Modules:
  attention  -- exact softmax attention and its per-row log-sum-exp (fp64)
  quant      -- K channel mean, per-block symmetric int8 (and fp8 e4m3) quantization, quantized
                attention, the per-call quantization-error probe
  rel_l1     -- relative L1 distance of two residual tensors
  fbcache    -- First Block Cache: the per-step cache decision, residual add / subtract in bf16
"""
from .attention import attention, attention_rows, log_sum_exp
from .quant import (k_channel_mean, smooth_k, quantize_blocks, quantize_qk,
                    attention_int8, log_sum_exp_int8, probe_rows,
                    quant_probe_error, Q_BLOCK, K_BLOCK, QMAX, E4M3_MAX, e4m3_value, e4m3_round,
                    quantize_blocks_fp8, quantize_qk_fp8, attention_fp8, log_sum_exp_fp8,
                    quantize_v_fp8, attention_fp8_full)
from .rel_l1 import rel_l1
from .fbcache import (FBCacheConfig, FBCacheState, fbcache_decide, fbcache_run, bf16_round,
                      resid_add, resid_sub)

__all__ = ["attention", "attention_rows", "log_sum_exp", "log_sum_exp_int8", "k_channel_mean", "smooth_k", "quantize_blocks",
           "quantize_qk", "attention_int8", "rel_l1", "Q_BLOCK", "K_BLOCK",
           "QMAX", "FBCacheConfig", "FBCacheState", "fbcache_decide", "fbcache_run", "bf16_round",
           "resid_add", "resid_sub", "probe_rows", "quant_probe_error", "E4M3_MAX", "e4m3_value",
           "e4m3_round", "quantize_blocks_fp8", "quantize_qk_fp8", "attention_fp8",
           "log_sum_exp_fp8", "quantize_v_fp8", "attention_fp8_full"]
