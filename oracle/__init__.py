"""CPU oracle for MLA over a compressed latent KV cache: plain, slow, fp64, obviously correct.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
leg may import this package.  The GPU library (mla_latent_kv_compress_amd) never imports it,
and the two share no code: no kernels, helpers, tables or constants.  The only code both sides
use is the seeded input generator, which holds none of the method's arithmetic.

Pages cited in this package:
  [MTRT]       "DeepSeek-Coder-V2的MLA多头潜在注意力深度解析 512维潜空间压缩KV缓存的完整原理",
               http://www.mtrt.cn/news/26941 -- the authority for what is computed.
  [WIKI]       "什么是多头潜在注意力（Multi-head Latent Attention）？",
               https://www.aiboss88.com/news/wiki-multi-head-latent-attention
  [HOTDRY-OPT] "DeepSeek-V3.2-Exp 中多头潜在注意力的优化：潜在向量压缩与头剪枝",
               https://blog.hotdry.top/agent/posts/2025/09/29/optimize-multi-head-latent-attention-deepseek-v3-2-exp/

Pins: every function is checked by tests/test_oracle_*.py against closed forms, invariants,
library routines (torch's bfloat16 and float8_e4m3fn conversions) and an independent scalar
brute force.  No page prints a worked numeric example of the attention output, so the output
values themselves are pinned only through those checks (see the design notes, "parity
unpinned").
"""
from .mla import (Dims, rms_norm, rope, rope_frequencies, kv_rows, cache_rows, queries, head_weights, softmax,
                  attend_explicit, attend_absorbed, decode_one, prefill_chunk, output_projection)
from .numerics import (E4M3_MAX, fp32_round, bf16_round, e4m3_quantise, e4m3_encode_values,
                       e4m3_decode_codes, fp8_store, store_rows)

__all__ = [
    "Dims", "rms_norm", "rope", "rope_frequencies", "kv_rows", "cache_rows", "queries", "head_weights", "softmax",
    "attend_explicit", "attend_absorbed", "decode_one", "prefill_chunk", "output_projection",
    "E4M3_MAX", "fp32_round", "bf16_round", "e4m3_quantise", "e4m3_encode_values",
    "e4m3_decode_codes", "fp8_store", "store_rows",
]
