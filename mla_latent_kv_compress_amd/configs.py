"""Layer shapes and the five synthetic workloads the library is tested and measured on.

Shapes follow the model configuration keys the MLA page lists ([MTRT], sections "为什么长上下文
必须压缩 KV 缓存", "MLA 的两个核心部件" and "源码里的压缩全流程": hidden 5120, 128 heads,
q_lora_rank 1536, kv_lora_rank 512, qk_rope_head_dim 64, per-head k_nope/v of 128).  The Lite
shape has no query compression (a single q_proj).
"""
from dataclasses import dataclass, field
import math

PAGE_SIZE = 64


@dataclass(frozen=True)
class LayerShape:
    hidden_size: int
    num_heads: int
    q_lora_rank: int              # 0: single q_proj
    kv_lora_rank: int
    qk_nope_head_dim: int
    qk_rope_head_dim: int
    v_head_dim: int
    rope_theta: float = 10000.0
    rms_eps: float = 1e-6
    softmax_scale: float = 0.0    # 0: 1/sqrt(qk_nope_head_dim + qk_rope_head_dim)
    # YaRN frequency interpolation of the rotary embedding (rope_factor <= 1: off); the pages give
    # no constants, so none of the workloads uses it
    rope_factor: float = 0.0
    rope_original_max_position: int = 0
    rope_beta_fast: float = 0.0
    rope_beta_slow: float = 0.0
    rope_mscale: float = 0.0

    @property
    def row_width(self):
        return self.kv_lora_rank + self.qk_rope_head_dim

    @property
    def qk_head_dim(self):
        return self.qk_nope_head_dim + self.qk_rope_head_dim

    @property
    def sigma(self):
        return self.softmax_scale or 1.0 / math.sqrt(self.qk_head_dim)

    def weight_shapes(self):
        """(name, shape) in (out, in) linear-layer layout, in draw order."""
        H, D = self.num_heads, self.hidden_size
        out = []
        if self.q_lora_rank:
            out += [("q_a_proj", (self.q_lora_rank, D)), ("q_a_norm", (self.q_lora_rank,)),
                    ("q_b_proj", (H * self.qk_head_dim, self.q_lora_rank))]
        else:
            out += [("q_proj", (H * self.qk_head_dim, D))]
        out += [("kv_a_proj", (self.row_width, D)), ("kv_a_norm", (self.kv_lora_rank,)),
                ("kv_b_proj", (H * (self.qk_nope_head_dim + self.v_head_dim), self.kv_lora_rank))]
        return out


TINY = LayerShape(256, 4, 96, 64, 32, 16, 32)
LITE = LayerShape(2048, 16, 0, 512, 128, 64, 128)
DSV2 = LayerShape(5120, 128, 1536, 512, 128, 64, 128)


@dataclass(frozen=True)
class Workload:
    name: str
    shape: LayerShape
    act_dtype: str                 # "f32" | "bf16"
    cache_dtype: str               # "f32" | "bf16" | "fp8"
    decode_batch: int
    history: int = 0               # cached tokens per sequence before the decode token
    history_range: tuple = None    # (lo, hi) inclusive: ragged history lengths
    num_splits: int = 0            # 0: chosen by the library
    prefill_seqs: int = 0
    prefill_len: int = 0
    prefill_chunk: int = 0
    description: str = field(default="", compare=False)


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_f32", TINY, "f32", "f32", decode_batch=1, history=128,
                 description="tiny fp32 layer, batch 1, 128 cached tokens + 1 decode token"),
        Workload("lite_bf16", LITE, "bf16", "bf16", decode_batch=32, history=4096,
                 description="Lite-shaped bf16 layer, decode batch 32 x 4096 cached tokens"),
        Workload("dsv2_bf16", DSV2, "bf16", "bf16", decode_batch=64, history=8192,
                 description="236B-shaped bf16 layer, decode batch 64 x 8192 cached tokens"),
        Workload("dsv2_128k", DSV2, "bf16", "bf16", decode_batch=4, history=131072, num_splits=64,
                 description="236B shape, decode batch 4 x 131072 cached tokens, 64 splits"),
        Workload("dsv2_mixed_fp8", DSV2, "bf16", "fp8", decode_batch=128, history_range=(512, 32768),
                 prefill_seqs=4, prefill_len=4096, prefill_chunk=1024,
                 description="236B shape, fp8 e4m3 cache: chunked prefill 4 x 4096 (chunks of 1024) "
                             "plus ragged decode batch 128 with 512..32768 cached tokens"),
    ]
}
