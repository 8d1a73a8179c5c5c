"""fp64 CPU oracle for ring-ordered blockwise exact attention.

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this package. The GPU library never calls it and
shares no code with it; it is the reference the HIP kernels are checked against.

Every function is the plain definition, written out in float64 numpy with the
score matrix materialised:
  * attention / attention_rows: softmax(scale * Q K^T) V and the per-row
    log-sum-exp of the scaled scores.
  * merge / merge_n: combining normalised partial results by their LSE.
  * partition_positions / ring_schedule / ring_attention: where each partition's
    tokens sit (contiguous or striped layout), the ring visiting order and the
    blockwise protocol built from the two above (used to pin "blockwise ==
    one-shot").
  * splitkv_decode: the split-KV decode partials and their reduction.
  * e4m3_to_float / dequantize: values of an FP8 (E4M3) KV cache.
  * attention_bwd / block_bwd: exact gradients of attention, whole and per
    (query block, KV block) pair given the saved row LSE.
  * accounting helpers that reproduce the pages' own tables.

Citation keys:
  [RING]  page "AI 推理系列（十一）：Ring Attention 如何让多张 GPU 共同计算一条超长序列"
  [IMPL]  page "LLM长文本推理Ring Attention环形注意力机制实现与优化"
  [CH]    page "长上下文的第一性挑战"
  [CPEV]  page "上下文并行 (CP) 收益评估实验设计"
"""
from .exact import (  # noqa: F401
    LAYOUTS,
    NEG_INF,
    attention,
    attention_rows,
    merge,
    merge_n,
    partition_positions,
    ring_schedule,
    ring_attention,
    splitkv_decode,
    visible,
)
from .fp8 import e4m3_to_float, dequantize  # noqa: F401
from .backward import attention_bwd, block_bwd  # noqa: F401
from .accounting import (  # noqa: F401
    kv_cache_bytes,
    decode_lower_bound_s,
    prefill_compute_time_s,
    visible_pairs_aligned_causal,
    visible_pairs_partition,
    attention_flops,
)
