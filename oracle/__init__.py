"""CPU oracle for paged grouped-query attention with NeoX rotary embedding.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything under ``oracle/``: only the tests, the smoke check's parity
comparison and the benchmark's CPU-baseline leg use it.  The oracle shares no
code, table or constant generator with the HIP library; it is a plain, slow,
obviously correct restatement of what the path computes, in float64 numpy.

Every function cites the passage of the reference pages it follows.  Pages are
named by title (and host), sections by the page's own numbering:

  * [P1] "Qwen2 模型结构代码详解" (lpnh.cn) -- config fields, GQA ratio, head
    split, rope_theta default.
  * [P2] "Qwen2大模型架构解析与vLLM优化实践" (intelliparadigm.com) -- fused QKV
    projection, GQA, get_rope(head_dim, rotary_dim=head_dim, base=rope_theta),
    Attention(num_heads, head_dim, scaling, num_kv_heads, cache_config),
    precomputed causal mask.
  * [P3] "vLLM 部署 Qwen" (gsyq.cn) -- PagedAttention: the KV cache cut into
    fixed-size blocks allocated like OS pages; continuous batching; block size.
  * [P4] "Qwen 开源工程笔记" (0539edu.com) -- FlashAttention-2 variable-length
    (packed) prefill.
  * [P5] "nano-vllm: Qwen3 骨架" (adg.csdn.net) -- per-sequence block table,
    Qwen3 attention shape.

Parity status: every function here is pinned by a CPU test against something
other than itself (closed forms, textbook values, a library routine on a
special case, brute force on tiny inputs, invariants); none is "parity
unpinned".
"""
from .reference import (  # noqa: F401
    rope_inv_freq,
    rope_neox,
    to_f64,
    from_f64,
    f64_to_bf16_bits,
    bf16_bits_to_f64,
    rope_cache_write,
    gather_kv,
    causal_visible,
    softmax_rows,
    kv_head_for,
    default_scale,
    attention_varlen,
    attention_decode,
    run_step,
)
