"""The generic path (shapes the tuned kernels do not take: head_dim 64, fp32
storage, more than 8 query heads per KV head, FP8 prefill at head_dim 64),
through the C ABI.

Prefill rows run one wave per row, or one workgroup of sixteen waves per row
when every row's context is long (at least 2048 keys and four times the
longest chunk: chunks after long prefixes); decode rows run one workgroup of
sixteen waves per (sequence, head).  These cases put chunks after long
prefixes (the workgroup-per-row kernel) beside cases just under its
threshold (the wave-per-row kernel), with 16-, 32- and 64-token blocks and
mixed batches.  Every row against the oracle.
"""
import pytest

from paged_gqa_attention_neox_amd import workloads as W
from gpu_common import full_check, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


FP8 = dict(cache_dtype="fp8", k_scale=W.FP8_K_SCALE, v_scale=W.FP8_V_SCALE)

# label: (dtype, H, Hkv, d, context lengths, query lengths, prefill sequences, extra arguments)
CASES = {
    "d64_chunks_after_5000": ("bf16", 14, 2, 64, [5064, 5001], [64, 1], 1, {}),
    "f32_d64_chunk_after_3000": ("f32", 4, 2, 64, [3100], [100], 1, {}),
    "g10_d128_chunks_after_2500": ("bf16", 20, 2, 128, [2532, 2510], [32, 10], 2, {}),
    "fp8_d64_chunk_after_4000": ("bf16", 14, 2, 64, [4048], [48], 1, FP8),
    "d64_block32_chunk_after_4096": ("bf16", 14, 2, 64, [4163], [67], 1, dict(block_size=32)),
    "d64_block64_chunk_after_2100": ("bf16", 8, 1, 64, [2200, 3000, 77], [100, 1, 1], 1,
                                     dict(block_size=64)),
    "d64_under_threshold": ("bf16", 14, 2, 64, [2047, 900], [16, 1], 1, {}),
    "d64_fresh_prefill": ("bf16", 14, 2, 64, [300, 257, 1], [300, 257, 1], 3, {}),
    "f32_d64_mixed": ("f32", 4, 2, 64, [2600, 40, 3333, 1], [40, 40, 1, 1], 2, {}),
}


@pytest.mark.parametrize("label", list(CASES))
def test_generic_path(label):
    dt, H, Hkv, d, ctx, ql, npf, kw = CASES[label]
    say(f"{label}: {dt} H{H}/{Hkv} d{d} contexts {ctx} rows {ql}")
    b = W.small_case(1400 + list(CASES).index(label), dt, H, Hkv, d, context_lens=ctx,
                     query_lens=ql, num_prefill=npf, keep_logical=False, **kw)
    full_check(b, label=label)
