"""GPU parity at large shapes, through the C ABI.

* A fresh 16384-token prefill of one sequence (Qwen2-7B shape): 512 query
  tiles per KV head, contexts up to 16384 keys.  q_out and both caches are
  checked in full; the attention output on sampled rows (tile and block
  boundaries, the first and last rows), each computed by the oracle as a
  one-row sequence over its own causal context: row i of a fresh prefill
  attends keys 0 .. i, which is exactly a sequence of one row with context
  i + 1 over the same block table.
* 4096 decode sequences with contexts of 1 to 64 tokens: thousands of
  segments per call, the decode's sequence scans over 64 chunks; every row
  against the oracle.
"""
import numpy as np
import pytest

import oracle.reference as R
from paged_gqa_attention_neox_amd import workloads as W
from gpu_common import check_caches, check_out, check_rotated, full_check, require_gpu, run_gpu, \
    run_oracle, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def test_fresh_prefill_16k_sampled_rows():
    n = 16384
    b = W.small_case(1201, "bf16", 28, 4, 128, context_lens=[n], query_lens=[n], num_prefill=1,
                     keep_logical=False)
    sh = b.shape
    say("fresh 16384-token prefill: GPU step")
    res, _ = run_gpu(b)
    say("oracle cache write")
    ora = run_oracle(b, seqs=[])
    check_rotated(res["q_out"], ora["q_out"], "bf16", "q_out")
    check_caches(b, res, ora)
    rows = np.array([0, 1, 15, 16, 31, 32, 33, 63, 64, 511, 512, 1023, 1024, 4095, 4096, 7777,
                     8191, 8192, 12345, 16351, 16352, 16383])
    want = np.full((b.num_tokens, sh.num_heads, sh.head_dim), np.nan)
    for i in rows:
        want[i] = R.attention_varlen(ora["q_out"][i:i + 1], ora["k_cache"], ora["v_cache"],
                                     np.array([0, 1]), np.array([i + 1], np.int32),
                                     b.block_tables[0:1], sh.num_heads, sh.num_kv_heads,
                                     sh.head_dim, sh.block_size, sh.dtype)[0]
    mx, mean = check_out(res["out"], want, "bf16", rows=rows, what="fresh 16k prefill rows")
    say(f"sampled rows: max abs {mx:.3e} mean abs {mean:.3e}")


def test_decode_4096_short_sequences():
    rng = np.random.default_rng(1202)
    ctx = rng.integers(1, 65, size=4096).tolist()
    b = W.small_case(1202, "bf16", 28, 4, 128, context_lens=ctx, query_lens=[1] * len(ctx),
                     num_prefill=0, keep_logical=False)
    full_check(b, label="decode_4096_short")
