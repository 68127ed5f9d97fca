"""qwen2_attn_decode_paged_noalloc through the C ABI against
qwen2_attn_decode_paged on the same inputs: two calls in a row on the
library's per-GPU scratch, the second with a smaller batch (fewer ranges and
partial states than the first left behind), each bitwise equal to the
workspace entry point's output (same kernels) and within the bf16 bar of it.
"""
import numpy as np
import pytest
import torch

import oracle.reference as R
from paged_gqa_attention_neox_amd import binding as B
from paged_gqa_attention_neox_amd import runner
from paged_gqa_attention_neox_amd import workloads as W
from gpu_common import bits, check_out, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _both(b):
    """Decode output of the workspace entry point and of the no-alloc one."""
    dev = runner.DeviceStep(b)
    dev.rope_write()
    dev.decode()
    sh = b.shape
    out2 = torch.full_like(dev.out, float("nan"))
    B.qwen2_attn_decode_paged_noalloc(dev.q_out, dev.k_cache, dev.v_cache, dev.d_bt, dev.d_ctx,
                                      out2, dev.d_max_c, sh.num_heads, sh.num_kv_heads,
                                      sh.head_dim, sh.block_size, sh.scale)
    torch.cuda.synchronize()
    return runner.to_host(dev.out), runner.to_host(out2)


def test_noalloc_matches_workspace_decode_twice_shrinking():
    big = W.small_case(701, "bf16", 28, 4, 128, context_lens=[9000, 300, 17, 4096, 2049, 1, 700, 12345],
                       query_lens=[1] * 8, num_prefill=0, keep_logical=False)
    small = W.small_case(702, "bf16", 28, 4, 128, context_lens=[513, 40, 1025],
                         query_lens=[1] * 3, num_prefill=0, keep_logical=False)
    for name, b in (("first call, 8 sequences up to 12345 tokens", big),
                    ("second call, 3 sequences up to 1025 tokens", small)):
        say(f"no-alloc decode: {name}")
        want, got = _both(b)
        assert np.array_equal(bits(got), bits(want)), name
        check_out(got, R.to_f64(want, "bf16"), "bf16", what=f"no-alloc vs workspace ({name})")
