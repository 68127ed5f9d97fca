"""Decode segments that many ranges share, through the C ABI.

A (sequence, KV head) segment cut by range boundaries is merged by the range
that completes it.  These batches put one to a few long sequences on the
whole GPU, so every segment spans tens to hundreds of ranges (up to 128
pieces in one merge, in several rounds of loads): both cache formats, one to
eight query heads per KV head, 32- and 64-token cache blocks, long segments
beside short ones, and the cascade's private level (three tiers of ranges, a
segment's pieces in ranges of different tiers).  Every output row against
the oracle.
"""
import numpy as np
import pytest

import oracle.reference as R

from paged_gqa_attention_neox_amd import runner
from paged_gqa_attention_neox_amd import workloads as W
from gpu_common import full_check, require_gpu, say
from test_gpu_cascade import cascade_check

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


FP8 = dict(cache_dtype="fp8", k_scale=W.FP8_K_SCALE, v_scale=W.FP8_V_SCALE)

# label: (H, Hkv, context lengths, extra small_case arguments)
CASES = {
    "one_32k_sequence": (28, 4, [32768], {}),
    "one_131k_sequence_ntk": (28, 4, [131072], dict(rope_scaling=(4.0, 32768))),
    "one_40k_sequence_fp8": (28, 4, [40000], dict(FP8, rope_scaling=(2.0, 32768))),
    "two_20k_sequences_g1": (4, 4, [20000, 19999], {}),
    "one_20k_sequence_g8_one_kv_head": (8, 1, [20000], {}),
    "one_50k_sequence_block32": (28, 4, [50000], dict(block_size=32, rope_scaling=(2.0, 32768))),
    "one_30k_sequence_block64": (28, 4, [30001], dict(block_size=64)),
    "long_and_short": (28, 4, [30000, 17, 1, 4097], {}),
}


@pytest.mark.parametrize("label", list(CASES))
def test_long_segments(label):
    H, Hkv, ctx, kw = CASES[label]
    say(f"{label}: H{H}/{Hkv} contexts {ctx}")
    b = W.small_case(1300 + list(CASES).index(label), "bf16", H, Hkv, 128, context_lens=ctx,
                     query_lens=[1] * len(ctx), num_prefill=0, keep_logical=False, **kw)
    full_check(b, label=label)


@pytest.mark.parametrize("fp8", [False, True])
def test_cascade_long_suffixes(fp8):
    """Three members of a 2048-token prefix with 20K-30K private keys each
    beside two unrelated sequences: about 20K units, so the private level
    takes the three-tier schedule and its long segments span ranges of every
    tier."""
    ctx = [2048 + 30000, 2048 + 25000, 2048 + 20000, 5000, 100]
    b = W.small_case(1320 + int(fp8), "bf16", 28, 4, 128, context_lens=ctx,
                     query_lens=[1] * len(ctx), num_prefill=0, keep_logical=False,
                     **(FP8 if fp8 else {}))
    W.with_prefix_groups(b, [([0, 1, 2], 2048)])
    cascade_check(b, f"cascade_long_suffixes{'_fp8' if fp8 else ''}")


@pytest.mark.parametrize("label", ["one_32k_sequence", "two_20k_sequences_g1", "cascade"])
def test_long_segments_run_to_run_bitwise(label):
    """Which workgroup completes (and so merges) a segment depends on timing;
    the merge order does not: repeated calls give identical bits."""
    if label == "cascade":
        ctx = [2048 + 30000, 2048 + 25000, 2048 + 20000, 5000, 100]
        b = W.small_case(1330, "bf16", 28, 4, 128, context_lens=ctx, query_lens=[1] * len(ctx),
                         num_prefill=0, keep_logical=False)
        W.with_prefix_groups(b, [([0, 1, 2], 2048)])
        dev = runner.DeviceStep(b, cascade=True)
    else:
        H, Hkv, ctx, kw = CASES[label]
        b = W.small_case(1331, "bf16", H, Hkv, 128, context_lens=ctx, query_lens=[1] * len(ctx),
                         num_prefill=0, keep_logical=False, **kw)
        dev = runner.DeviceStep(b)
    dev.rope_write()
    outs = []
    for i in range(4):
        say(f"{label}: decode call {i}")
        dev.out.fill_(float("nan"))          # a segment left unmerged would stay NaN
        dev.decode()
        outs.append(runner.to_host(dev.out).copy())
    assert not np.isnan(R.to_f64(outs[0], "bf16")).any()
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
