"""GPU parity of the shared-prefix (cascade) decode,
qwen2_attn_decode_paged_cascade and its FP8 twin, through the C ABI.

The cascade is only an evaluation order of the plain decode (softmax over
each member's whole block table), so the GPU outputs are compared with the
oracle's plain decode definition, attention_decode, on every sequence of
every batch, to the step dtype's tolerance.  The plain decode on the GPU and
the cascade must also agree to that tolerance.
Sequences outside every group, members whose context does not exceed the
prefix, and a reused workspace are covered too.
"""
import numpy as np
import pytest
import torch

import oracle.reference as R
from paged_gqa_attention_neox_amd import binding as B
from paged_gqa_attention_neox_amd import workloads as W
from gpu_common import bits, check_out, require_gpu, run_gpu, run_oracle, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def plain_decode_oracle(b, ora):
    """Oracle outputs of the decode rows by the plain decode definition (each
    member attends to its whole table; no prefix grouping)."""
    sh = b.shape
    Tp = b.num_prefill_tokens
    ctx, bt = b.decode_part()
    return R.attention_decode(ora["q_out"][Tp:], ora["k_cache"], ora["v_cache"], bt, ctx,
                              sh.num_heads, sh.num_kv_heads, sh.head_dim, sh.block_size, sh.dtype,
                              cache_dtype=sh.cache_dtype, k_scale=sh.k_scale, v_scale=sh.v_scale)


def cascade_check(b, label, plain_too=True):
    say(f"{label}: cascade GPU step")
    res, _ = run_gpu(b, cascade=True)
    say(f"{label}: oracle")
    ora = run_oracle(b, seqs=range(b.num_prefill))       # prefill rows by the plain oracle
    Tp = b.num_prefill_tokens
    want = plain_decode_oracle(b, ora)
    dt = b.shape.dtype
    mx, mean = check_out(res["out"][Tp:], want, dt)
    say(f"{label}: decode out max abs {mx:.3e} mean abs {mean:.3e}")
    if b.num_prefill:
        check_out(res["out"][:Tp], ora["out"][:Tp], dt)
    if plain_too:
        plain, _ = run_gpu(b)
        check_out(res["out"][Tp:], plain["out"][Tp:].astype(np.float64) if dt == "f32"
                  else R.to_f64(plain["out"][Tp:], dt), dt, what="cascade vs plain")
    return res


def test_cascade_mixed_tp2_full():
    """The mixed batch at the TP=2 share of Qwen2-7B: 48 of its 96 decode
    sequences share a 1024-token prefix (one group)."""
    cascade_check(W.mixed_tp2(), "mixed_tp2")


def test_cascade_shared_prompt_full():
    """Qwen2-7B decode, 4 groups of 16 sequences sharing a 4096-token
    prompt; every sequence against the plain decode definition."""
    cascade_check(W.shared_prompt_decode(), "shared_prompt")


CASES = [
    # (name, H, Hkv, contexts, groups (decode-local members, prefix tokens), fp8)
    ("g7_two_groups", 28, 4, [300, 1100, 513, 2000, 47, 1040, 700, 129],
     [([1, 3, 5], 1024), ([0, 2, 6], 128)], False),
    ("g2_one_key_suffix", 16, 8, [17, 33, 65, 200], [([0, 1, 2, 3], 16)], False),
    ("g8_many_members", 32, 4, [400 + 37 * i for i in range(40)], [(list(range(0, 40, 2)), 384),
                                                                   (list(range(1, 40, 2)), 256)],
     False),
    ("g1_mha", 4, 4, [90, 200, 150], [([2, 0, 1], 80)], False),
    ("g7_single_member", 28, 4, [500, 3000], [([1], 2048)], False),
    ("g7_long_prefix_chunks", 28, 4, [9000, 8500, 12000], [([0, 1, 2], 8192)], False),
    ("fp8_g7", 28, 4, [300, 1100, 513, 2000, 47], [([1, 3], 256), ([2, 4], 32)], True),
    ("fp8_g8_suffix_in_one_block", 32, 4, [1025, 1030, 1040], [([0, 1, 2], 1024)], True),
    # the private level's schedule switches at 32768 units of suffix blocks:
    # exactly 32768 takes one tier of equal ranges, one unit less the three
    # shrinking tiers
    ("g7_one_tier_at_threshold", 28, 4, [17408] * 8, [(list(range(8)), 1024)], False),
    ("g7_three_tiers_below_threshold", 28, 4, [17408] * 7 + [17392], [(list(range(8)), 1024)],
     False),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_cascade_small_cases(case):
    name, H, Hkv, ctx, groups, fp8 = case
    kw = dict(cache_dtype="fp8", k_scale=W.FP8_K_SCALE, v_scale=W.FP8_V_SCALE) if fp8 else {}
    b = W.small_case(601 + CASES.index(case), "bf16", H, Hkv, 128, context_lens=ctx,
                     query_lens=[1] * len(ctx), num_prefill=0, keep_logical=False, **kw)
    W.with_prefix_groups(b, groups)
    cascade_check(b, f"cascade_{name}")


def test_cascade_member_without_suffix_is_decoded_plainly():
    """A listed member whose context ends inside the prefix breaks the
    grouping contract; the library decodes it over its whole table, so its
    output is still the plain attention (the other members keep the
    cascade)."""
    b = W.small_case(640, "bf16", 28, 4, 128, context_lens=[600, 700, 300], query_lens=[1] * 3,
                     num_prefill=0, keep_logical=False)
    W.with_prefix_groups(b, [([0, 1], 512)])
    # member 2 joins the group with a context shorter than the prefix
    # (its table keeps its own blocks; the prefix group is not used for it)
    ind, seqs, lens = b.prefix_groups
    b.prefix_groups = (np.array([0, 3], np.int32), np.array([0, 1, 2], np.int32), lens)
    res, _ = run_gpu(b, cascade=True)
    ora = run_oracle(b, seqs=[])
    check_out(res["out"], plain_decode_oracle(b, ora), "bf16")


def test_cascade_workspace_reuse():
    """Two calls on one workspace, the second with fewer members and a
    shorter prefix: stale per-sequence state from the first call must not
    leak into the second."""
    b1 = W.small_case(650, "bf16", 28, 4, 128, context_lens=[900, 1000, 1100, 1200],
                      query_lens=[1] * 4, num_prefill=0, keep_logical=False)
    W.with_prefix_groups(b1, [([0, 1, 2, 3], 768)])
    b2 = W.small_case(651, "bf16", 28, 4, 128, context_lens=[900, 1000, 1100, 1200],
                      query_lens=[1] * 4, num_prefill=0, keep_logical=False)
    W.with_prefix_groups(b2, [([2, 3], 256)])
    from paged_gqa_attention_neox_amd import runner
    d1 = runner.DeviceStep(b1, cascade=True)
    d1.step()
    d2 = runner.DeviceStep(b2, cascade=True)
    assert d2.workspace.numel() <= d1.workspace.numel()
    d2.workspace = d1.workspace
    d2.step()
    r2 = d2.results()
    check_out(r2["out"], plain_decode_oracle(b2, run_oracle(b2, seqs=[])), "bf16")


def test_cascade_no_groups_is_plain_decode_bitwise():
    """Without groups the cascade call is the plain decode: bitwise equal."""
    b = W.small_case(660, "bf16", 28, 4, 128, context_lens=[300, 1100, 2000], query_lens=[1] * 3,
                     num_prefill=0, keep_logical=False)
    plain, dev = run_gpu(b)
    out = torch.empty_like(dev.out)
    z = torch.zeros(1, dtype=torch.int32, device="cuda")
    e = torch.zeros(0, dtype=torch.int32, device="cuda")
    sh = b.shape
    ws = torch.empty(B.qwen2_attn_decode_cascade_workspace_size(3, dev.d_max_c, 0, 0, 0, 28, 4,
                                                                128, 16, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")
    B.qwen2_attn_decode_paged_cascade(dev.q_out, dev.k_cache, dev.v_cache, dev.d_bt, dev.d_ctx,
                                      z, e, e, 0, out, ws, dev.d_max_c, 28, 4, 128, 16, sh.scale)
    torch.cuda.synchronize()
    assert np.array_equal(bits(plain["out"]), bits(out.cpu().view(torch.int16).numpy().view(np.uint16)))
