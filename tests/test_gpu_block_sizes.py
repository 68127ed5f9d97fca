"""GPU parity with 32- and 64-token cache blocks, through the C ABI.

The matrix-core kernels read a cache block of 16 << k tokens as 2^k
16-token blocks (sub-block b % 2^k of table entry b >> k), and the rope
writer scatters into the longer K rows and V dims rows.  Every case runs
the whole step (rope + cache write, prefill, decode) and compares with the
oracle, whose paged layout takes the block size as a parameter: q_out and
the caches bitwise (K within the rotation bound), outputs to the step
dtype's tolerance.  Ragged contexts end inside a sub-block, inside the
first or last sub-block of an entry, and exactly on entry boundaries.
"""
import pytest

from paged_gqa_attention_neox_amd import workloads as W
from gpu_common import full_check, key_groups, require_gpu, say
from test_gpu_cascade import cascade_check

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


_EDGES = [1, 15, 16, 17, 31, 32, 33, 47, 48, 63, 64, 65, 127, 128, 129, 511, 513, 1025, 1600]
_FP8 = dict(cache_dtype="fp8", k_scale=W.FP8_K_SCALE, v_scale=W.FP8_V_SCALE)

CASES = [
    # (name, block size, dtype, H, Hkv, d, contexts, query lens, num_prefill, extra)
    ("decode_edges_b32", 32, "bf16", 28, 4, 128, _EDGES, [1] * len(_EDGES), 0, {}),
    ("decode_edges_b64", 64, "bf16", 28, 4, 128, _EDGES, [1] * len(_EDGES), 0, {}),
    # long segments: a wave's blocks run past its first 64 block ids
    ("decode_long_b64", 64, "bf16", 28, 4, 128, [9000, 3000, 70], [1] * 3, 0, {}),
    ("decode_g2_b32", 32, "bf16", 16, 8, 128, [129, 2048, 1, 700], [1] * 4, 0, {}),
    ("decode_g8_b64", 64, "bf16", 32, 4, 128, [777, 1500], [1] * 2, 0, {}),
    ("decode_g1_b32", 32, "bf16", 4, 4, 128, [300, 700, 3], [1] * 3, 0, {}),
    # 65536 (sequence, KV head, 16-token block) units: one range per CU
    ("decode_256_ranges_b32", 32, "bf16", 28, 4, 128, [16384] * 16, [1] * 16, 0, {}),
    ("decode_fp8_b32", 32, "bf16", 28, 4, 128, _EDGES, [1] * len(_EDGES), 0, _FP8),
    ("decode_fp8_b64", 64, "bf16", 28, 4, 128, [5000, 65, 64, 1], [1] * 4, 0, _FP8),
    ("prefill_ragged_b32", 32, "bf16", 28, 4, 128, [1, 17, 64, 65, 130, 200],
     [1, 17, 64, 65, 130, 200], 6, {}),
    ("prefill_ragged_b64", 64, "bf16", 28, 4, 128, [1, 17, 64, 65, 130, 200],
     [1, 17, 64, 65, 130, 200], 6, {}),
    ("prefill_chunks_b64", 64, "bf16", 14, 2, 128, [100, 700, 48], [37, 300, 48], 3, {}),
    ("prefill_g2_b32", 32, "bf16", 16, 8, 128, [500, 33], [200, 33], 2, {}),
    ("prefill_fp8_b32", 32, "bf16", 28, 4, 128, [300, 90, 513], [300, 90, 100], 3, _FP8),
    ("prefill_fp8_b64", 64, "bf16", 28, 4, 128, [1, 65, 130], [1, 65, 130], 3, _FP8),
    ("mixed_b32", 32, "bf16", 28, 4, 128, [90, 300, 2000, 1, 513], [90, 44, 1, 1, 1], 2, {}),
    ("mixed_b64", 64, "bf16", 28, 4, 128, [90, 300, 2000, 1, 513], [90, 44, 1, 1, 1], 2, {}),
    # the generic kernel (head_dim 64, fp32 storage) with longer blocks
    ("generic_d64_b32", 32, "bf16", 8, 2, 64, [70, 530, 33], [70, 5, 1], 2, {}),
    ("generic_f32_b64", 64, "f32", 8, 2, 128, [70, 530], [70, 1], 1, {}),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_block_size_cases(case):
    name, bs, dt, H, Hkv, d, ctx, ql, npf, kw = case
    b = W.small_case(700 + CASES.index(case), dt, H, Hkv, d, context_lens=ctx, query_lens=ql,
                     num_prefill=npf, block_size=bs, keep_logical=False, **kw)
    full_check(b, label=name)


TWO_GROUP = [
    # short query tiles over long contexts: the two-key-group prefill layout
    ("prefill_2group_g7_b32", 32, 28, 4, [1537, 700], [512, 100]),
    ("prefill_2group_short_prefix_b64", 64, 28, 4, [2000, 56], [40, 36]),
]


@pytest.mark.parametrize("case", TWO_GROUP, ids=[c[0] for c in TWO_GROUP])
def test_block_size_two_key_groups(case):
    name, bs, H, Hkv, ctx, ql = case
    assert key_groups(ctx, ql, Hkv, H) == 2, name
    b = W.small_case(740 + TWO_GROUP.index(case), "bf16", H, Hkv, 128, context_lens=ctx,
                     query_lens=ql, num_prefill=len(ql), block_size=bs, keep_logical=False)
    full_check(b, label=name)


CASCADE = [
    # (name, block size, contexts, groups (members, prefix tokens), fp8)
    ("cascade_b32", 32, [300, 1100, 513, 2000, 47, 1040, 700, 129],
     [([1, 3, 5], 1024), ([0, 2, 6], 128)], False),
    ("cascade_b64", 64, [900, 1000, 1100, 1200, 70], [([0, 1, 2, 3], 768)], False),
    ("cascade_fp8_b64", 64, [1025, 1030, 1040, 2000], [([0, 1, 2], 1024)], True),
]


@pytest.mark.parametrize("case", CASCADE, ids=[c[0] for c in CASCADE])
def test_block_size_cascade(case):
    """The shared-prefix decode over longer blocks (prefixes of whole
    blocks), against the plain decode definition."""
    name, bs, ctx, groups, fp8 = case
    b = W.small_case(760 + CASCADE.index(case), "bf16", 28, 4, 128, context_lens=ctx,
                     query_lens=[1] * len(ctx), num_prefill=0, block_size=bs, keep_logical=False,
                     **(_FP8 if fp8 else {}))
    W.with_prefix_groups(b, groups)
    say(f"{name}: {len(groups)} groups")
    cascade_check(b, name)
