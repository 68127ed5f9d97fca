"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Full-size workloads (the five configurations), small cases spanning several
tiles with ragged tails, and the bitwise properties: V copied bit for bit,
unwritten slots untouched, K at position 0 unrotated, a single visible key
returning its V row, a dominant needle key returning its V row, results
independent of the physical block placement, and run-to-run determinism.
"""
import numpy as np
import pytest
import torch

import oracle.reference as R
from paged_gqa_attention_neox_amd import runner
from paged_gqa_attention_neox_amd import workloads as W
from gpu_common import (bits, check_caches, check_out, check_rotated, full_check, key_groups,
                        require_gpu, run_gpu, run_oracle, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


# ---------------------------------------------------------------------------
# the five configurations
# ---------------------------------------------------------------------------
def test_tiny_f32_prefill_then_decode():
    """16-token fp32 prefill then 4 decode steps (cache threaded through)."""
    steps = W.tiny_f32_steps()
    kc = vc = None
    okc, ovc = steps[0].k_cache, steps[0].v_cache
    for i, st in enumerate(steps):
        say(f"tiny_f32 step {i}")
        dev = runner.DeviceStep(st, k_cache=kc, v_cache=vc)
        dev.step()
        res = dev.results()
        kc, vc = dev.k_cache, dev.v_cache
        q_out, okc, ovc = R.rope_cache_write(st.qkv, "f32", st.positions, st.slot_mapping, okc, ovc,
                                             4, 2, 64, 16, 1e6)
        out = R.attention_varlen(q_out, okc, ovc, st.cu_seqlens_q, st.context_lens, st.block_tables,
                                 4, 2, 64, 16, "f32")
        check_rotated(res["q_out"], q_out, "f32", f"q_out step {i}")
        assert np.array_equal(bits(res["v_cache"]), bits(ovc))
        check_rotated(res["k_cache"][np.isfinite(okc)], okc[np.isfinite(okc)], "f32", "K cache")
        assert np.array_equal(np.isnan(res["k_cache"]), np.isnan(okc))
        check_out(res["out"], out, "f32")


def test_qwen3_decode_full():
    full_check(W.qwen3_decode())


def test_qwen2_prefill_full():
    full_check(W.qwen2_prefill())


def test_qwen2_prefill_long_prefix_sampled():
    """The bench's long-key-loop prefill (8 chunks of 256 rows after 8192-token
    prefixes), in its bench launch; the oracle attention on two chunks."""
    full_check(W.qwen2_prefill_long_prefix(), seqs=[0, 7])


def test_qwen2_long_decode_full():
    """The Qwen2-7B long-context decode (batch 64, contexts 2K-32K), every
    sequence and head against the oracle."""
    full_check(W.qwen2_long_decode(), label="qwen2_long_decode")


def test_mixed_tp2_full():
    full_check(W.mixed_tp2())


# ---------------------------------------------------------------------------
# small cases: tiles, ragged tails, partitions, groups, head dims
# ---------------------------------------------------------------------------
SMALL = [
    # (name, dtype, H, Hkv, d, contexts, query lens, num_prefill)
    ("decode_partition_edges", "bf16", 28, 4, 128, [1, 15, 16, 17, 511, 512, 513, 1024, 1025, 1600],
     [1] * 10, 0),
    ("decode_g1", "bf16", 4, 4, 128, [300, 700, 3], [1] * 3, 0),
    ("decode_g2", "bf16", 16, 8, 128, [129, 2048, 1], [1] * 3, 0),
    ("decode_g4", "bf16", 16, 4, 128, [1000, 33], [1] * 2, 0),
    ("decode_g8", "bf16", 32, 4, 128, [777, 1500], [1] * 2, 0),
    # one 32k-token sequence on one KV head: its segment is cut into more
    # than 128 pieces, so their merge runs in several chunks
    ("decode_one_long_segment", "bf16", 8, 1, 128, [32768], [1], 0),
    # many short sequences: most ranges hold several whole segments
    ("decode_many_short", "bf16", 28, 4, 128, list(range(1, 400, 7)), [1] * 57, 0),
    ("decode_g16_generic", "bf16", 32, 2, 128, [600, 40], [1] * 2, 0),
    ("decode_d64_generic", "bf16", 8, 2, 64, [70, 530], [1] * 2, 0),
    ("decode_f32", "f32", 8, 2, 128, [70, 530], [1] * 2, 0),
    ("prefill_ragged", "bf16", 28, 4, 128, [1, 17, 64, 65, 130, 200], [1, 17, 64, 65, 130, 200], 6),
    ("prefill_chunks", "bf16", 14, 2, 128, [100, 700, 48], [37, 300, 48], 3),
    ("prefill_f32_d64", "f32", 4, 2, 64, [33, 20], [33, 7], 2),
    ("mixed_small", "bf16", 28, 4, 128, [90, 300, 2000, 1, 513], [90, 44, 1, 1, 1], 2),
    ("prefill_g1", "bf16", 4, 4, 128, [33, 95, 1], [33, 95, 1], 3),
    ("prefill_g2_chunk", "bf16", 16, 8, 128, [160, 77], [31, 77], 2),
    ("prefill_g4", "bf16", 16, 4, 128, [64, 129], [64, 129], 2),
    ("prefill_g8_chunk", "bf16", 32, 4, 128, [1000, 40], [65, 40], 2),
    ("prefill_long_chunk", "bf16", 28, 4, 128, [2100], [100], 1),
    ("prefill_d64_generic", "bf16", 8, 2, 64, [50, 20], [50, 5], 2),
    # a thousand decode rows of short contexts: many ranges, most holding
    # several whole segments
    ("decode_1000_short", "bf16", 28, 4, 128, [1 + (37 * i) % 300 for i in range(1000)],
     [1] * 1000, 0),
    # 160 tiny prefill sequences (1..40 tokens): 640 (sequence, KV head) pairs
    ("prefill_160_tiny", "bf16", 28, 4, 128, list(range(1, 41)) * 4, list(range(1, 41)) * 4, 160),
    # the plain decode's range count for bf16 switches at 65536 units
    # ((sequence, KV head, block) triples): exactly 65536 takes one range per
    # CU, one unit less two per CU (512 ranges, the cap)
    ("decode_256_ranges_at_threshold", "bf16", 28, 4, 128, [16384] * 16, [1] * 16, 0),
    ("decode_512_ranges_below_threshold", "bf16", 28, 4, 128, [16384] * 15 + [16368], [1] * 16,
     0),
    # 32768 units: 512 ranges of 64 units
    ("decode_32k_units", "bf16", 28, 4, 128, [16384] * 8, [1] * 8, 0),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_cases(case):
    name, dt, H, Hkv, d, ctx, ql, npf = case
    b = W.small_case(101 + SMALL.index(case), dt, H, Hkv, d, context_lens=ctx, query_lens=ql,
                     num_prefill=npf, keep_logical=False)
    full_check(b, label=name)


# many sequences: the one-key-group layout (32-row tiles, one wave per head)
_LENS = [1, 17, 31, 32, 33, 63, 64, 65, 95, 96, 97, 127, 128, 129, 160, 191, 200, 224, 250, 255,
         256, 257, 300, 131]
ONE_GROUP = [
    ("prefill_1group_g7", 28, 4, _LENS, _LENS),
    ("prefill_1group_g7_chunks", 28, 4, [x + 40 for x in _LENS], _LENS),
    ("prefill_1group_g1", 8, 8, _LENS[:20], _LENS[:20]),
    ("prefill_1group_g2", 16, 8, _LENS[:20], _LENS[:20]),
    ("prefill_1group_g3", 12, 4, _LENS, _LENS),
    ("prefill_1group_g4", 16, 4, _LENS, _LENS),
    ("prefill_1group_g5", 20, 4, _LENS, _LENS),
    ("prefill_1group_g6", 24, 4, _LENS, _LENS),
    ("prefill_1group_g8", 32, 4, _LENS, _LENS),
    # two query heads per KV head: one group even for few long rows
    ("prefill_1group_g2_long", 16, 8, [500, 33], [200, 33]),
    ("prefill_1group_g2_4000", 8, 4, [4000, 300], [64, 300]),
]


@pytest.mark.parametrize("case", ONE_GROUP, ids=[c[0] for c in ONE_GROUP])
def test_prefill_one_key_group(case):
    name, H, Hkv, ctx, ql = case
    assert key_groups(ctx, ql, Hkv, H) == 1, name
    b = W.small_case(170 + ONE_GROUP.index(case), "bf16", H, Hkv, 128, context_lens=ctx,
                     query_lens=ql, num_prefill=len(ql), keep_logical=False)
    full_check(b, label=name)


TWO_GROUP = [
    # (name, H, Hkv, contexts, query lens): few long rows, the two-key-group layout
    ("prefill_2group_g1", 4, 4, [300, 40], [300, 40]),
    ("prefill_2group_g5", 20, 4, [640, 1], [640, 1]),
    ("prefill_2group_g7_long", 28, 4, [1537, 700], [512, 100]),
    # a 20-token prefix: the first 16-row tile (positions 20..35) has two
    # 32-key tiles, and the second key group's only tile (keys 32..63) lies
    # wholly past its rows 20..31; those columns must come out of the merge
    # with the first group's keys alone
    ("prefill_2group_g7_short_prefix", 28, 4, [2000, 56], [40, 36]),
    # even groups over several waves (no padding column) and odd G = 3
    ("prefill_2group_g3", 12, 4, [700, 45], [300, 45]),
    ("prefill_2group_g4", 16, 4, [900, 77], [333, 77]),
    ("prefill_2group_g6", 24, 4, [1000, 200], [256, 200]),
    ("prefill_2group_g8", 32, 4, [1200, 30], [64, 30]),
    ("prefill_2group_g8_chunks", 32, 4, [800, 100, 57], [400, 100, 57]),
]


@pytest.mark.parametrize("case", TWO_GROUP, ids=[c[0] for c in TWO_GROUP])
def test_prefill_two_key_groups(case):
    name, H, Hkv, ctx, ql = case
    assert key_groups(ctx, ql, Hkv, H) == 2, name
    b = W.small_case(190 + TWO_GROUP.index(case), "bf16", H, Hkv, 128, context_lens=ctx,
                     query_lens=ql, num_prefill=len(ql), keep_logical=False)
    full_check(b, label=name)


def test_prefix_sharing_small():
    b = W.small_case(150, "bf16", 14, 2, 128, context_lens=[96, 200, 64 + 1, 300],
                     query_lens=[32, 1, 1, 1], num_prefill=1,
                     shares_prefix=[True, True, True, False], shared_prefix_len=64,
                     keep_logical=False)
    full_check(b, label="prefix_sharing_small")


# ---------------------------------------------------------------------------
# bitwise properties
# ---------------------------------------------------------------------------
def test_position_zero_k_unrotated_and_slot_skip():
    b = W.small_case(160, "bf16", 28, 4, 128, context_lens=[40, 9], query_lens=[40, 9],
                     num_prefill=2, keep_logical=False)
    b.positions = np.zeros_like(b.positions)
    b.slot_mapping = b.slot_mapping.copy()
    b.slot_mapping[5] = -1
    say("position-zero rope write")
    dev = runner.DeviceStep(b)
    dev.rope_write()
    res = dev.results()
    heads = b.qkv.reshape(b.num_tokens, 36, 128)
    assert np.array_equal(res["q_out"], heads[:, :28])
    for t, sl in enumerate(b.slot_mapping):
        blk, off = divmod(int(sl), 16)
        if sl < 0:
            continue
        assert np.array_equal(res["k_cache"][blk, :, off, :], heads[t, 28:32])
        assert np.array_equal(res["v_cache"][blk, :, :, off], heads[t, 32:36])
    blk, off = divmod(int(b.block_tables[0, 5 // 16]) * 16 + 5 % 16, 16)
    assert np.all(res["k_cache"][blk, :, off, :] == W.BF16_NAN_BITS)
    assert np.all(res["v_cache"][blk, :, :, off] == W.BF16_NAN_BITS)


def test_single_key_returns_v_bitwise():
    b = W.small_case(161, "bf16", 28, 4, 128, context_lens=[1, 1, 1], query_lens=[1, 1, 1],
                     num_prefill=0, keep_logical=False)
    res, _ = run_gpu(b)
    heads = b.qkv.reshape(3, 36, 128)
    for t in range(3):
        for h in range(28):
            assert np.array_equal(res["out"][t, h], heads[t, 32 + h // 7])
    b2 = W.small_case(162, "bf16", 28, 4, 128, context_lens=[1, 5], query_lens=[1, 5],
                      num_prefill=2, keep_logical=False)
    res2, _ = run_gpu(b2)
    heads2 = b2.qkv.reshape(6, 36, 128)
    for t in (0, 1):          # first row of each sequence sees only itself
        for h in range(28):
            assert np.array_equal(res2["out"][t, h], heads2[t, 32 + h // 7])


def _needle_batch(seed, ctx):
    return W.small_case(seed, "bf16", 28, 4, 128, context_lens=[ctx], query_lens=[1], num_prefill=0,
                        keep_logical=False)


@pytest.mark.parametrize("ctx,needle", [(40, 7), (1500, 1234), (3000, 10)])
def test_needle_bitwise(ctx, needle):
    """A cached key equal to 32x the rotated query of head 7g dominates every
    other score by >100 natural-log units: fp32 exp underflows to exactly 0,
    so head 7g's output is that key's V row, bit for bit, across partitions."""
    b = _needle_batch(170 + ctx, ctx)
    say(f"needle ctx={ctx}: rope write")
    dev = runner.DeviceStep(b)
    dev.rope_write()
    q_rot = runner.to_host(dev.q_out)[0]                    # [28][128] bf16 bits
    kc = runner.to_host(dev.k_cache)
    blk, off = divmod(int(b.block_tables[0, needle // 16]) * 16 + needle % 16, 16)
    for g in range(4):
        qv = W.bf16_bits_to_f32(q_rot[7 * g]) * np.float32(32.0)
        kc[blk, g, off, :] = W.f32_to_bf16_bits(qv)
    dev.k_cache.copy_(runner.to_device(kc, "bf16"))
    say(f"needle ctx={ctx}: decode")
    dev.decode()
    res = dev.results()
    for g in range(4):
        assert np.array_equal(res["out"][0, 7 * g], res["v_cache"][blk, g, :, off]), g


def test_block_permutation_invariance_bitwise():
    """Same logical cache content under a different physical placement gives
    bit-identical outputs (decode with split partitions, and prefill)."""
    b = W.small_case(180, "bf16", 28, 4, 128, context_lens=[1300, 40, 700],
                     query_lens=[64, 1, 1], num_prefill=1, keep_logical=False)
    res1, _ = run_gpu(b)
    rng = np.random.default_rng(5)
    perm = rng.permutation(b.num_blocks)          # new id of each old block
    b2 = W.small_case(180, "bf16", 28, 4, 128, context_lens=[1300, 40, 700],
                      query_lens=[64, 1, 1], num_prefill=1, keep_logical=False)
    kc2 = np.empty_like(b.k_cache)
    vc2 = np.empty_like(b.v_cache)
    kc2[perm] = b.k_cache
    vc2[perm] = b.v_cache
    b2.k_cache, b2.v_cache = kc2, vc2
    b2.block_tables = perm[b.block_tables].astype(np.int32)
    blk, off = np.divmod(b.slot_mapping, 16)
    b2.slot_mapping = (perm[blk] * 16 + off).astype(np.int32)
    res2, _ = run_gpu(b2)
    assert np.array_equal(res1["out"], res2["out"])
    assert np.array_equal(res1["q_out"], res2["q_out"])


def test_run_to_run_deterministic():
    b = W.small_case(190, "bf16", 28, 4, 128, context_lens=[200, 3000, 513],
                     query_lens=[200, 1, 1], num_prefill=1, keep_logical=False)
    outs = []
    for i in range(3):
        say(f"determinism run {i}")
        res, _ = run_gpu(b)
        outs.append(res["out"])
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_causal_future_does_not_leak_bitwise():
    b = W.small_case(200, "bf16", 28, 4, 128, context_lens=[300], query_lens=[300], num_prefill=1,
                     keep_logical=False)
    say("causal: base")
    dev = runner.DeviceStep(b)
    dev.step()
    base = dev.results()["out"]
    # overwrite keys/values of positions > 150 after the write, rerun attention only
    kc = runner.to_host(dev.k_cache)
    vc = runner.to_host(dev.v_cache)
    for p in range(151, 300):
        blk, off = divmod(int(b.slot_mapping[p]), 16)
        kc[blk, :, off, :] = W.f32_to_bf16_bits(np.full((4, 128), 3.0, np.float32))
        vc[blk, :, :, off] = W.f32_to_bf16_bits(np.full((4, 128), -7.0, np.float32))
    dev.k_cache.copy_(runner.to_device(kc, "bf16"))
    dev.v_cache.copy_(runner.to_device(vc, "bf16"))
    say("causal: perturbed")
    dev.prefill()
    pert = dev.results()["out"]
    assert np.array_equal(pert[:151], base[:151])
    assert not np.array_equal(pert[151:], base[151:])


def test_in_place_q_out_matches():
    b = W.small_case(210, "bf16", 28, 4, 128, context_lens=[50, 700], query_lens=[50, 1],
                     num_prefill=1, keep_logical=False)
    res, dev = run_gpu(b)
    dev2 = runner.DeviceStep(b)
    dev2.q_out = dev2.q.view(b.num_tokens, 28, 128)         # rotate in place inside the fused rows
    from paged_gqa_attention_neox_amd import binding as B
    sh = b.shape
    B.qwen2_rope_cache_write(dev2.q, dev2.q, dev2.k, dev2.v, dev2.positions, dev2.slots, dev2.cos_sin,
                             dev2.k_cache, dev2.v_cache, 28, 4, 128, 16)
    dev2.prefill()
    dev2.decode()
    torch.cuda.synchronize()
    assert np.array_equal(runner.to_host(dev2.q_out), res["q_out"])
    assert np.array_equal(runner.to_host(dev2.out), res["out"])
    del sh


def test_tiny_prefill20_equals_prefill16_plus_decodes():
    steps = W.tiny_f32_steps()
    kc = vc = None
    outs = []
    for st in steps:
        dev = runner.DeviceStep(st, k_cache=kc, v_cache=vc)
        dev.step()
        outs.append(dev.results()["out"])
        kc, vc = dev.k_cache, dev.v_cache
    seq = np.concatenate(outs)
    full = W.Batch(name="tiny20", shape=steps[0].shape,
                   qkv=np.concatenate([s.qkv for s in steps]), positions=np.arange(20, dtype=np.int32),
                   slot_mapping=np.concatenate([s.slot_mapping for s in steps]),
                   k_cache=steps[0].k_cache, v_cache=steps[0].v_cache,
                   block_tables=steps[-1].block_tables, context_lens=np.array([20], np.int32),
                   query_lens=np.array([20], np.int32), num_prefill=1,
                   poison_block=steps[0].poison_block)
    res, _ = run_gpu(full)
    assert np.abs(res["out"] - seq).max() <= 1e-5
