"""The synthetic workloads use the shapes the pages print (tests/golden/page_constants.json)."""
import json
import math
import os

import numpy as np

from paged_gqa_attention_neox_amd import workloads as W

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")))


def _tp_share(total_heads, total_kv, tp):
    # the head split rule printed on the page, restated
    heads = total_heads // tp
    kv = total_kv // tp if total_kv >= tp else max(1, total_kv // tp)
    return heads, kv


def test_qwen2_shapes_from_page():
    g = GOLD["qwen2_7b"]
    head_dim = g["hidden_size"] // g["num_attention_heads"]
    assert head_dim == 128
    for b in (W.qwen2_prefill(), ):
        sh = b.shape
        assert (sh.num_heads, sh.num_kv_heads, sh.head_dim) == (28, 4, head_dim)
        assert sh.group == 7
        assert sh.rope_theta == g["rope_theta"] and sh.max_position == g["max_position_embeddings"]
        assert abs(sh.scale - 1 / math.sqrt(128)) < 1e-18
        assert sh.block_size == GOLD["cache"]["block_size_tokens"]


def test_tp2_share_shape():
    g = GOLD["qwen2_7b"]
    heads, kv = _tp_share(g["num_attention_heads"], g["num_key_value_heads"], 2)
    b = W.mixed_tp2()
    assert (b.shape.num_heads, b.shape.num_kv_heads) == (heads, kv) == (14, 2)
    # TP=8 replicates KV heads (each GPU gets one)
    assert _tp_share(28, 4, 8)[1] == 1


def test_qwen3_shape():
    g = GOLD["qwen3_0_6b"]
    b = W.qwen3_decode()
    assert (b.shape.num_heads, b.shape.num_kv_heads, b.shape.head_dim) == (
        g["num_attention_heads"], g["num_key_value_heads"], g["head_dim"])


def test_workload_structure():
    b = W.qwen2_prefill()
    assert b.num_seqs == 8 and np.all((b.query_lens >= 128) & (b.query_lens <= 512))
    assert np.array_equal(b.query_lens, b.context_lens)
    m = W.mixed_tp2()
    assert m.num_prefill == 4 and m.num_decode == 96
    assert np.all(m.query_lens[:4] == 512)
    dec = m.context_lens[4:]
    assert dec.min() >= 256 and dec.max() <= 8192
    shared = m.block_tables[:, 0] == m.block_tables[0, 0]
    assert shared.sum() == 2 + 48
    # shared prefix: 64 identical block ids in every sharing row
    assert np.all(m.block_tables[shared, :64] == m.block_tables[0, :64])
    # decode slots land in private blocks (position >= 1024)
    assert np.all(m.positions[2048:][shared[4:]] >= 1024)
    steps = W.tiny_f32_steps()
    assert [int(s.positions[0]) for s in steps] == [0, 16, 17, 18, 19]
    assert not (steps[0].block_tables[0, 0] == 0 and steps[4].block_tables[0, 1] == 1)


def test_poison_and_nan_tails():
    b = W.qwen3_decode()
    assert np.all(b.k_cache[b.poison_block] == W.BF16_NAN_BITS)
    # the slot of every new token is still NaN before the step (written by the step)
    blk, off = np.divmod(b.slot_mapping, 16)
    assert np.all(b.k_cache[blk, :, off, :] == W.BF16_NAN_BITS)
    # block-table padding points at the poison block
    nblk = (b.context_lens + 15) // 16
    for s in range(b.num_seqs):
        assert np.all(b.block_tables[s, nblk[s]:] == b.poison_block)
    # the ids in use are distinct across sequences (no sharing in this workload)
    used = np.concatenate([b.block_tables[s, :nblk[s]] for s in range(b.num_seqs)])
    assert len(np.unique(used)) == len(used)


def test_runner_cascade_auto_follows_the_library_rule(monkeypatch):
    """cascade="auto" asks qwen2_attn_decode_cascade_worthwhile with the
    batch's groups (host side only: the query is replaced here)."""
    from paged_gqa_attention_neox_amd import binding as B
    from paged_gqa_attention_neox_amd import runner
    seen = []

    def fake(n_pre, n_mem, max_len, hkv, d, fp8):
        seen.append((n_pre, n_mem, max_len, hkv, d, fp8))
        return len(seen) > 1

    monkeypatch.setattr(B, "qwen2_attn_decode_cascade_worthwhile", fake)
    b = W.mixed_tp2()
    ind, seqs, lens = b.prefix_groups
    assert runner.use_cascade(b, "auto") is False
    assert seen == [(len(lens), len(seqs), int(max(lens)), 2, 128, False)]
    assert runner.use_cascade(b, "auto") is True
    assert runner.use_cascade(b, True) is True and runner.use_cascade(b, False) is False
    assert len(seen) == 2
    plain = W.qwen2_prefill()
    assert runner.use_cascade(plain, "auto") is False and runner.use_cascade(plain, True) is False
