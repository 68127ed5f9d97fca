"""GPU parity with an FP8 (E4M3FN) KV cache, through the *_fp8 C entry points,
against the float64 oracle reading the same codes.

The cache codes are compared exactly (one rounding of the same float64 value
on both sides); the attention outputs to the bf16 tolerance (the arithmetic
differs only in accumulation order and the bf16 probabilities).  Scales are
not powers of two, so a missing or swapped scale shows up.
"""
import numpy as np
import pytest

from paged_gqa_attention_neox_amd import runner
from paged_gqa_attention_neox_amd import workloads as W
from gpu_common import (check_caches, check_out, check_rotated, key_groups, require_gpu, run_gpu,
                        run_oracle, say)

pytestmark = pytest.mark.gpu

KS, VS = W.FP8_K_SCALE, W.FP8_V_SCALE


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def fp8_check(b, label, seqs=None):
    say(f"{label}: GPU step")
    res, _ = run_gpu(b)
    say(f"{label}: oracle")
    ora = run_oracle(b, seqs=seqs)
    check_rotated(res["q_out"], ora["q_out"], b.shape.dtype, "q_out")
    check_caches(b, res, ora)
    rows = None
    if seqs is not None:
        cu = b.cu_seqlens_q
        rows = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in seqs])
    mx, mean = check_out(res["out"], ora["out"], b.shape.dtype, rows=rows)
    say(f"{label}: out max abs {mx:.3e} mean abs {mean:.3e}")


_LENS = [1, 17, 31, 32, 33, 63, 64, 65, 95, 96, 97, 127, 128, 129, 160, 191, 200, 224, 250, 255,
         256, 257, 300, 131]
CASES = [
    # (name, H, Hkv, contexts, query lens, num_prefill)
    ("decode_partition_edges", 28, 4, [1, 15, 16, 17, 511, 512, 513, 1024, 1025, 1600], [1] * 10, 0),
    ("decode_g1", 4, 4, [300, 700, 3], [1] * 3, 0),
    ("decode_g2", 16, 8, [129, 2048, 1], [1] * 3, 0),
    ("decode_g4", 16, 4, [1000, 33], [1] * 2, 0),
    ("decode_g8", 32, 4, [777, 1500], [1] * 2, 0),
    ("prefill_chunks", 14, 2, [100, 700, 48], [37, 300, 48], 3),
    ("mixed", 28, 4, [90, 300, 2000, 1, 513], [90, 44, 1, 1, 1], 2),
    # MFMA prefill over FP8 tiles: the one-key-group layout (many rows, ragged
    # tails, chunks after cached context) and the two-key-group layout (few
    # long rows), over G 1, 3-8; two query heads per KV head (G = 2) always
    # take the one-group layout
    ("prefill_1group_g7", 28, 4, _LENS, _LENS, len(_LENS)),
    ("prefill_1group_g7_chunks", 28, 4, [x + 40 for x in _LENS], _LENS, len(_LENS)),
    ("prefill_1group_g8", 32, 4, _LENS, _LENS, len(_LENS)),
    ("prefill_1group_g3", 12, 4, _LENS, _LENS, len(_LENS)),
    ("prefill_1group_g5", 20, 4, _LENS, _LENS, len(_LENS)),
    ("prefill_1group_g6", 24, 4, _LENS, _LENS, len(_LENS)),
    ("prefill_2group_g3", 12, 4, [700, 45], [300, 45], 2),
    ("prefill_2group_g4", 16, 4, [900, 77], [333, 77], 2),
    ("prefill_2group_g5", 20, 4, [640, 1], [640, 1], 2),
    ("prefill_2group_g6", 24, 4, [1000, 200], [256, 200], 2),
    ("prefill_2group_g1", 4, 4, [300, 40], [300, 40], 2),
    ("prefill_g2_long", 16, 8, [500, 33], [200, 33], 2),
    ("prefill_2group_g7_long", 28, 4, [1537, 700], [512, 100], 2),
    ("prefill_2group_g8", 32, 4, [1200, 30], [64, 30], 2),
    # the second key group's only tile wholly past some rows (20-token prefix)
    ("prefill_2group_g7_short_prefix", 28, 4, [2000, 56], [40, 36], 2),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fp8_small_cases(case):
    name, H, Hkv, ctx, ql, npf = case
    if "1group" in name:
        assert key_groups(ctx, ql, Hkv, H) == 1, name
    if "2group" in name:
        assert key_groups(ctx, ql, Hkv, H) == 2, name
    b = W.small_case(401 + CASES.index(case), "bf16", H, Hkv, 128, context_lens=ctx,
                     query_lens=ql, num_prefill=npf, keep_logical=False, cache_dtype="fp8",
                     k_scale=KS, v_scale=VS)
    fp8_check(b, f"fp8_{name}")


def test_fp8_prefix_sharing():
    b = W.small_case(420, "bf16", 14, 2, 128, context_lens=[96, 200, 65, 300],
                     query_lens=[32, 1, 1, 1], num_prefill=1,
                     shares_prefix=[True, True, True, False], shared_prefix_len=64,
                     keep_logical=False, cache_dtype="fp8", k_scale=KS, v_scale=VS)
    fp8_check(b, "fp8_prefix_sharing")


def test_fp8_long_decode_full():
    """The Qwen2-7B long-context decode with an FP8 cache at full size, every
    sequence against the oracle."""
    fp8_check(W.qwen2_long_decode_fp8(), "fp8_long_decode")


def test_fp8_halves_decode_bytes_and_tracks_bf16():
    """Same draws with a bf16 cache and an FP8 cache: the FP8 outputs stay
    within the quantisation error of the bf16 ones (a property, not parity:
    E4M3FN keeps 3 mantissa bits)."""
    bb = W.small_case(430, "bf16", 28, 4, 128, context_lens=[900, 2000, 33], query_lens=[1] * 3,
                      num_prefill=0, keep_logical=False)
    b8 = W.small_case(430, "bf16", 28, 4, 128, context_lens=[900, 2000, 33], query_lens=[1] * 3,
                      num_prefill=0, keep_logical=False, cache_dtype="fp8", k_scale=KS,
                      v_scale=VS)
    assert b8.decode_kv_bytes() * 2 == bb.decode_kv_bytes()
    rb, _ = run_gpu(bb)
    r8, _ = run_gpu(b8)
    ob = runner.to_host(runner.to_device(rb["out"], "bf16")).astype(np.uint32) << 16
    o8 = runner.to_host(runner.to_device(r8["out"], "bf16")).astype(np.uint32) << 16
    fb, f8 = ob.view(np.float32), o8.view(np.float32)
    assert np.all(np.isfinite(f8))
    assert np.abs(fb - f8).mean() < 0.05 * np.abs(fb).mean() + 1e-3


def test_fp8_qwen2_prefill_full():
    """The Qwen2-7B prefill batch (8 sequences of 128..512 tokens) over an FP8
    cache, every output row against the oracle."""
    fp8_check(W.qwen2_prefill_fp8(), "fp8_qwen2_prefill")
