"""GPU parity of the Qwen3 q/k RMSNorm fused into the cache write
(qwen3_rope_cache_write and its FP8 twin, through the C ABI) against the
float64 oracle, which normalises every q and k head before the rotation.

The normalised, rotated q and k are rounded once on both sides, so they are
compared like the plain rotation (bit for bit up to last-place float64
differences); the attention outputs to the step dtype's tolerance.  A
property that needs no oracle closes the file: with eps = 0 the norm removes
any positive per-head scale, so q and k inputs multiplied by 4 (exact in
float32) give bitwise the same step.
"""
import copy

import numpy as np
import pytest

from paged_gqa_attention_neox_amd import workloads as W
from gpu_common import bits, check_caches, check_out, check_rotated, require_gpu, run_gpu, run_oracle, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def qkn_check(b, label, seqs=None):
    assert b.q_norm_weight is not None
    say(f"{label}: GPU step")
    res, _ = run_gpu(b)
    say(f"{label}: oracle")
    ora = run_oracle(b, seqs=seqs)
    dt = b.shape.dtype
    check_rotated(res["q_out"], ora["q_out"], dt, "q_out")
    check_caches(b, res, ora)
    rows = None
    if seqs is not None:
        cu = b.cu_seqlens_q
        rows = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in seqs])
    mx, mean = check_out(res["out"], ora["out"], dt, rows=rows)
    say(f"{label}: out max abs {mx:.3e} mean abs {mean:.3e}")
    return res


def test_qwen3_decode_qknorm_full():
    """The Qwen3-0.6B decode (batch 32, contexts 128-2048) with q/k norm."""
    qkn_check(W.qwen3_decode_qknorm(), "qwen3_decode_qknorm")


CASES = [
    # (name, dtype, H, Hkv, d, contexts, query lens, num_prefill, cache dtype)
    ("decode_g2", "bf16", 16, 8, 128, [129, 2048, 1, 700], [1] * 4, 0, None),
    ("prefill_chunks_g7", "bf16", 14, 2, 128, [100, 700, 48], [37, 300, 48], 3, None),
    ("mixed_d64", "bf16", 8, 2, 64, [90, 300, 17, 1], [90, 1, 1, 1], 1, None),
    ("f32_d64", "f32", 4, 2, 64, [40, 7, 300], [3, 1, 1], 1, None),
    ("f32_d128", "f32", 8, 4, 128, [200, 33, 1000], [64, 1, 1], 1, None),
    ("fp8_mixed", "bf16", 28, 4, 128, [90, 300, 2000, 1, 513], [90, 44, 1, 1, 1], 2, "fp8"),
    ("fp8_decode_g8", "bf16", 32, 4, 128, [777, 1500], [1, 1], 0, "fp8"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_qknorm_small_cases(case):
    name, dt, H, Hkv, d, ctx, ql, npf, cdt = case
    fp8 = {} if cdt is None else dict(cache_dtype=cdt, k_scale=W.FP8_K_SCALE,
                                      v_scale=W.FP8_V_SCALE)
    b = W.small_case(501 + CASES.index(case), dt, H, Hkv, d, context_lens=ctx, query_lens=ql,
                     num_prefill=npf, keep_logical=False, qk_norm=True, **fp8)
    qkn_check(b, f"qknorm_{name}")


def test_qknorm_differs_from_plain_rotation():
    """The norm is applied: the same batch without weights stores other q/k."""
    b = W.small_case(530, "bf16", 8, 2, 128, context_lens=[64, 300], query_lens=[64, 1],
                     num_prefill=1, keep_logical=False, qk_norm=True)
    plain = copy.copy(b)
    plain.q_norm_weight = plain.k_norm_weight = None
    rn, _ = run_gpu(b)
    rp, _ = run_gpu(plain)
    assert np.mean(bits(rn["q_out"]) != bits(rp["q_out"])) > 0.9
    # v is not normalised: the V cache is identical
    assert np.array_equal(bits(rn["v_cache"]), bits(rp["v_cache"]))


def test_qknorm_scale_invariance_bitwise():
    """eps = 0: q and k heads scaled by 4 (exact in float32) normalise to the
    same vectors, so q_out, both caches and the attention output agree bit
    for bit.  Needs no oracle."""
    b = W.small_case(540, "f32", 8, 2, 128, context_lens=[80, 500, 19], query_lens=[80, 1, 1],
                     num_prefill=1, keep_logical=False, qk_norm=True)
    b.shape = copy.copy(b.shape)
    b.shape.rms_eps = 0.0
    s = copy.copy(b)
    qk = (b.shape.num_heads + b.shape.num_kv_heads) * b.shape.head_dim
    s.qkv = b.qkv.copy()
    s.qkv[:, :qk] *= np.float32(4.0)
    r1, _ = run_gpu(b)
    r4, _ = run_gpu(s)
    for key in ("q_out", "k_cache", "v_cache", "out"):
        assert np.array_equal(bits(r1[key]), bits(r4[key])), key
