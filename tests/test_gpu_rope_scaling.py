"""GPU parity with dynamic-NTK rope scaling: the scaled table
(qwen2_rope_table_init_dynamic_ntk) against the oracle's base and float64
cos/sin, and whole steps at positions past the native 32768 window (the
rotation and attention kernels read the longer table as usual).
"""
import numpy as np
import pytest
import torch

import oracle.reference as R
from paged_gqa_attention_neox_amd import binding as B
from paged_gqa_attention_neox_amd import runner
from paged_gqa_attention_neox_amd import workloads as W
from gpu_common import check_caches, check_out, check_rotated, require_gpu, run_gpu, run_oracle, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("factor,original,d", [(2.0, 4096, 128), (4.0, 32768, 128), (3.0, 1000, 64)])
def test_scaled_table_matches_oracle(factor, original, d):
    """The scaled table is the plain table built with the oracle's scaled base,
    bit for bit (both sides form the base with the C library's pow in
    float64), and its entries are cos and sin of p times the oracle's
    frequencies within 16 float64 ulps of the angle plus 2 of the result
    (device and host pow/sincos round differently; one ulp of an angle of
    8e3 rad is 1.8e-12)."""
    n = B.qwen2_rope_dynamic_ntk_positions(original, factor)
    t = torch.empty(n, d, dtype=torch.float64, device="cuda")
    B.qwen2_rope_table_init_dynamic_ntk(t, original, factor, 1e6)
    base, rows = R.rope_dynamic_ntk(1e6, d, factor, original)
    assert rows == n
    t_base = torch.empty(n, d, dtype=torch.float64, device="cuda")
    B.qwen2_rope_table_init(t_base, base)
    assert torch.equal(t, t_base)
    got = t.cpu().numpy()
    a = np.arange(n, dtype=np.float64)[:, None] * R.rope_inv_freq(d, base)[None, :]
    ref = np.concatenate([np.cos(a), np.sin(a)], axis=1)
    err = np.abs(got - ref)
    lim = 16.0 * np.spacing(np.concatenate([a, a], axis=1)) + 2.0 * np.spacing(np.abs(ref))
    assert np.all(err <= lim), float((err / lim).max())
    # the plain table over the same rows differs (the base moved)
    t0 = torch.empty(n, d, dtype=torch.float64, device="cuda")
    B.qwen2_rope_table_init(t0, 1e6)
    assert not torch.equal(t0, t)


CASES = [
    # (name, H, Hkv, contexts, query lens, num_prefill, (factor, original))
    ("decode_past_32k", 8, 2, [40000, 70001, 33000, 131072], [1] * 4, 0, (4.0, 32768)),
    ("prefill_chunk_past_32k", 8, 2, [36000, 40], [48, 40], 2, (4.0, 32768)),
    ("p2_setting_factor2_4096", 28, 4, [5000, 300, 8192], [64, 300, 1], 2, (2.0, 4096)),
    # Qwen2-7B heads: a chunk after a 40K-token prefix (two key groups, 2500
    # block ids staged), and one after a 130K-token prefix (8126 ids leave the
    # two-group layout no LDS room: the one-group layout takes it)
    ("prefill_chunk_40k_g7", 28, 4, [40000, 300], [64, 300], 2, (2.0, 32768)),
    ("prefill_chunk_130k_g7", 28, 4, [130000, 64], [32, 64], 2, (4.0, 32768)),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_scaled_rope_steps(case):
    name, H, Hkv, ctx, ql, npf, rs = case
    # prefill sequences first, then decodes
    b = W.small_case(601 + CASES.index(case), "bf16", H, Hkv, 128, context_lens=ctx,
                     query_lens=ql, num_prefill=npf, keep_logical=False, rope_scaling=rs)
    assert int(b.positions.max()) >= 4096 and b.shape.max_position == int(rs[0] * rs[1])
    say(f"rope scaling {name}: GPU step")
    res, _ = run_gpu(b)
    say(f"rope scaling {name}: oracle")
    ora = run_oracle(b)
    check_rotated(res["q_out"], ora["q_out"], "bf16", "q_out")
    check_caches(b, res, ora)
    mx, mean = check_out(res["out"], ora["out"], "bf16")
    say(f"rope scaling {name}: out max abs {mx:.3e} mean abs {mean:.3e}")


def test_qwen2_131k_decode_full():
    """Qwen2-7B decode at 65k-131k contexts with the factor-4 table; every
    sequence against the oracle."""
    b = W.qwen2_131k_decode()
    say("qwen2_131k_decode: GPU step")
    res, _ = run_gpu(b)
    say("qwen2_131k_decode: oracle")
    ora = run_oracle(b)
    check_rotated(res["q_out"], ora["q_out"], "bf16", "q_out")
    check_caches(b, res, ora)
    mx, mean = check_out(res["out"], ora["out"], "bf16")
    say(f"qwen2_131k_decode: out max abs {mx:.3e} mean abs {mean:.3e}")
