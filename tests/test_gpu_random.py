"""Seeded random configurations of the whole step against the oracle,
through the C ABI.

Each case draws, from its own seed, a point in the space the hand-written
cases cover one axis at a time: storage dtype (bf16, f32), cache (bf16 or
FP8 E4M3FN), head_dim (64, 128), cache block size (16, 32, 64), KV heads and
group size (1..8 on the matrix-core kernels, 10 on the generic one), the
Qwen3 q/k norm, a mix of prefill chunks (with and without a prefix already in
the cache) and decodes with log-uniform contexts, and for some batches a
shared-prefix group decoded through the cascade entry point.  The checks are
those of the fixed cases: q_out and the caches against the oracle (bitwise,
K within the rotation bound), outputs to the step dtype's tolerance.
"""
import numpy as np
import pytest

from paged_gqa_attention_neox_amd import workloads as W
from gpu_common import full_check, require_gpu, say
from test_gpu_cascade import cascade_check

pytestmark = pytest.mark.gpu

NUM_CASES = 48


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def draw(i: int):
    """Configuration i: (small_case keyword arguments, prefix groups or None)."""
    rng = np.random.default_rng(9100 + i)
    dt = "f32" if rng.random() < 0.25 else "bf16"
    d = 64 if rng.random() < 0.2 else 128
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 3, 4, 5, 6, 7, 8, 10]))
    bs = int(rng.choice([16, 32, 64]))
    fp8 = dt == "bf16" and rng.random() < 0.3
    qkn = rng.random() < 0.2
    nseq = int(rng.integers(1, 9))
    npf = int(rng.integers(0, nseq + 1))
    ql, ctx = [], []
    for s in range(nseq):
        if s < npf:
            n = int(rng.integers(1, 301))
            prefix = 0 if rng.random() < 0.5 else int(rng.integers(1, 701))
            ql.append(n)
            ctx.append(n + prefix)
        else:
            ql.append(1)
            ctx.append(int(np.exp(rng.uniform(0.0, np.log(3000.0)))) or 1)
    kw = dict(context_lens=ctx, query_lens=ql, num_prefill=npf, block_size=bs, qk_norm=qkn)
    if fp8:
        kw.update(cache_dtype="fp8", k_scale=W.FP8_K_SCALE, v_scale=W.FP8_V_SCALE)
    groups = None
    dec = list(range(nseq - npf))
    if len(dec) >= 2 and rng.random() < 0.7:
        members = sorted(int(m) for m in rng.choice(dec, size=int(rng.integers(2, len(dec) + 1)),
                                                    replace=False))
        shortest = min(ctx[npf + m] for m in members)
        if shortest > bs:
            prefix_len = bs * int(rng.integers(1, (shortest - 1) // bs + 1))
            groups = [(members, prefix_len)]
    return dict(dtype=dt, num_heads=g * hkv, num_kv_heads=hkv, head_dim=d, **kw), groups


@pytest.mark.parametrize("i", range(NUM_CASES))
def test_random_config(i):
    kw, groups = draw(i)
    dt, H, Hkv, d = kw.pop("dtype"), kw.pop("num_heads"), kw.pop("num_kv_heads"), kw.pop("head_dim")
    label = (f"random_{i}: {dt} H{H}/{Hkv} d{d} B{kw['block_size']} "
             f"{'fp8 ' if 'cache_dtype' in kw else ''}{'qknorm ' if kw['qk_norm'] else ''}"
             f"ctx {kw['context_lens']} ql {kw['query_lens']} groups {groups}")
    say(label)
    b = W.small_case(9100 + i, dt, H, Hkv, d, keep_logical=False, **kw)
    if groups is None:
        full_check(b, label=f"random_{i}")
    else:
        W.with_prefix_groups(b, groups)
        cascade_check(b, f"random_{i}")
