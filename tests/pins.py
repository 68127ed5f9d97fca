"""Pins for the CPU oracle: checks against facts other than the oracle itself.

Each pin is a function of the oracle module ``R`` (``oracle.reference``) and
raises AssertionError when the oracle disagrees with the fact it checks.
They are run against the real oracle (tests/test_oracle_pins.py) and against
deliberately broken copies of it (tests/test_oracle_mutations.py), which shows
that a plausible mistake in any step is caught by at least one pin.

Kinds of pin used here:
  * textbook values: cos 1, sin 1; powers of ten for the frequency law;
  * closed forms: a unit vector rotates onto its NeoX partner; constant V
    gives a constant output; q = 0 gives the mean of the visible V rows;
    a single visible key returns that key's V row; a dominant "needle" key
    returns its V row;
  * library routines on special cases: torch's fp32->bf16 rounding for
    fp32-representable inputs, torch scaled_dot_product_attention in float64
    for contiguous causal GQA, numpy complex multiplication for the rotation;
  * brute force on tiny inputs (tests/brute.py, separate code, exact
    rational rounding);
  * invariants the pages fix: RoPE preserves norms and makes q.k depend only
    on m - n; GQA equals MHA with each KV head repeated; the paged layout
    equals the contiguous one under any block permutation; softmax rows sum
    to one; causal masking.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from paged_gqa_attention_neox_amd import workloads as W
import brute

COS1 = 0.5403023058681398     # cos(1 rad)
SIN1 = 0.8414709848078965     # sin(1 rad)


# ---------------------------------------------------------------------------
# rounding
# ---------------------------------------------------------------------------
def pin_bf16_rounding_values(R):
    """Hand-checked bf16 encodings, including ties and a value just above a
    tie that a double rounding through fp32 would get wrong."""
    cases = [
        (1.0, 0x3F80), (-2.0, 0xC000), (0.0, 0x0000), (-0.0, 0x8000),
        (1.0 + 2.0**-8, 0x3F80),                 # tie -> even (down)
        (1.0 + 3 * 2.0**-8, 0x3F82),             # tie -> even (up)
        (1.0 + 2.0**-8 + 2.0**-40, 0x3F81),      # just above the tie -> up
        (1.0 + 2.0**-8 - 2.0**-40, 0x3F80),      # just below -> down
        (3.140625, 0x4049), (-0.1, 0xBDCD),
        (2.0**-126, 0x0080), (2.0**-133, 0x0001),  # smallest normal / subnormal
        (3.0e38, 0x7F62), (3.5e38, 0x7F80),        # largest region / overflow
    ]
    for x, want in cases:
        got = int(R.f64_to_bf16_bits(np.array([x]))[0])
        assert got == want, (x, hex(got), hex(want))


def pin_bf16_rounding_matches_torch(R):
    """On fp32-representable inputs one rounding fp32->bf16 is torch's."""
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    bits[::3] = (bits[::3] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)   # exact ties
    exp = (bits >> np.uint32(23)) & np.uint32(0xFF)
    bits = bits[(exp != 0xFF) & (exp < 0xFE)]                             # finite, no overflow
    f = bits.view(np.float32)
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = R.f64_to_bf16_bits(f.astype(np.float64))
    assert np.array_equal(got, want), int(np.sum(got != want))


# ---------------------------------------------------------------------------
# rotary embedding
# ---------------------------------------------------------------------------
def _unit(d, i):
    x = np.zeros((1, 1, d))
    x[0, 0, i] = 1.0
    return x


def pin_rope_unit_vector_neox(R):
    """e_0 at position 1 (f_0 = 1 for any base) -> cos 1 at index 0 and
    sin 1 at index d/2: NeoX half-split pairing, counter-clockwise sign."""
    for d in (64, 128):
        y = R.rope_neox(_unit(d, 0), np.array([1]), 1.0e6)[0, 0]
        want = np.zeros(d)
        want[0], want[d // 2] = COS1, SIN1
        assert np.allclose(y, want, atol=1e-15), (d, y[:3], y[d // 2:d // 2 + 2])
        y = R.rope_neox(_unit(d, d // 2), np.array([1]), 1.0e6)[0, 0]
        want = np.zeros(d)
        want[0], want[d // 2] = -SIN1, COS1
        assert np.allclose(y, want, atol=1e-15)


def pin_rope_frequency_closed_forms(R):
    """f_i = theta^(-2i/d): at i = d/4 the frequency is theta^(-1/2)
    (1e-3 for theta = 1e6, 1e-2 for theta = 1e4), so position 1/f rotates by
    exactly one radian; at i = d/8, theta = 1e6 the frequency is
    10^-1.5 = 1/sqrt(1000)."""
    for d, theta, p in ((128, 1.0e6, 1000), (64, 1.0e6, 1000), (128, 1.0e4, 100)):
        i = d // 4
        y = R.rope_neox(_unit(d, i), np.array([p]), theta)[0, 0]
        assert abs(y[i] - COS1) < 1e-12 and abs(y[i + d // 2] - SIN1) < 1e-12, (d, theta)
    d = 128
    y = R.rope_neox(_unit(d, 16), np.array([1000]), 1.0e6)[0, 0]
    ang = 1000.0 / math.sqrt(1000.0)
    assert abs(y[16] - math.cos(ang)) < 1e-12 and abs(y[16 + 64] - math.sin(ang)) < 1e-12
    f = R.rope_inv_freq(128, 1.0e6)
    assert f.shape == (64,) and f[0] == 1.0 and abs(f[32] - 1e-3) < 1e-18
    r = f[1:] / f[:-1]                                     # geometric progression
    assert np.allclose(r, r[0], rtol=1e-13) and abs(r[0] - 10 ** (-6 / 64)) < 1e-15


def pin_rope_identity_at_zero(R):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 3, 128))
    y = R.rope_neox(x, np.zeros(5, np.int64), 1.0e6)
    assert np.array_equal(y, x)


def pin_rope_norm_preserved(R):
    rng = np.random.default_rng(2)
    x = rng.standard_normal((64, 4, 128))
    p = rng.integers(0, 32768, size=64)
    y = R.rope_neox(x, p, 1.0e6)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)


def pin_rope_relative_position(R):
    """<R_m q, R_n k> depends on m - n only."""
    rng = np.random.default_rng(3)
    for _ in range(20):
        q = rng.standard_normal((1, 1, 128))
        k = rng.standard_normal((1, 1, 128))
        m, n, s = (int(v) for v in rng.integers(0, 16000, size=3))
        a = np.sum(R.rope_neox(q, np.array([m]), 1e6) * R.rope_neox(k, np.array([n]), 1e6))
        b = np.sum(R.rope_neox(q, np.array([m + s]), 1e6) * R.rope_neox(k, np.array([n + s]), 1e6))
        assert abs(a - b) <= 1e-9 * max(1.0, abs(a)), (a, b)


def pin_rope_composition(R):
    rng = np.random.default_rng(4)
    x = rng.standard_normal((8, 2, 64))
    a = rng.integers(0, 10000, size=8)
    b = rng.integers(0, 10000, size=8)
    y1 = R.rope_neox(R.rope_neox(x, a, 1e6), b, 1e6)
    y2 = R.rope_neox(x, a + b, 1e6)
    assert np.allclose(y1, y2, atol=1e-9)


def pin_rope_complex_form(R):
    """Rotation of the pair (x_i, x_{i+d/2}) is multiplication of the complex
    number x_i + i x_{i+d/2} by exp(i p f_i) (numpy complex arithmetic)."""
    rng = np.random.default_rng(5)
    d = 128
    x = rng.standard_normal((16, 3, d))
    p = rng.integers(0, 32768, size=16)
    f = R.rope_inv_freq(d, 1e6)
    z = (x[..., :d // 2] + 1j * x[..., d // 2:]) * np.exp(1j * (p[:, None, None] * f[None, None, :]))
    y = R.rope_neox(x, p, 1e6)
    assert np.allclose(y[..., :d // 2], z.real, atol=1e-12)
    assert np.allclose(y[..., d // 2:], z.imag, atol=1e-12)


# ---------------------------------------------------------------------------
# cache write / gather
# ---------------------------------------------------------------------------
def pin_gather_matches_generator_layout(R):
    """The generator fills the pool block by block (reshape/transpose code of
    its own); the oracle's per-position gather must return its logical rows."""
    for dt in ("bf16", "f32"):
        b = W.small_case(11, dt, 4, 2, 16, context_lens=[37, 16, 5], query_lens=[1, 1, 1],
                         num_prefill=0)
        for s in range(b.num_seqs):
            m = int(b.context_lens[s]) - 1
            K, V = R.gather_kv(b.k_cache, b.v_cache, b.block_tables[s], m, 16, dt)
            assert np.array_equal(K, R.to_f64(b.pre_k[s], dt))
            assert np.array_equal(V, R.to_f64(b.pre_v[s], dt))


def pin_cache_write_v_copy_and_sentinels(R):
    """V lands bit-exact; K at position 0 is the unrotated k (cos 0 = 1);
    every slot not named keeps its prior bits; slot -1 writes nothing."""
    b = W.small_case(12, "bf16", 4, 2, 32, context_lens=[21, 9], query_lens=[21, 9], num_prefill=2)
    pos = np.zeros_like(b.positions)
    slots = b.slot_mapping.copy()
    slots[3] = -1
    q_out, kc, vc = R.rope_cache_write(b.qkv, "bf16", pos, slots, b.k_cache, b.v_cache, 4, 2, 32, 16, 1e6)
    heads = b.qkv.reshape(-1, 8, 32)
    assert np.array_equal(q_out, heads[:, :4])
    touched = np.zeros(kc.shape[:1] + (16,), bool)
    for t, slot in enumerate(slots):
        if slot < 0:
            continue
        blk, off = divmod(int(slot), 16)
        touched[blk, off] = True
        assert np.array_equal(kc[blk, :, off, :], heads[t, 4:6])
        assert np.array_equal(vc[blk, :, :, off], heads[t, 6:8])
    kt = np.broadcast_to(touched[:, None, :, None], kc.shape)
    vt = np.broadcast_to(touched[:, None, None, :], vc.shape)
    assert np.array_equal(kc[~kt], b.k_cache[~kt]) and np.array_equal(vc[~vt], b.v_cache[~vt])
    assert np.all(kc[~kt] == 0x7FC0)   # untouched slots of fresh blocks stay NaN


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------
def _oracle_out(R, b):
    sh = b.shape
    q_out, kc, vc = R.rope_cache_write(b.qkv, sh.dtype, b.positions, b.slot_mapping, b.k_cache,
                                       b.v_cache, sh.num_heads, sh.num_kv_heads, sh.head_dim,
                                       sh.block_size, sh.rope_theta)
    out = R.attention_varlen(q_out, kc, vc, b.cu_seqlens_q, b.context_lens, b.block_tables,
                             sh.num_heads, sh.num_kv_heads, sh.head_dim, sh.block_size, sh.dtype)
    return q_out, kc, vc, out


def pin_brute_force_tiny(R):
    """Whole step vs the brute force on tiny random cases: prefill chunks
    after cached context, decodes, GQA groups 1..3, odd block sizes."""
    cases = [
        dict(seed=21, dtype="f32", num_heads=4, num_kv_heads=2, head_dim=8,
             context_lens=[7, 12, 5], query_lens=[7, 4, 1], num_prefill=2, block_size=4),
        dict(seed=22, dtype="bf16", num_heads=6, num_kv_heads=2, head_dim=8,
             context_lens=[9, 3, 17], query_lens=[3, 1, 1], num_prefill=1, block_size=2),
        dict(seed=23, dtype="bf16", num_heads=3, num_kv_heads=3, head_dim=4,
             context_lens=[6, 1], query_lens=[6, 1], num_prefill=1, block_size=1),
        dict(seed=24, dtype="f32", num_heads=2, num_kv_heads=1, head_dim=16,
             context_lens=[19, 2], query_lens=[19, 1], num_prefill=1, block_size=16),
    ]
    for cs in cases:
        b = W.small_case(**cs)
        q_out, kc, vc, out = _oracle_out(R, b)
        bq, bout = brute.run(b)
        assert np.array_equal(R.to_f64(q_out, cs["dtype"]), np.array(bq)), cs["seed"]
        assert np.allclose(out, np.array(bout), rtol=0, atol=1e-12), (cs["seed"], np.abs(out - np.array(bout)).max())


def pin_sdpa_contiguous_gqa(R):
    """Fresh causal prefill (n == c) equals torch SDPA in float64 on the
    logical K/V with each KV head repeated G times (enable_gqa)."""
    b = W.small_case(31, "f32", 8, 2, 32, context_lens=[40, 23], query_lens=[40, 23],
                     num_prefill=2, block_size=16)
    q_out, kc, vc, out = _oracle_out(R, b)
    cu = b.cu_seqlens_q
    for s in range(2):
        c = int(b.context_lens[s])
        # logical K/V, read back through the generator-independent slot list
        ks, vs = [], []
        for t in range(cu[s], cu[s + 1]):
            blk, off = divmod(int(b.slot_mapping[t]), 16)
            ks.append(kc[blk, :, off, :].astype(np.float64))
            vs.append(vc[blk, :, :, off].astype(np.float64))
        K = torch.from_numpy(np.stack(ks)).permute(1, 0, 2)[None]       # [1][Hkv][c][d]
        V = torch.from_numpy(np.stack(vs)).permute(1, 0, 2)[None]
        Q = torch.from_numpy(q_out[cu[s]:cu[s + 1]].astype(np.float64)).permute(1, 0, 2)[None]
        o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True, enable_gqa=True)
        want = o[0].permute(1, 0, 2).numpy()
        assert want.shape == (c, 8, 32)
        assert np.allclose(out[cu[s]:cu[s + 1]], want, rtol=0, atol=1e-12)


def _decode_case(seed, dtype="f32", H=4, Hkv=2, d=16, ctx=(30, 1, 17), scale_v=1.0):
    return W.small_case(seed, dtype, H, Hkv, d, context_lens=list(ctx), query_lens=[1] * len(ctx),
                        num_prefill=0, value_scale=scale_v)


def pin_constant_v_and_row_sums(R):
    """Probabilities of every row sum to 1 and a constant V yields that
    constant."""
    b = _decode_case(41)
    q_out, kc, vc, _ = _oracle_out(R, b)
    sh = b.shape
    out, probs = R.attention_varlen(q_out, kc, vc, b.cu_seqlens_q, b.context_lens, b.block_tables,
                                    sh.num_heads, sh.num_kv_heads, sh.head_dim, 16, "f32",
                                    return_probs=True)
    for ps in probs:
        for p in ps:
            assert np.allclose(p.sum(axis=-1), 1.0, atol=1e-12)
    vc2 = np.full_like(vc, 0.75)
    out2 = R.attention_varlen(q_out, kc, vc2, b.cu_seqlens_q, b.context_lens, b.block_tables,
                              sh.num_heads, sh.num_kv_heads, sh.head_dim, 16, "f32")
    assert np.allclose(out2, 0.75, atol=1e-13)


def pin_single_key_returns_v0(R):
    """Context 1 (the first token of a sequence): the output is its V row,
    for every head of the group."""
    b = _decode_case(42, ctx=(1, 1))
    q_out, kc, vc, out = _oracle_out(R, b)
    heads = b.qkv.reshape(b.num_tokens, 8, 16)
    for t in range(2):
        for h in range(4):
            assert np.array_equal(out[t, h], heads[t, 4 + 2 + h // 2].astype(np.float64))


def pin_zero_query_gives_mean(R):
    """q = 0 makes every score 0: the output is the plain mean of the
    visible V rows (prefill rows see a growing prefix)."""
    b = W.small_case(43, "f32", 4, 2, 16, context_lens=[13], query_lens=[13], num_prefill=1)
    q_out, kc, vc, _ = _oracle_out(R, b)
    sh = b.shape
    out = R.attention_varlen(np.zeros_like(q_out), kc, vc, b.cu_seqlens_q, b.context_lens,
                             b.block_tables, 4, 2, 16, 16, "f32")
    heads = b.qkv.reshape(13, 8, 16).astype(np.float64)
    for i in range(13):
        for h in range(4):
            want = heads[:i + 1, 6 + h // 2].mean(axis=0)
            assert np.allclose(out[i, h], want, atol=1e-13)


def pin_needle(R):
    """One cached key equal to a large multiple of the rotated query makes
    its score exceed every other by far more than exp's range: the output
    is that key's V row (to 1e-12)."""
    b = _decode_case(44, ctx=(25,))
    sh = b.shape
    q_out, kc, vc, _ = _oracle_out(R, b)
    j = 9
    blk, off = divmod(int(b.block_tables[0, j // 16]) * 16 + j % 16, 16)
    for g in range(2):
        kc[blk, g, off, :] = 64.0 * q_out[0, 2 * g].astype(np.float32)   # needle for head 2g
    out = R.attention_varlen(q_out, kc, vc, b.cu_seqlens_q, b.context_lens, b.block_tables,
                             4, 2, 16, 16, "f32")
    for g in range(2):
        assert np.allclose(out[0, 2 * g], vc[blk, g, :, off].astype(np.float64), atol=1e-12)


def pin_causal_future_invisible(R):
    """Changing K/V at positions after row i leaves rows 0..i unchanged."""
    b = W.small_case(45, "f32", 4, 2, 16, context_lens=[20], query_lens=[20], num_prefill=1)
    q_out, kc, vc, out = _oracle_out(R, b)
    cut = 11
    kc2, vc2 = kc.copy(), vc.copy()
    for j in range(cut + 1, 20):
        blk, off = divmod(int(b.slot_mapping[j]), 16)
        kc2[blk, :, off, :] += 3.0
        vc2[blk, :, :, off] -= 5.0
    out2 = R.attention_varlen(q_out, kc2, vc2, b.cu_seqlens_q, b.context_lens, b.block_tables,
                              4, 2, 16, 16, "f32")
    assert np.array_equal(out2[:cut + 1], out[:cut + 1])
    assert not np.allclose(out2[cut + 1:], out[cut + 1:])


def pin_gqa_equals_mha(R):
    """GQA over Hkv heads equals MHA whose KV head h is GQA's KV head
    h // (H/Hkv) (each KV head repeated G times, consecutively)."""
    H, Hkv, d, G = 6, 2, 16, 3
    b = _decode_case(46, H=H, Hkv=Hkv, d=d, ctx=(20, 7))
    q_out, kc, vc, out = _oracle_out(R, b)
    rep = np.repeat(np.arange(Hkv), G)
    kc_m, vc_m = kc[:, rep], vc[:, rep]
    out_m = R.attention_varlen(q_out, kc_m, vc_m, b.cu_seqlens_q, b.context_lens, b.block_tables,
                               H, H, d, 16, "f32")
    assert np.array_equal(out, out_m)
    # and the grouping is consecutive, not round-robin
    rr = np.tile(np.arange(Hkv), G)
    out_rr = R.attention_varlen(q_out, kc[:, rr], vc[:, rr], b.cu_seqlens_q, b.context_lens,
                                b.block_tables, H, H, d, 16, "f32")
    assert not np.allclose(out, out_rr)


def pin_paged_equals_contiguous(R):
    """Two pools holding the same logical content under different block
    permutations give identical outputs; so does a pool with blocks in
    logical order (the contiguous layout)."""
    b = _decode_case(47, ctx=(45, 33), H=4, Hkv=2, d=16)
    q_out, kc, vc, out = _oracle_out(R, b)
    rng = np.random.default_rng(0)
    for perm in (rng.permutation(b.num_blocks), np.arange(b.num_blocks)[::-1]):
        inv = np.empty_like(perm)
        inv[perm] = np.arange(len(perm))
        kc2 = np.empty_like(kc)
        vc2 = np.empty_like(vc)
        kc2[inv] = kc
        vc2[inv] = vc
        bt2 = inv[b.block_tables]
        out2 = R.attention_varlen(q_out, kc2, vc2, b.cu_seqlens_q, b.context_lens, bt2, 4, 2, 16,
                                  16, "f32")
        assert np.array_equal(out2, out)


def pin_decode_is_last_prefill_row(R):
    """Tiny fp32 sequence: 16-token prefill then 4 decode steps equals the
    matching rows of one 20-token prefill."""
    steps = W.tiny_f32_steps()
    sh = steps[0].shape
    kc, vc = steps[0].k_cache, steps[0].v_cache
    outs = []
    for st in steps:
        q_out, kc, vc = R.rope_cache_write(st.qkv, "f32", st.positions, st.slot_mapping, kc, vc,
                                           4, 2, 64, 16, 1e6)
        outs.append(R.attention_varlen(q_out, kc, vc, st.cu_seqlens_q, st.context_lens,
                                       st.block_tables, 4, 2, 64, 16, "f32"))
    qkv = np.concatenate([st.qkv for st in steps])
    pos = np.arange(20, dtype=np.int32)
    slots = np.concatenate([st.slot_mapping for st in steps])
    q_out, kc2, vc2 = R.rope_cache_write(qkv, "f32", pos, slots, steps[0].k_cache, steps[0].v_cache,
                                         4, 2, 64, 16, 1e6)
    full = R.attention_varlen(q_out, kc2, vc2, np.array([0, 20]), np.array([20]),
                              steps[-1].block_tables, 4, 2, 64, 16, "f32")
    seq = np.concatenate(outs)
    assert np.allclose(seq, full, rtol=0, atol=1e-13), np.abs(seq - full).max()
    assert np.array_equal(kc.view(np.uint32), kc2.view(np.uint32))      # bitwise, NaN tails included
    assert np.array_equal(vc.view(np.uint32), vc2.view(np.uint32))
    del sh


# ---------------------------------------------------------------------------
# FP8 E4M3FN cache codes
# ---------------------------------------------------------------------------
def pin_fp8_decode_table(R):
    """Values the E4M3FN definition fixes (sign, 4-bit exponent with bias 7,
    3-bit mantissa, subnormals below 2**-6, NaN at S.1111.111, no infinity)."""
    table = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
             0x39: 1.125, 0x3F: 1.875, 0x40: 2.0, 0x48: 4.0, 0x77: 240.0, 0x78: 256.0,
             0x7E: 448.0, 0x80: -0.0, 0xB8: -1.0, 0xFE: -448.0}
    for c, v in table.items():
        got = float(R.fp8_e4m3_decode(np.array([c], np.uint8))[0])
        assert got == v and math.copysign(1.0, got) == math.copysign(1.0, v), (hex(c), got, v)
    assert np.isnan(R.fp8_e4m3_decode(np.array([0x7F, 0xFF], np.uint8))).all()


def pin_fp8_matches_torch(R):
    """torch's float8_e4m3fn: decode of all 256 codes, and round-to-nearest-
    even encoding of random in-range values and of every midpoint between
    neighbouring codes."""
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    dec = R.fp8_e4m3_decode(codes)
    fin = np.isfinite(ref)
    assert np.array_equal(dec[fin], ref[fin]) and np.isnan(dec[~fin]).all()
    rng = np.random.default_rng(11)
    pos = np.sort(ref[fin & (ref > 0)])
    x = np.concatenate([rng.standard_normal(20000) * np.exp2(rng.integers(-14, 9, 20000)),
                        (pos[:-1] + pos[1:]) / 2, -(pos[:-1] + pos[1:]) / 2, ref[fin]])
    x = x[np.abs(x) <= 448.0]
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(R.fp8_e4m3_encode(x), want)


def pin_fp8_roundtrip_ties_saturation(R):
    """Every finite code re-encodes to itself; ties go to the even mantissa;
    magnitudes past 448 saturate; the relative error of a normal value is at
    most 2**-4 (half a unit in the last of 3 mantissa bits)."""
    codes = np.arange(256, dtype=np.uint8)
    fin = (codes & 0x7F) != 0x7F
    assert np.array_equal(R.fp8_e4m3_encode(R.fp8_e4m3_decode(codes[fin])), codes[fin])
    ties = {1.0625: 0x38, 1.1875: 0x3A, 2.0 ** -10: 0x00, 3 * 2.0 ** -10: 0x02, 432.0: 0x7E}
    for v, c in ties.items():
        assert int(R.fp8_e4m3_encode(np.array([v]))[0]) == c, (v, c)
    big = np.array([448.0, 449.0, 464.0, 465.0, 1e6, -500.0, -1e30])
    assert R.fp8_e4m3_encode(big).tolist() == [0x7E] * 5 + [0xFE] * 2
    rng = np.random.default_rng(12)
    x = rng.uniform(2.0 ** -6, 448.0, 50000) * rng.choice([-1.0, 1.0], 50000)
    err = np.abs(R.fp8_e4m3_decode(R.fp8_e4m3_encode(x)) - x)
    assert np.all(err <= 2.0 ** -4 * np.abs(x) * (1 + 1e-12))


def pin_fp8_cache_write(R):
    """FP8 cache write: values that are exact E4M3FN multiples of the scale
    are stored exactly; other K and V entries land within the format's
    half-step of the float64 reference rows; slots not named keep their
    previous codes."""
    b = W.small_case(61, "bf16", 4, 2, 16, context_lens=[20, 5], query_lens=[20, 5],
                     num_prefill=2, keep_logical=True)
    sh = b.shape
    ks, vs = 0.0312, 0.0287
    kc0 = np.full(b.k_cache.shape, 0x55, np.uint8)
    vc0 = np.full(b.v_cache.shape, 0xAA, np.uint8)
    _, kc, vc = R.rope_cache_write(b.qkv, sh.dtype, b.positions, b.slot_mapping, kc0, vc0,
                                   sh.num_heads, sh.num_kv_heads, sh.head_dim, sh.block_size,
                                   sh.rope_theta, "fp8", ks, vs)
    T, H, Hkv, d, B = b.num_tokens, sh.num_heads, sh.num_kv_heads, sh.head_dim, sh.block_size
    heads = R.bf16_bits_to_f64(b.qkv).reshape(T, H + 2 * Hkv, d)
    krot = R.rope_neox(heads[:, H:H + Hkv], b.positions, sh.rope_theta)
    written = np.zeros(kc.shape[:3], bool)
    for t in range(T):
        blk, off = divmod(int(b.slot_mapping[t]), B)
        written[blk, :, off] = True
        kd = R.fp8_e4m3_decode(kc[blk, :, off, :]) * ks
        vd = R.fp8_e4m3_decode(vc[blk, :, :, off]) * vs
        for got, ref, sc in ((kd, krot[t], ks), (vd, heads[t, H + Hkv:], vs)):
            tol = np.maximum(2.0 ** -4 * np.abs(ref), 2.0 ** -10 * sc) * (1 + 1e-9)
            assert np.all(np.abs(got - ref) <= tol)
    assert np.all(kc[~written] == 0x55)
    assert np.all(vc.transpose(0, 1, 3, 2)[~written] == 0xAA)
    # exact multiples of the scale: the codes' own values come back exactly
    vals = R.fp8_e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    xs = (vals * 0.25)[None, :]
    assert np.array_equal(R.fp8_e4m3_encode(xs / 0.25)[0], np.arange(0, 0x7F, dtype=np.uint8))


def pin_fp8_attention_reads_dequantized_cache(R):
    """Attention over an FP8 cache equals attention over a float cache holding
    the decoded values times the scales (power-of-two scales keep the float
    copy exact)."""
    b = W.small_case(62, "bf16", 8, 2, 16, context_lens=[40, 9, 33], query_lens=[7, 1, 33],
                     num_prefill=3, keep_logical=True)
    sh = b.shape
    ks, vs = 0.25, 2.0
    rng = np.random.default_rng(63)
    kc = rng.integers(0, 256, b.k_cache.shape).astype(np.uint8)
    vc = rng.integers(0, 256, b.v_cache.shape).astype(np.uint8)
    kc[(kc & 0x7F) == 0x7F] = 0x38
    vc[(vc & 0x7F) == 0x7F] = 0xB8
    kf = (R.fp8_e4m3_decode(kc) * ks).astype(np.float32)
    vf = (R.fp8_e4m3_decode(vc) * vs).astype(np.float32)
    q = R.from_f64(rng.standard_normal((b.num_tokens, sh.num_heads, sh.head_dim)), "f32")
    args = (b.cu_seqlens_q, b.context_lens, b.block_tables, sh.num_heads, sh.num_kv_heads,
            sh.head_dim, sh.block_size, "f32")
    want = R.attention_varlen(q, kf, vf, *args)
    got = R.attention_varlen(q, kc, vc, *args, cache_dtype="fp8", k_scale=ks, v_scale=vs)
    assert np.array_equal(got, want)


# ---------------------------------------------------------------------------
# Qwen3 q/k RMSNorm
# ---------------------------------------------------------------------------
def pin_rms_norm_matches_torch(R):
    """torch.nn.functional.rms_norm (float64) on random heads and weights."""
    rng = np.random.default_rng(71)
    x = rng.standard_normal((5, 3, 128)) * rng.uniform(0.01, 10, (5, 3, 1))
    w = rng.standard_normal(128) * 0.2 + 1.0
    for eps in (1e-6, 1e-2, 0.0):
        want = torch.nn.functional.rms_norm(torch.from_numpy(x), (128,), torch.from_numpy(w),
                                            eps).numpy()
        np.testing.assert_allclose(R.rms_norm_heads(x, w, eps), want, rtol=1e-13, atol=1e-15)


def pin_rms_norm_closed_forms(R):
    """With w = 1 and eps = 0 the output has RMS exactly 1 (norm sqrt(d)) and
    is invariant to scaling x; a constant head c maps to sign(c) c / sqrt(c^2
    + eps) per element; eps keeps a zero head at zero."""
    rng = np.random.default_rng(72)
    x = rng.standard_normal((4, 64))
    y = R.rms_norm_heads(x, np.ones(64), 0.0)
    np.testing.assert_allclose(np.sqrt((y * y).mean(-1)), 1.0, rtol=1e-14)
    np.testing.assert_allclose(R.rms_norm_heads(37.5 * x, np.ones(64), 0.0), y, rtol=1e-13)
    for c, eps in ((0.5, 1e-6), (-3.0, 0.25)):
        got = R.rms_norm_heads(np.full((1, 16), c), np.ones(16), eps)
        np.testing.assert_allclose(got, c / math.sqrt(c * c + eps), rtol=1e-15)
    assert np.all(R.rms_norm_heads(np.zeros((2, 8)), np.ones(8), 1e-6) == 0.0)


def pin_qk_norm_in_cache_write(R):
    """The cache write with q/k norm weights: stored q/k have the norm of the
    normalised head times the weight (the rotation preserves norms), v is
    untouched, and unit weights with eps 0 leave every stored head with RMS 1
    up to the storage rounding."""
    b = W.small_case(73, "f32", 4, 2, 32, context_lens=[9, 4], query_lens=[9, 4], num_prefill=2,
                     keep_logical=True)
    sh = b.shape
    T, H, Hkv, d = b.num_tokens, sh.num_heads, sh.num_kv_heads, sh.head_dim
    args = (b.qkv, sh.dtype, b.positions, b.slot_mapping, b.k_cache, b.v_cache, H, Hkv, d,
            sh.block_size, sh.rope_theta)
    one = np.ones(d, np.float32)
    q_out, kc, vc = R.rope_cache_write(*args, q_norm_weight=one, k_norm_weight=one, rms_eps=0.0)
    assert np.allclose(np.sqrt((q_out.astype(np.float64) ** 2).mean(-1)), 1.0, rtol=1e-6)
    B = sh.block_size
    for t in range(T):
        blk, off = divmod(int(b.slot_mapping[t]), B)
        k = kc[blk, :, off, :].astype(np.float64)
        assert np.allclose(np.sqrt((k * k).mean(-1)), 1.0, rtol=1e-6)
        assert np.array_equal(vc[blk, :, :, off], b.qkv[t].reshape(H + 2 * Hkv, d)[H + Hkv:])
    w = np.linspace(0.5, 1.5, d).astype(np.float32)
    q2, _, _ = R.rope_cache_write(*args, q_norm_weight=w, k_norm_weight=one, rms_eps=0.0)
    x = b.qkv.reshape(T, H + 2 * Hkv, d)[:, :H].astype(np.float64)
    want = np.sqrt(((x / np.sqrt((x * x).mean(-1, keepdims=True)) * w) ** 2).sum(-1))
    assert np.allclose(np.sqrt((q2.astype(np.float64) ** 2).sum(-1)), want, rtol=1e-6)

def pin_dynamic_ntk_closed_forms(R):
    """Dynamic-NTK scaling, the parts fixed without any formula: factor 1
    changes nothing, the table spans factor x original positions, the fastest
    frequency (i = 0) stays 1 and every other one turns slower."""
    for d in (64, 128):
        base, L = R.rope_dynamic_ntk(1e6, d, 1.0, 32768)
        assert base == 1e6 and L == 32768
        for s, L0 in ((2.0, 4096), (4.0, 32768), (3.0, 1000)):
            base, L = R.rope_dynamic_ntk(1e6, d, s, L0)
            assert L == int(s * L0)
            f0, f1 = R.rope_inv_freq(d, 1e6), R.rope_inv_freq(d, base)
            assert f1[0] == f0[0] == 1.0
            assert np.all(f1[1:] < f0[1:])


def pin_dynamic_ntk_matches_transformers(R):
    """The scaled frequencies against an independent implementation of the
    published dynamic-NTK rule: transformers' rope utilities
    (``_compute_dynamic_ntk_parameters``) at a sequence length of factor x
    original positions, the length the oracle's table spans.  The library
    returns float32 frequencies, so they agree to float32 precision.  Settings:
    the [P2] §7.1 one (factor 2 over 4096), factor 4 over Qwen2's native
    32768, and factor 3 over 1000, at head_dim 64 and 128."""
    tr = pytest.importorskip("transformers")
    from transformers.modeling_rope_utils import _compute_dynamic_ntk_parameters
    for d in (64, 128):
        for s, L0 in ((2.0, 4096), (4.0, 32768), (3.0, 1000)):
            cfg = tr.Qwen2Config(hidden_size=4 * d, num_attention_heads=4, num_key_value_heads=2,
                                 max_position_embeddings=L0,
                                 rope_parameters={"rope_type": "dynamic", "rope_theta": 1e6,
                                                  "factor": s})
            base, L = R.rope_dynamic_ntk(1e6, d, s, L0)
            assert L == int(s * L0)
            want, _ = _compute_dynamic_ntk_parameters(cfg, device="cpu", seq_len=L)
            want = want.double().numpy()
            assert want.shape == (d // 2,)
            np.testing.assert_allclose(R.rope_inv_freq(d, base), want, rtol=1e-6, atol=0)


# ---------------------------------------------------------------------------
# shared-prefix (cascade) decode
# ---------------------------------------------------------------------------
def _cascade_case(R, seed, dtype, H, Hkv, d, ctx, groups, B=16, fp8=False):
    kw = dict(cache_dtype="fp8", k_scale=W.FP8_K_SCALE, v_scale=W.FP8_V_SCALE) if fp8 else {}
    b = W.small_case(seed, dtype, H, Hkv, d, context_lens=list(ctx), query_lens=[1] * len(ctx),
                     num_prefill=0, block_size=B, keep_logical=False, **kw)
    W.with_prefix_groups(b, groups)
    sh = b.shape
    cd = "fp8" if fp8 else None
    q_out, kc, vc = R.rope_cache_write(b.qkv, dtype, b.positions, b.slot_mapping, b.k_cache,
                                       b.v_cache, H, Hkv, d, B, sh.rope_theta, cd, sh.k_scale,
                                       sh.v_scale)
    return b, q_out, kc, vc


def _cascade(R, b, q_out, kc, vc, groups=None):
    sh = b.shape
    ind, seqs, lens = b.prefix_groups if groups is None else groups
    cd = sh.cache_dtype
    return R.attention_decode_cascade(q_out, kc, vc, b.block_tables, b.context_lens, ind, seqs,
                                      lens, sh.num_heads, sh.num_kv_heads, sh.head_dim,
                                      sh.block_size, sh.dtype, cache_dtype=cd,
                                      k_scale=sh.k_scale, v_scale=sh.v_scale)


def pin_cascade_equals_plain_decode(R):
    """The cascade (shared prefix attended once per group, private suffix per
    member, exact merge) equals softmax attention over each member's whole
    block table: several groups, a non-member, GQA 2..8, odd block sizes, a
    one-key suffix, FP8 codes."""
    cases = [
        (61, "f32", 4, 2, 16, (40, 70, 33, 90, 17), [([0, 1, 3], 32), ([2], 16)], 16, False),
        (62, "bf16", 6, 2, 8, (9, 14, 11, 5, 20), [([1, 2, 4], 8)], 4, False),
        (63, "bf16", 8, 1, 32, (49, 51, 50), [([0, 1, 2], 48)], 16, False),
        (64, "bf16", 4, 2, 16, (30, 45, 21), [([2, 0], 16), ([1], 32)], 16, True),
    ]
    for seed, dt, H, Hkv, d, ctx, groups, B, fp8 in cases:
        b, q_out, kc, vc = _cascade_case(R, seed, dt, H, Hkv, d, ctx, groups, B, fp8)
        sh = b.shape
        plain = R.attention_decode(q_out, kc, vc, b.block_tables, b.context_lens, H, Hkv, d, B,
                                   dt, cache_dtype=sh.cache_dtype, k_scale=sh.k_scale,
                                   v_scale=sh.v_scale)
        cas = _cascade(R, b, q_out, kc, vc)
        assert np.allclose(cas, plain, rtol=0, atol=1e-12), (seed, np.abs(cas - plain).max())


def pin_cascade_needles(R):
    """Closed forms on each side of the merge: with every query head equal to
    u, a key 40 u in the shared prefix makes every member's output that key's
    V row; the same key in one member's private suffix does so for that
    member only (others keep their plain output)."""
    H, Hkv, d, B = 4, 2, 16, 16
    ctx, groups = (40, 37, 50), [([0, 1, 2], 32)]
    b, q_out, kc, vc = _cascade_case(R, 65, "f32", H, Hkv, d, ctx, groups, B)
    u = np.linspace(-1.0, 1.0, d).astype(np.float32)
    q_out[:] = u
    for where, key in (("prefix", 5), ("suffix", 34)):
        kc2, vc2 = kc.copy(), vc.copy()
        seq = 1                                         # the suffix needle sits in member 1
        blk, off = int(b.block_tables[seq, key // B]), key % B
        kc2[blk, :, off, :] = 40.0 * u
        out = _cascade(R, b, q_out, kc2, vc2)
        want = vc2[blk, :, :, off].astype(np.float64)  # [Hkv][d]
        for s in range(3):
            for h in range(H):
                if where == "prefix" or s == seq:
                    assert np.allclose(out[s, h], want[h // 2], rtol=0, atol=1e-12), (where, s, h)
                else:
                    assert not np.allclose(out[s, h], want[h // 2], rtol=0, atol=1e-3), (where, s, h)


def pin_cascade_contract(R):
    """Groupings that break the sharing contract are refused: members that
    do not hold the same prefix blocks, a prefix that reaches a member's last
    key, a partial block, a member listed twice."""
    b, q_out, kc, vc = _cascade_case(R, 66, "f32", 4, 2, 16, (40, 70, 33), [([0, 1], 32)], 16)
    bad = [
        ([0, 2], [0, 2], [32]),          # member 2 holds its own blocks
        ([0, 2], [0, 1], [48]),          # 48 >= context 40 of member 0
        ([0, 2], [0, 1], [24]),          # not whole blocks
        ([0, 2], [0, 0], [16]),          # listed twice
    ]
    for ind, seqs, lens in bad:
        try:
            _cascade(R, b, q_out, kc, vc, (np.array(ind), np.array(seqs), np.array(lens)))
        except ValueError:
            continue
        raise AssertionError(f"grouping {ind, seqs, lens} accepted")


ALL_PINS = [
    pin_cascade_equals_plain_decode, pin_cascade_needles, pin_cascade_contract,
    pin_dynamic_ntk_closed_forms, pin_dynamic_ntk_matches_transformers,
    pin_rms_norm_matches_torch, pin_rms_norm_closed_forms, pin_qk_norm_in_cache_write,
    pin_fp8_decode_table, pin_fp8_matches_torch, pin_fp8_roundtrip_ties_saturation,
    pin_fp8_cache_write, pin_fp8_attention_reads_dequantized_cache,
    pin_bf16_rounding_values, pin_bf16_rounding_matches_torch,
    pin_rope_unit_vector_neox, pin_rope_frequency_closed_forms, pin_rope_identity_at_zero,
    pin_rope_norm_preserved, pin_rope_relative_position, pin_rope_composition,
    pin_rope_complex_form,
    pin_gather_matches_generator_layout, pin_cache_write_v_copy_and_sentinels,
    pin_brute_force_tiny, pin_sdpa_contiguous_gqa, pin_constant_v_and_row_sums,
    pin_single_key_returns_v0, pin_zero_query_gives_mean, pin_needle,
    pin_causal_future_invisible, pin_gqa_equals_mha, pin_paged_equals_contiguous,
    pin_decode_is_last_prefill_row,
]
