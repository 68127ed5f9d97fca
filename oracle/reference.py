"""Plain float64 restatement of the paged GQA attention step.

TEST INFRASTRUCTURE ONLY (see the package docstring for who may use it).

The step, in the order the pages describe it for one Qwen2 attention layer
served by vLLM ([P2] §2.2 and §4.1; [P3] §2.1):

  1. the fused QKV projection output is split into q, k, v by columns
     (q heads, then k heads, then v heads) -- [P2] §2.2 (QKVParallelLinear),
     §4.3 (packed_modules_mapping q_proj, k_proj, v_proj -> qkv_proj);
  2. rotary position embedding is applied to q and k with the full head
     dimension rotated and base rope_theta -- [P2] §2.2 (get_rope(head_dim,
     rotary_dim=head_dim, max_position, base=rope_theta)); [P1] §2
     (rope_theta read with default 1000000);
  3. k and v are written into the paged KV cache, fixed-size blocks handed
     out like OS memory pages -- [P3] §2.1 (PagedAttention), [P5] §5
     (seq.block_table);
  4. attention of every query row over its sequence's cached keys, causal,
     with GQA (query heads grouped over fewer KV heads) and scaling
     head_dim ** -0.5 -- [P1] §2 (28:4, "7 Q heads share one KV group"),
     [P2] §2.2 and §7.3 (causal mask), [P4] §3 (flash-attn varlen packed
     prefill), [P3] §2.1 (PagedAttention decode).

Where the pages are silent the plainest reading is taken (each one is listed
with the function that uses it):
  * NeoX pairing: element i is rotated with element i + d/2 (half split);
  * frequency law f_i = theta ** (-2 i / d), i < d/2;
  * dynamic-NTK rope scaling ([P2] §7.1, [P1] §3): a larger base for a
    table of factor * original_max_position positions (rope_dynamic_ntk);
  * slot = physical_block * block_size + offset, slot < 0 means "skip";
  * query row i of a sequence with n new rows and context c sits at
    position c - n + i and sees keys 0..c-n+i (bottom-right causal);
  * softmax is base e, max-subtracted, masked keys excluded;
  * rotated q and k, and the output, are rounded once from float64 to the
    storage dtype (round to nearest even); v is copied bit for bit.
  * Qwen3 q/k norm ([P5] §5: the attention module holds q_norm and k_norm
    RMSNorm modules; §3.2 passes rms_norm_eps): each q and k head is
    RMS-normalised over head_dim with a learned [head_dim] weight,
    y = x / sqrt(mean(x^2) + eps) * w, after the QKV split and before the
    rotation (the pages print the modules, not their order of use), in
    float64 together with the rotation, rounded once;
  * shared-prefix (cascade) decode ([P1] §3 and §4: with prefix caching
    the attention layer reuses the KV blocks of an identical prefix): the
    shared prefix blocks are attended once per group of sequences that hold
    them, each member's private suffix separately, and the two partial
    softmax states are merged exactly; the result is defined to be the plain
    decode attention over the member's whole block table
    (attention_decode_cascade);
  * FP8 KV cache ([P2] §4.1 and §4.2 list FP8 KV-cache quantization with
    per-layer cache scale parameters; §6.3 names the E4M3FN format): the
    cache holds E4M3FN codes of the exact rotated key (or the value) divided
    by one scale per tensor (k_scale, v_scale), rounded once to nearest even
    and saturated at +-448; attention reads code value * scale.

Cache layouts (interface definition):
  K cache [num_blocks][num_kv_heads][block_size][head_dim]
  V cache [num_blocks][num_kv_heads][head_dim][block_size]

Storage conventions: bf16 tensors are numpy uint16 bit patterns, fp32 tensors
are numpy float32, FP8 cache entries are numpy uint8 E4M3FN codes.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "rope_inv_freq", "rope_dynamic_ntk", "rope_neox", "to_f64", "from_f64", "f64_to_bf16_bits",
    "bf16_bits_to_f64", "rope_cache_write", "gather_kv", "causal_visible",
    "softmax_rows", "kv_head_for", "default_scale", "attention_varlen",
    "attention_decode", "run_step", "fp8_e4m3_decode", "fp8_e4m3_encode", "E4M3_MAX",
    "rms_norm_heads", "attention_decode_cascade", "check_prefix_groups",
]


# ---------------------------------------------------------------------------
# storage <-> float64
# ---------------------------------------------------------------------------
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64, exactly (bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 to bf16 once, round-to-nearest-even; return uint16 bits.

    bf16 keeps 8 significant bits and fp32's exponent range.  For |x| in
    [2**(e-1), 2**e) the spacing is 2**(e-8); below the smallest normal
    (2**-126) the spacing stays 2**-133.  Dividing by the spacing is exact
    (a power of two), ``np.rint`` rounds half to even, and the product is
    exactly representable, so there is a single rounding."""
    x = np.asarray(x, dtype=np.float64)
    finite = np.isfinite(x)
    xf = np.where(finite, x, 0.0)
    _, e = np.frexp(xf)
    e = np.maximum(e, -125)
    ulp = np.ldexp(1.0, e - 8)
    r = np.rint(xf / ulp) * ulp
    with np.errstate(over="ignore"):
        f32 = r.astype(np.float32)           # exact, or +-inf past the bf16 range
    bits = (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = np.where(np.isnan(x), np.uint16(0x7FC0), bits)
    bits = np.where(np.isposinf(x), np.uint16(0x7F80), bits)
    bits = np.where(np.isneginf(x), np.uint16(0xFF80), bits)
    return bits.astype(np.uint16)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array -> float64 (exact widening)."""
    if dtype == "bf16":
        return bf16_bits_to_f64(a)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def from_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """float64 -> storage dtype, one round-to-nearest-even rounding."""
    if dtype == "bf16":
        return f64_to_bf16_bits(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# 2. rotary position embedding (NeoX half split)
# ---------------------------------------------------------------------------
def rope_inv_freq(head_dim: int, theta: float) -> np.ndarray:
    """Rotation frequencies f_i = theta ** (-2 i / d), i = 0 .. d/2 - 1.

    [P2] §2.2: get_rope(head_dim, rotary_dim=head_dim, ..., base=rope_theta)
    -- the whole head is rotated with base rope_theta; [P1] §2: Qwen2's
    rope_theta is 1e6.  The pages do not print the law; this is the standard
    one for a given base."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * i / float(head_dim))


def rope_dynamic_ntk(theta: float, head_dim: int, factor: float, original_max_position: int):
    """Dynamic-NTK rope scaling: (scaled base, table length).

    [P2] §7.1 gives the setting {"type": "dynamic", "factor": 2.0,
    "original_max_position": 4096} and says it raises the RoPE base
    frequency so that longer contexts fit while short ones keep their
    behaviour; [P1] §3: vLLM hands rope_scaling to get_rope, and Qwen2 needs
    it past its native 32768 positions.  The pages print no formula.  Reading
    taken (the published NTK-aware rule, as vLLM's get_rope uses it): one
    table covers L = factor * original_max_position positions, and the base
    becomes
        theta' = theta * (factor * L / original - (factor - 1)) ** (d / (d - 2))
    so the slowest rotation (i = d/2 - 1) turns factor * L / original -
    (factor - 1) times slower while the fastest (i = 0) is unchanged.  With
    factor 1 nothing changes."""
    s = float(factor)
    L = int(s * int(original_max_position))
    d = float(head_dim)
    base = float(theta) * (s * L / float(original_max_position) - (s - 1.0)) ** (d / (d - 2.0))
    return base, L


def rope_neox(x: np.ndarray, positions: np.ndarray, theta: float) -> np.ndarray:
    """Rotate ``x[..., t, head, :]`` by the angle positions[t] * f_i.

    x: float64 [T][heads][d]; positions: int [T].  NeoX pairing: for
    i < d/2 the pair (x_i, x_{i+d/2}) is rotated:
        y_i       = x_i * cos(a) - x_{i+d/2} * sin(a)
        y_{i+d/2} = x_{i+d/2} * cos(a) + x_i * sin(a),  a = p * f_i
    The angle is formed in float64 for every position."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    f = rope_inv_freq(d, theta)
    a = np.asarray(positions, dtype=np.float64)[:, None] * f[None, :]    # [T][d/2]
    c = np.cos(a)[:, None, :]
    s = np.sin(a)[:, None, :]
    x1 = x[..., :half]
    x2 = x[..., half:]
    y = np.empty_like(x)
    y[..., :half] = x1 * c - x2 * s
    y[..., half:] = x2 * c + x1 * s
    return y


# ---------------------------------------------------------------------------
# FP8 E4M3FN codes (the FP8 KV cache)
# ---------------------------------------------------------------------------
E4M3_MAX = 448.0                    # largest finite E4M3FN value, 1.75 * 2**8


def fp8_e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """E4M3FN code -> float64.  Bit 7 sign, bits 6..3 exponent e (bias 7),
    bits 2..0 mantissa m: e = 0 gives m/8 * 2**-6 (subnormal), otherwise
    (1 + m/8) * 2**(e - 7); the two codes with e = 15, m = 7 are NaN (there
    is no infinity).  ([P2] §6.3 names the format; the layout is its
    definition.)"""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))
    return np.where((e == 15) & ((c & 7) == 7), np.nan, sign * mag)


def fp8_e4m3_encode(x: np.ndarray) -> np.ndarray:
    """float64 -> E4M3FN code, rounded once to nearest (ties to the even
    code) and saturated at +-448 (a cache entry must stay finite: the plain
    reading where the pages give no overflow rule).  Zero keeps its sign."""
    x = np.asarray(x, dtype=np.float64)
    sign = np.signbit(x).astype(np.int64) << 7
    a = np.minimum(np.abs(x), E4M3_MAX)                     # saturate (0x7f is NaN)
    out = np.zeros(x.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    # subnormal range: multiples of 2**-9; m = 8 lands on the smallest normal
    out[sub] = np.rint(a[sub] / 2.0 ** -9).astype(np.int64)
    nrm = ~sub
    if np.any(nrm):
        an = a[nrm]
        e = np.floor(np.log2(an)).astype(np.int64)
        # guard the floor(log2) against rounding at exact powers of two
        e = np.where(np.exp2(e.astype(np.float64)) > an, e - 1, e)
        e = np.where(np.exp2((e + 1).astype(np.float64)) <= an, e + 1, e)
        frac = an / np.exp2(e.astype(np.float64))          # [1, 2), exact
        m = np.rint((frac - 1.0) * 8.0).astype(np.int64)    # ties to even
        carry = m == 8
        e = np.where(carry, e + 1, e)
        m = np.where(carry, 0, m)
        out[nrm] = ((e + 7) << 3) | m
    return (out | sign).astype(np.uint8)


# ---------------------------------------------------------------------------
# Qwen3 per-head RMSNorm of q and k
# ---------------------------------------------------------------------------
def rms_norm_heads(x: np.ndarray, weight: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis (head_dim): x / sqrt(mean(x^2) + eps) * w,
    float64.  ([P5] §5 q_norm / k_norm RMSNorm modules; §3.2 rms_norm_eps.)"""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + float(eps)) * np.asarray(weight, dtype=np.float64)


# ---------------------------------------------------------------------------
# 1-3. split fused QKV, rotate, write the paged cache
# ---------------------------------------------------------------------------
def rope_cache_write(qkv, dtype, positions, slot_mapping, k_cache, v_cache,
                     num_heads, num_kv_heads, head_dim, block_size, theta,
                     cache_dtype=None, k_scale=1.0, v_scale=1.0,
                     q_norm_weight=None, k_norm_weight=None, rms_eps=1e-6):
    """Split the fused QKV rows, rotate q and k, scatter k and v into the cache.

    qkv: storage [T][(H + 2 Hkv) * d]; columns [0, H d) are q, then Hkv k
    heads, then Hkv v heads ([P2] §2.2 fused QKV; §4.3 packed q, k, v).
    Returns (q_out [T][H][d] storage, k_cache', v_cache') -- new arrays, the
    inputs are not modified.  For each token with slot >= 0:
        block = slot // B, offset = slot % B
        K[block][g][offset][:] = rot(k[t][g]);  V[block][g][:][offset] = v[t][g]
    Slots not named keep their previous bits ([P3] §2.1 paged blocks).
    cache_dtype "fp8": the caches hold E4M3FN codes, K = code(rot(k) /
    k_scale), V = code(v / v_scale), each one rounding from float64.
    q_norm_weight / k_norm_weight ([head_dim], storage dtype): Qwen3 q/k norm,
    rot(rms_norm(q)) and rot(rms_norm(k)) instead of rot(q), rot(k)."""
    H, Hkv, d, B = num_heads, num_kv_heads, head_dim, block_size
    qkv = np.asarray(qkv)
    T = qkv.shape[0]
    heads = qkv.reshape(T, H + 2 * Hkv, d)
    x = to_f64(heads, dtype)
    xq, xk = x[:, :H], x[:, H:H + Hkv]
    if q_norm_weight is not None:
        xq = rms_norm_heads(xq, to_f64(q_norm_weight, dtype), rms_eps)
    if k_norm_weight is not None:
        xk = rms_norm_heads(xk, to_f64(k_norm_weight, dtype), rms_eps)
    q_rot = rope_neox(xq, positions, theta)
    k_rot = rope_neox(xk, positions, theta)
    q_out = from_f64(q_rot, dtype)
    if cache_dtype == "fp8":
        k_store = fp8_e4m3_encode(k_rot / float(k_scale))
        v_store = fp8_e4m3_encode(x[:, H + Hkv:] / float(v_scale))
    else:
        k_store = from_f64(k_rot, dtype)
        v_store = heads[:, H + Hkv:]          # stored unchanged (bit copy)
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    for t in range(T):
        slot = int(slot_mapping[t])
        if slot < 0:
            continue
        blk, off = divmod(slot, B)
        kc[blk, :, off, :] = k_store[t]
        vc[blk, :, :, off] = v_store[t]
    return q_out, kc, vc


def gather_kv(k_cache, v_cache, block_table_row, context_len, block_size, dtype,
              cache_dtype=None, k_scale=1.0, v_scale=1.0):
    """Logical keys/values 0..c-1 of one sequence through its block table.

    Logical position j lives in physical block block_table[j // B] at offset
    j % B ([P3] §2.1; [P5] §5 seq.block_table).  Returns float64 K, V of
    shape [c][Hkv][d] (FP8 caches: code value times the tensor's scale)."""
    B = block_size
    j = np.arange(int(context_len))
    blk = np.asarray(block_table_row)[j // B].astype(np.int64)
    off = j % B
    if cache_dtype == "fp8":
        # the decoder applied to each of the 256 codes once, then looked up
        # per element (the same values as decoding every element)
        value = fp8_e4m3_decode(np.arange(256, dtype=np.uint8))
        K = value[np.asarray(k_cache)[blk, :, off, :]] * float(k_scale)
        V = value[np.asarray(v_cache)[blk, :, :, off]] * float(v_scale)
        return K, V
    K = to_f64(np.asarray(k_cache)[blk, :, off, :], dtype)
    V = to_f64(np.asarray(v_cache)[blk, :, :, off], dtype)
    return K, V


# ---------------------------------------------------------------------------
# 4. attention
# ---------------------------------------------------------------------------
def causal_visible(num_rows: int, context_len: int) -> np.ndarray:
    """Boolean [n][c]: query row i (position c - n + i) sees key j iff
    j <= c - n + i.  [P2] §7.3 (causal mask); the alignment of new rows after
    cached context is the plainest reading (the pages do not spell it out)."""
    n, c = int(num_rows), int(context_len)
    pq = c - n + np.arange(n)
    return np.arange(c)[None, :] <= pq[:, None]


def softmax_rows(z: np.ndarray, visible: np.ndarray) -> np.ndarray:
    """Row softmax over visible entries: m = max z, w = exp(z - m),
    pi = w / sum(w); masked entries are excluded (probability exactly 0)."""
    zm = np.where(visible, z, -np.inf)
    m = zm.max(axis=-1, keepdims=True)
    w = np.where(visible, np.exp(zm - m), 0.0)
    return w / w.sum(axis=-1, keepdims=True)


def kv_head_for(h: int, num_heads: int, num_kv_heads: int) -> int:
    """GQA: consecutive groups of H/Hkv query heads share one KV head
    ([P1] §2: 28 query heads over 4 KV heads, seven per group)."""
    return h // (num_heads // num_kv_heads)


def default_scale(head_dim: int) -> float:
    """Softmax scaling head_dim ** -0.5 ([P1] §2: 1/sqrt(128) for Qwen2-7B)."""
    return float(head_dim) ** -0.5


def attention_varlen(q, k_cache, v_cache, cu_seqlens_q, context_lens, block_tables,
                     num_heads, num_kv_heads, head_dim, block_size, dtype,
                     scale=None, return_probs=False, cache_dtype=None, k_scale=1.0,
                     v_scale=1.0):
    """Causal GQA attention of packed query rows over the paged cache.

    q: storage [T][H][d] (already rotated).  Sequence s owns rows
    cu_seqlens_q[s]..cu_seqlens_q[s+1] and context_lens[s] keys (the new rows
    included).  Head h reads KV head g = h // (H / Hkv) ([P1] §2: seven
    query heads share one KV group).  Scores z = scale * <q_h, K_j> with
    scale = head_dim ** -0.5 ([P1] §2 / [P2] §4.1 scaling); output
    o = sum_j pi_j V_j.  Returns float64 [T][H][d] (and the probabilities per
    sequence and head when return_probs)."""
    H, Hkv, d = num_heads, num_kv_heads, head_dim
    if scale is None:
        scale = default_scale(d)
    qf = to_f64(q, dtype).reshape(-1, H, d)
    out = np.zeros(qf.shape, dtype=np.float64)
    probs = []
    cu = np.asarray(cu_seqlens_q)
    for s in range(len(cu) - 1):
        r0, r1 = int(cu[s]), int(cu[s + 1])
        n, c = r1 - r0, int(context_lens[s])
        if n == 0:
            probs.append(None)
            continue
        K, V = gather_kv(k_cache, v_cache, block_tables[s], c, block_size, dtype,
                         cache_dtype, k_scale, v_scale)
        vis = causal_visible(n, c)
        ps = []
        for h in range(H):
            g = kv_head_for(h, H, Hkv)
            z = scale * (qf[r0:r1, h, :] @ K[:, g, :].T)          # [n][c]
            pi = softmax_rows(z, vis)
            out[r0:r1, h, :] = pi @ V[:, g, :]
            if return_probs:
                ps.append(pi)
        probs.append(ps if return_probs else None)
    if return_probs:
        return out, probs
    return out


def attention_decode(q, k_cache, v_cache, block_tables, context_lens,
                     num_heads, num_kv_heads, head_dim, block_size, dtype, scale=None,
                     cache_dtype=None, k_scale=1.0, v_scale=1.0):
    """Single-token decode: one query row per sequence at position c - 1,
    attending to all c cached keys (its own key included, written before the
    attention) -- [P3] §2.1 PagedAttention.  The same definition as
    attention_varlen with one row per sequence."""
    S = len(context_lens)
    cu = np.arange(S + 1, dtype=np.int64)
    return attention_varlen(q, k_cache, v_cache, cu, context_lens, block_tables,
                            num_heads, num_kv_heads, head_dim, block_size, dtype, scale,
                            cache_dtype=cache_dtype, k_scale=k_scale, v_scale=v_scale)


def check_prefix_groups(block_tables, context_lens, prefix_indptr, prefix_seqs, prefix_lens,
                        block_size):
    """The contract of a shared-prefix grouping: group p's members are
    prefix_seqs[prefix_indptr[p]:prefix_indptr[p+1]], its prefix is the first
    prefix_lens[p] tokens (whole blocks) of every member, held in the same
    physical blocks (prefix caching shares block ids, [P1] §3), and every
    member has at least one private key after it (its new token).  A sequence
    belongs to at most one group.  Raises ValueError otherwise."""
    ind = np.asarray(prefix_indptr, np.int64)
    seqs = np.asarray(prefix_seqs, np.int64)
    lens = np.asarray(prefix_lens, np.int64)
    S, B = len(context_lens), int(block_size)
    if ind.ndim != 1 or len(ind) != len(lens) + 1 or ind[0] != 0 or np.any(np.diff(ind) < 0) \
            or ind[-1] != len(seqs):
        raise ValueError("prefix_indptr must rise from 0 to len(prefix_seqs)")
    if len(np.unique(seqs)) != len(seqs) or np.any(seqs < 0) or np.any(seqs >= S):
        raise ValueError("a member is out of range or listed twice")
    for p in range(len(lens)):
        members = seqs[ind[p]:ind[p + 1]]
        L = int(lens[p])
        if L < 0 or L % B:
            raise ValueError(f"group {p}: prefix length {L} is not a whole number of blocks")
        if len(members) == 0:
            continue
        ids = np.asarray(block_tables[members[0]])[:L // B]
        for s in members:
            if L >= int(context_lens[s]):
                raise ValueError(f"group {p}: member {s} has no key after the prefix")
            if not np.array_equal(np.asarray(block_tables[s])[:L // B], ids):
                raise ValueError(f"group {p}: member {s} does not hold the shared prefix blocks")


def _partial_state(q, K, V, scale):
    """Softmax partial state of one query over a set of keys: reference
    maximum m, normaliser l = sum_j e^(z_j - m), unnormalised output
    a = sum_j e^(z_j - m) V_j, with z_j = scale <q, K_j>."""
    z = scale * (K @ q)
    m = z.max()
    w = np.exp(z - m)
    return m, w.sum(), w @ V


def attention_decode_cascade(q, k_cache, v_cache, block_tables, context_lens, prefix_indptr,
                             prefix_seqs, prefix_lens, num_heads, num_kv_heads, head_dim,
                             block_size, dtype, scale=None, cache_dtype=None, k_scale=1.0,
                             v_scale=1.0):
    """Decode attention evaluated as a two-level cascade.

    For each group p (see check_prefix_groups) the L_p shared prefix keys
    are gathered once, through the first member's block table, and every
    member's query heads are attended to them: partial state (m1, l1, a1).
    Each member's private keys L_p..c-1 give (m2, l2, a2).  Softmax over the
    union of two disjoint key sets is the merge
        M = max(m1, m2),  o = (a1 e^(m1-M) + a2 e^(m2-M)) / (l1 e^(m1-M) + l2 e^(m2-M)).
    Sequences in no group are attended as in attention_decode.  Returns
    float64 [S][H][d]."""
    H, Hkv, d, B = num_heads, num_kv_heads, head_dim, int(block_size)
    if scale is None:
        scale = default_scale(d)
    check_prefix_groups(block_tables, context_lens, prefix_indptr, prefix_seqs, prefix_lens, B)
    out = attention_decode(q, k_cache, v_cache, block_tables, context_lens, H, Hkv, d, B, dtype,
                           scale, cache_dtype=cache_dtype, k_scale=k_scale, v_scale=v_scale)
    qf = to_f64(q, dtype).reshape(-1, H, d)
    ind = np.asarray(prefix_indptr, np.int64)
    seqs = np.asarray(prefix_seqs, np.int64)
    for p in range(len(ind) - 1):
        members = seqs[ind[p]:ind[p + 1]]
        L = int(prefix_lens[p])
        if len(members) == 0 or L == 0:
            continue
        # the shared prefix, gathered once for the whole group
        Kp, Vp = gather_kv(k_cache, v_cache, block_tables[members[0]], L, B, dtype,
                           cache_dtype, k_scale, v_scale)
        for s in members:
            c = int(context_lens[s])
            # the member's own keys after the prefix
            K, V = gather_kv(k_cache, v_cache, block_tables[s], c, B, dtype, cache_dtype,
                             k_scale, v_scale)
            Ks, Vs = K[L:], V[L:]
            for h in range(H):
                g = kv_head_for(h, H, Hkv)
                m1, l1, a1 = _partial_state(qf[s, h], Kp[:, g, :], Vp[:, g, :], scale)
                m2, l2, a2 = _partial_state(qf[s, h], Ks[:, g, :], Vs[:, g, :], scale)
                M = max(m1, m2)
                e1, e2 = np.exp(m1 - M), np.exp(m2 - M)
                out[s, h] = (a1 * e1 + a2 * e2) / (l1 * e1 + l2 * e2)
    return out


def run_step(batch, k_cache=None, v_cache=None):
    """The whole step for a workload batch: rope + cache write over every
    token, then prefill attention over the prefill sequences and decode
    attention over the rest.  Returns dict(q_out, k_cache, v_cache, out) with
    ``out`` float64 [T][H][d] (rows in token order)."""
    sh = batch.shape
    kc0 = batch.k_cache if k_cache is None else k_cache
    vc0 = batch.v_cache if v_cache is None else v_cache
    cd = getattr(sh, "cache_dtype", None)
    ks, vs = getattr(sh, "k_scale", 1.0), getattr(sh, "v_scale", 1.0)
    qn, kn = getattr(batch, "q_norm_weight", None), getattr(batch, "k_norm_weight", None)
    q_out, kc, vc = rope_cache_write(batch.qkv, sh.dtype, batch.positions, batch.slot_mapping,
                                     kc0, vc0, sh.num_heads, sh.num_kv_heads, sh.head_dim,
                                     sh.block_size, sh.rope_theta, cd, ks, vs, qn, kn,
                                     getattr(sh, "rms_eps", 1e-6))
    out = attention_varlen(q_out, kc, vc, batch.cu_seqlens_q, batch.context_lens,
                           batch.block_tables, sh.num_heads, sh.num_kv_heads, sh.head_dim,
                           sh.block_size, sh.dtype, cache_dtype=cd, k_scale=ks, v_scale=vs)
    return {"q_out": q_out, "k_cache": kc, "v_cache": vc, "out": out}
