"""Seeded synthetic inputs for the paged GQA attention path.

This module only builds inputs: shapes, lengths, block tables, slot mappings
and the contents of the paged KV pool *before* a step runs.  It performs none
of the attention arithmetic (no rotation, no softmax, no reduction); both the
HIP path and the CPU oracle consume what it produces.

Shapes follow the model configurations the pages print:
  * Qwen2-7B: hidden 3584, 28 query heads, 4 KV heads, so head_dim 128 and a
    GQA group of 7; rope_theta 1e6; max_position_embeddings 32768
    ("Qwen2 model structure explained in vLLM", section 2, config JSON).
  * Qwen3-0.6B: 16 query heads, 8 KV heads, head_dim 128
    ("nano-vllm ... Qwen3 skeleton", section 2, configuration table).
  * Tensor-parallel share at TP=2: 14 query heads, 2 KV heads (same page as
    Qwen2-7B, section 2, head split rule).
  * Request lengths 128..512 for the prefill batch follow the length spread
    used in the continuous-batching measurement ("vLLM deployment of Qwen",
    section 2.1).
  * KV cache in fixed-size blocks of 16 tokens (the vLLM `--block-size`
    default; same page, section 5.1).

Cache layouts (an interface definition, identical for every consumer):
  * K cache: ``[num_blocks][num_kv_heads][block_size][head_dim]``
  * V cache: ``[num_blocks][num_kv_heads][head_dim][block_size]``
A token at logical position ``p`` of a sequence lives in physical block
``block_table[p // B]`` at offset ``p % B``; its slot number is
``block * B + offset``.

Values are stored as raw storage bits: bf16 as ``uint16`` arrays, fp32 as
``float32`` arrays, an FP8 cache as ``uint8`` E4M3FN codes (torch's
float8_e4m3fn conversion of the drawn value divided by the cache's scale).
Unused blocks, and slots past a sequence's context, hold NaN (code 0x7f in an
FP8 cache) so that any read outside the context shows up in the output.

Draw order for every workload (one ``numpy.random.default_rng(seed)``):
lengths -> prefix-sharing choices -> block permutation -> fused QKV rows ->
pre-existing cache contents (K then V, sequence by sequence, shared prefix
first).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

BF16_NAN_BITS = np.uint16(0x7FC0)
F32_NAN = np.float32("nan")
FP8_NAN_CODE = np.uint8(0x7F)

DTYPES = ("bf16", "f32")


# --------------------------------------------------------------------------
# storage helpers (plain data conversion; no method arithmetic)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even); return uint16 bits."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 exactly."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def storage_nan(dtype: str):
    return {"bf16": BF16_NAN_BITS, "f32": F32_NAN, "fp8": FP8_NAN_CODE}[dtype]


def storage_np_dtype(dtype: str):
    return {"bf16": np.uint16, "f32": np.float32, "fp8": np.uint8}[dtype]


def to_fp8_codes(x: np.ndarray, scale: float) -> np.ndarray:
    """Synthetic FP8 cache contents: float32 values divided by the scale,
    clamped to the finite range and converted with torch's float8_e4m3fn."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)) / float(scale)
    return t.clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def normal_storage(rng: np.random.Generator, shape, scale: float, dtype: str) -> np.ndarray:
    """N(0,1) * scale drawn in float32, then stored in ``dtype``.

    Each call takes one 63-bit seed from ``rng`` and draws the array with a
    torch CPU generator (several times faster than numpy for the large pools)."""
    seed = int(rng.integers(0, 2**63 - 1))
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(tuple(int(v) for v in np.atleast_1d(shape)) if not isinstance(shape, tuple) else shape,
                    generator=g, dtype=torch.float32)
    if scale != 1.0:
        x.mul_(float(scale))
    if dtype == "bf16":
        return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return x.numpy()


# --------------------------------------------------------------------------
# workload description
# --------------------------------------------------------------------------
@dataclass
class AttnShape:
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int = 16
    dtype: str = "bf16"
    rope_theta: float = 1.0e6
    max_position: int = 32768
    cache_dtype: Optional[str] = None   # None: the caches use `dtype`; "fp8": E4M3FN codes
    k_scale: float = 1.0                # FP8 cache: value = code * scale
    v_scale: float = 1.0
    rms_eps: float = 1e-6               # Qwen3 q/k norm epsilon (when the batch has weights)
    # dynamic-NTK rope scaling (factor, original_max_position), or None; the
    # table then has max_position = floor(factor * original) rows
    rope_scaling: Optional[tuple] = None

    @property
    def group(self) -> int:
        return self.num_heads // self.num_kv_heads

    @property
    def qkv_width(self) -> int:
        return (self.num_heads + 2 * self.num_kv_heads) * self.head_dim

    @property
    def scale(self) -> float:
        # head_dim ** -0.5, the softmax scaling the attention layer is built with
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    @property
    def cache_storage(self) -> str:
        return self.cache_dtype or self.dtype

    @property
    def cache_elem_bytes(self) -> int:
        return 1 if self.cache_dtype == "fp8" else self.elem_bytes


@dataclass
class Batch:
    """One step's inputs.  Sequences ``[0, num_prefill)`` are prefill chunks
    (query rows ``cu_seqlens_q[s]..cu_seqlens_q[s+1]``); the remaining
    sequences are single-token decodes whose query rows follow the prefill
    rows in the same order."""

    name: str
    shape: AttnShape
    qkv: np.ndarray            # [T][(H+2Hkv)*d] storage
    positions: np.ndarray      # int32 [T]
    slot_mapping: np.ndarray   # int32 [T]
    k_cache: np.ndarray        # [nb][Hkv][B][d] storage (state before the step)
    v_cache: np.ndarray        # [nb][Hkv][d][B] storage
    block_tables: np.ndarray   # int32 [S][max_blocks]
    context_lens: np.ndarray   # int32 [S] (includes this step's tokens)
    query_lens: np.ndarray     # int32 [S]
    num_prefill: int
    poison_block: int
    shared_prefix_blocks: int = 0
    seed: int = 0
    # logical pre-existing K/V per sequence ([m][Hkv][d] storage); only kept on request
    pre_k: Optional[List[np.ndarray]] = None
    pre_v: Optional[List[np.ndarray]] = None
    notes: dict = field(default_factory=dict)
    # Qwen3 q/k norm weights ([head_dim], step dtype), or None
    q_norm_weight: Optional[np.ndarray] = None
    k_norm_weight: Optional[np.ndarray] = None
    # shared prefixes of the decode sequences: (indptr [P+1], members
    # (decode-local indices), prefix lengths in tokens [P]), or None
    prefix_groups: Optional[tuple] = None

    # ---- derived views ----
    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.qkv.shape[0])

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def cu_seqlens_q(self) -> np.ndarray:
        cu = np.zeros(self.num_seqs + 1, dtype=np.int32)
        cu[1:] = np.cumsum(self.query_lens)
        return cu

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def num_prefill_tokens(self) -> int:
        return int(self.query_lens[: self.num_prefill].sum())

    @property
    def num_decode(self) -> int:
        return self.num_seqs - self.num_prefill

    def prefill_part(self):
        """(cu_seqlens_q, context_lens, block_tables) of the prefill sequences."""
        p = self.num_prefill
        cu = np.zeros(p + 1, dtype=np.int32)
        cu[1:] = np.cumsum(self.query_lens[:p])
        return cu, self.context_lens[:p].copy(), self.block_tables[:p].copy()

    def decode_part(self):
        """(context_lens, block_tables) of the decode sequences."""
        p = self.num_prefill
        return self.context_lens[p:].copy(), self.block_tables[p:].copy()

    # ---- algorithmic work (what the method must move / compute) ----
    def decode_kv_bytes(self) -> int:
        sh = self.shape
        c = self.context_lens[self.num_prefill:].astype(np.int64)
        return int(c.sum()) * 2 * sh.num_kv_heads * sh.head_dim * sh.cache_elem_bytes

    def decode_bytes(self) -> int:
        """KV read once per KV head + q read + out written + block-table rows + context lens."""
        sh = self.shape
        c = self.context_lens[self.num_prefill:].astype(np.int64)
        nd = self.num_decode
        qo = 2 * nd * sh.num_heads * sh.head_dim * sh.elem_bytes
        bt = 4 * int(((c + sh.block_size - 1) // sh.block_size).sum()) + 4 * nd
        return self.decode_kv_bytes() + qo + bt

    def decode_cascade_bytes(self) -> int:
        """decode_bytes with every group's shared prefix read once per KV head
        instead of once per member (the block-table entries likewise)."""
        if self.prefix_groups is None:
            return self.decode_bytes()
        sh = self.shape
        ind, members, lens = self.prefix_groups
        per_token = 2 * sh.num_kv_heads * sh.head_dim * sh.cache_elem_bytes
        saved = 0
        for p in range(len(lens)):
            m = int(ind[p + 1] - ind[p])
            if m > 1:
                L = int(lens[p])
                saved += (m - 1) * (L * per_token + 4 * (L // sh.block_size))
        return self.decode_bytes() - saved

    def prefill_flops(self) -> int:
        """4*d*H per unmasked (query, key) pair: QK^T and PV, causal entries only."""
        sh = self.shape
        tot = 0
        for s in range(self.num_prefill):
            n = int(self.query_lens[s])
            c = int(self.context_lens[s])
            # row i sees keys 0..c-n+i  -> (c - n + i + 1) keys
            tot += n * (c - n + 1) + n * (n - 1) // 2
        return 4 * sh.head_dim * sh.num_heads * tot

    def rope_write_bytes(self) -> int:
        sh = self.shape
        t = self.num_tokens
        e = sh.elem_bytes
        d = sh.head_dim
        return (t * sh.qkv_width * e + t * sh.num_heads * d * e
                + t * 2 * sh.num_kv_heads * d * sh.cache_elem_bytes + 8 * t)


# --------------------------------------------------------------------------
# builder
# --------------------------------------------------------------------------
def _build(name: str, shape: AttnShape, seed: int, rng: np.random.Generator,
           context_lens: np.ndarray, query_lens: np.ndarray, num_prefill: int,
           shares_prefix: np.ndarray, shared_prefix_len: int, value_scale: float,
           pool_size: Optional[int] = None, keep_logical: bool = False) -> Batch:
    B = shape.block_size
    Hkv, d, dt = shape.num_kv_heads, shape.head_dim, shape.dtype
    S = int(context_lens.shape[0])
    assert shared_prefix_len % B == 0
    spb = shared_prefix_len // B

    blocks_per_seq = (context_lens + B - 1) // B
    private = np.where(shares_prefix, blocks_per_seq - spb, blocks_per_seq).astype(np.int64)
    assert (private >= 0).all()
    needed = spb + int(private.sum())
    if pool_size is None:
        pool_size = int(math.ceil(1.25 * needed))
    assert pool_size > needed, "pool must keep at least one unused (poison) block"

    ids = rng.permutation(pool_size).astype(np.int32)
    shared_ids = ids[:spb]
    poison = int(ids[needed])
    max_blocks = int(blocks_per_seq.max())
    bt = np.full((S, max_blocks), poison, dtype=np.int32)
    nxt = spb
    for s in range(S):
        start = 0
        if shares_prefix[s]:
            bt[s, :spb] = shared_ids
            start = spb
        cnt = int(blocks_per_seq[s]) - start
        bt[s, start:start + cnt] = ids[nxt:nxt + cnt]
        nxt += cnt
    assert nxt == needed

    # query rows: prefill rows first, then one row per decode sequence
    T = int(query_lens.sum())
    qkv = normal_storage(rng, (T, shape.qkv_width), value_scale, dt)
    positions = np.empty(T, dtype=np.int32)
    slots = np.empty(T, dtype=np.int32)
    row = 0
    for s in range(S):
        n, c = int(query_lens[s]), int(context_lens[s])
        p = np.arange(c - n, c, dtype=np.int64)
        positions[row:row + n] = p
        slots[row:row + n] = bt[s, p // B].astype(np.int64) * B + p % B
        row += n

    # pool, NaN everywhere, then the context that earlier steps left behind
    cdt = shape.cache_storage
    k_cache = np.full((pool_size, Hkv, B, d), storage_nan(cdt), dtype=storage_np_dtype(cdt))
    v_cache = np.full((pool_size, Hkv, d, B), storage_nan(cdt), dtype=storage_np_dtype(cdt))

    def draw_kv(shape3):
        """Pre-existing context rows: (k, v) in the cache's storage, plus the
        logical values in the step dtype when the cache is FP8."""
        if cdt != "fp8":
            kk = normal_storage(rng, shape3, value_scale, dt)
            vv = normal_storage(rng, shape3, value_scale, dt)
            return kk, vv, kk, vv
        kf = normal_storage(rng, shape3, value_scale, "f32")
        vf = normal_storage(rng, shape3, value_scale, "f32")
        return to_fp8_codes(kf, shape.k_scale), to_fp8_codes(vf, shape.v_scale), kf, vf

    def put(block_ids: np.ndarray, pos: np.ndarray, kv: np.ndarray, vv: np.ndarray):
        """Place logical rows kv/vv ([m][Hkv][d], positions pos[0].. contiguous,
        pos[0] a multiple of B) into their blocks; the tail of the last block
        stays NaN."""
        m = kv.shape[0]
        if m == 0:
            return
        assert pos[0] % B == 0
        nblk = (m + B - 1) // B
        blk = block_ids[pos[0] // B: pos[0] // B + nblk]
        pad = nblk * B - m
        if pad:
            fill = np.full((pad, Hkv, d), storage_nan(cdt), dtype=kv.dtype)
            kv = np.concatenate([kv, fill])
            vv = np.concatenate([vv, fill])
        kb = kv.reshape(nblk, B, Hkv, d)
        vb = vv.reshape(nblk, B, Hkv, d)
        k_cache[blk] = kb.transpose(0, 2, 1, 3)
        v_cache[blk] = vb.transpose(0, 2, 3, 1)

    pre_k: List[np.ndarray] = []
    pre_v: List[np.ndarray] = []
    shared_k = shared_v = None
    if spb:
        pos = np.arange(shared_prefix_len, dtype=np.int64)
        sk, sv, shared_k, shared_v = draw_kv((shared_prefix_len, Hkv, d))
        put(shared_ids.astype(np.int64), pos, sk, sv)
    for s in range(S):
        n, c = int(query_lens[s]), int(context_lens[s])
        m = c - n
        start = shared_prefix_len if shares_prefix[s] else 0
        assert m >= start or m == 0 or not shares_prefix[s]
        cnt = max(0, m - start)
        pos = np.arange(start, start + cnt, dtype=np.int64)
        kc_, vc_, kk, vv = draw_kv((cnt, Hkv, d))
        if cnt:
            put(bt[s].astype(np.int64), pos, kc_, vc_)
        if keep_logical:
            if start:
                pre_k.append(np.concatenate([shared_k[:min(m, start)], kk]))
                pre_v.append(np.concatenate([shared_v[:min(m, start)], vv]))
            else:
                pre_k.append(kk)
                pre_v.append(vv)

    return Batch(name=name, shape=shape, qkv=qkv, positions=positions, slot_mapping=slots,
                 k_cache=k_cache, v_cache=v_cache, block_tables=bt,
                 context_lens=context_lens.astype(np.int32), query_lens=query_lens.astype(np.int32),
                 num_prefill=num_prefill, poison_block=poison, shared_prefix_blocks=spb, seed=seed,
                 pre_k=pre_k if keep_logical else None, pre_v=pre_v if keep_logical else None,
                 prefix_groups=_one_group(shares_prefix[num_prefill:], shared_prefix_len))


def _one_group(dec_share: np.ndarray, prefix_len: int):
    """The decode sequences holding the shared prefix as one prefix group
    (decode-local indices), or None."""
    members = np.flatnonzero(np.asarray(dec_share, bool)).astype(np.int32)
    if prefix_len == 0 or len(members) == 0:
        return None
    return (np.array([0, len(members)], np.int32), members, np.array([prefix_len], np.int32))


# --------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------
def tiny_f32_steps(seed: int = 1) -> List[Batch]:
    """Tiny fp32 GQA: one sequence, a 16-token causal prefill (positions 0..15)
    then 4 single-token decode steps (positions 16..19); 4 q heads, 2 KV heads,
    head_dim 64, block 16, a 4-block pool whose physical ids are permuted.

    Returns the 5 steps in order.  Every step carries the same initial (all-NaN)
    pool; a runner must thread each step's output cache into the next step."""
    shape = AttnShape(num_heads=4, num_kv_heads=2, head_dim=64, block_size=16, dtype="f32")
    rng = np.random.default_rng(seed)
    B = shape.block_size
    ids = rng.permutation(4).astype(np.int32)
    while ids[0] == 0 and ids[1] == 1:          # redraw an identity logical->physical map
        ids = rng.permutation(4).astype(np.int32)
    bt = ids[None, :2].copy()                   # logical blocks 0, 1
    poison = int(ids[2])
    qkv = normal_storage(rng, (20, shape.qkv_width), 1.0, "f32")
    k_cache = np.full((4, 2, B, 64), F32_NAN, dtype=np.float32)
    v_cache = np.full((4, 2, 64, B), F32_NAN, dtype=np.float32)

    def slots(pos):
        pos = np.asarray(pos, np.int64)
        return (bt[0, pos // B].astype(np.int64) * B + pos % B).astype(np.int32)

    p0 = np.arange(16, dtype=np.int32)
    steps = [Batch(name="tiny_f32_prefill16", shape=shape, qkv=qkv[:16].copy(), positions=p0,
                   slot_mapping=slots(p0), k_cache=k_cache, v_cache=v_cache, block_tables=bt.copy(),
                   context_lens=np.array([16], np.int32), query_lens=np.array([16], np.int32),
                   num_prefill=1, poison_block=poison, seed=seed,
                   pre_k=[k_cache[:0, 0, 0, :]], pre_v=[v_cache[:0, 0, :, 0]])]
    for k in range(4):
        p = np.array([16 + k], np.int32)
        steps.append(Batch(name=f"tiny_f32_decode{k}", shape=shape, qkv=qkv[16 + k:17 + k].copy(),
                           positions=p, slot_mapping=slots(p), k_cache=k_cache, v_cache=v_cache,
                           block_tables=bt.copy(), context_lens=np.array([17 + k], np.int32),
                           query_lens=np.array([1], np.int32), num_prefill=0,
                           poison_block=poison, seed=seed))
    return steps


def qwen3_decode(seed: int = 2, num_seqs: int = 32, keep_logical: bool = False) -> Batch:
    """Qwen3-0.6B-shaped decode, bf16: 16 q heads, 8 KV heads, head_dim 128,
    block 16; batch 32; context lengths uniform in [128, 2048]; values N(0,1)*0.5."""
    shape = AttnShape(num_heads=16, num_kv_heads=8, head_dim=128)
    rng = np.random.default_rng(seed)
    ctx = rng.integers(128, 2048, size=num_seqs, endpoint=True).astype(np.int32)
    return _build("qwen3_0.6b_decode_b32", shape, seed, rng, ctx, np.ones(num_seqs, np.int32), 0,
                  np.zeros(num_seqs, bool), 0, 0.5, keep_logical=keep_logical)


def qwen2_prefill(seed: int = 3, num_seqs: int = 8, keep_logical: bool = False) -> Batch:
    """Qwen2-7B-shaped varlen causal prefill, bf16: 28 q heads, 4 KV heads,
    head_dim 128; 8 packed sequences with lengths uniform in [128, 512];
    fresh (permuted) cache blocks written in the same step."""
    shape = AttnShape(num_heads=28, num_kv_heads=4, head_dim=128)
    rng = np.random.default_rng(seed)
    n = rng.integers(128, 512, size=num_seqs, endpoint=True).astype(np.int32)
    return _build("qwen2_7b_prefill_8x[128,512]", shape, seed, rng, n.copy(), n.copy(), num_seqs,
                  np.zeros(num_seqs, bool), 0, 1.0, keep_logical=keep_logical)


def qwen2_prefill_long_prefix(seed: int = 9, num_seqs: int = 8, keep_logical: bool = False) -> Batch:
    """Qwen2-7B-shaped chunked prefill, bf16: 28 q heads, 4 KV heads, head_dim
    128; 8 sequences, each a 256-row chunk after an 8192-token prefix already
    in the cache (positions 8192..8447): long key loops per query tile."""
    shape = AttnShape(num_heads=28, num_kv_heads=4, head_dim=128)
    rng = np.random.default_rng(seed)
    n = np.full(num_seqs, 256, np.int32)
    return _build("qwen2_7b_prefill_8x256_after_8192", shape, seed, rng, n + 8192, n, num_seqs,
                  np.zeros(num_seqs, bool), 0, 1.0, keep_logical=keep_logical)


def qwen3_prefill(seed: int = 8, num_seqs: int = 8, keep_logical: bool = False) -> Batch:
    """Qwen3-0.6B-shaped varlen causal prefill, bf16: 16 q heads, 8 KV heads
    (group 2), head_dim 128; 8 packed sequences with lengths uniform in
    [128, 512]; values N(0,1)*0.5 as in the Qwen3 decode workload."""
    shape = AttnShape(num_heads=16, num_kv_heads=8, head_dim=128)
    rng = np.random.default_rng(seed)
    n = rng.integers(128, 512, size=num_seqs, endpoint=True).astype(np.int32)
    return _build("qwen3_0.6b_prefill_8x[128,512]", shape, seed, rng, n.copy(), n.copy(), num_seqs,
                  np.zeros(num_seqs, bool), 0, 0.5, keep_logical=keep_logical)


def qwen2_long_decode(seed: int = 4, num_seqs: int = 64, keep_logical: bool = False) -> Batch:
    """Qwen2-7B-shaped long-context decode, bf16: 28 q heads, 4 KV heads,
    head_dim 128; batch 64; context lengths log-uniform in [2048, 32768]."""
    shape = AttnShape(num_heads=28, num_kv_heads=4, head_dim=128)
    rng = np.random.default_rng(seed)
    u = rng.uniform(math.log(2048), math.log(32768), size=num_seqs)
    ctx = np.clip(np.floor(np.exp(u)), 2048, 32768).astype(np.int32)
    return _build("qwen2_7b_decode_b64_ctx[2048,32768]", shape, seed, rng, ctx,
                  np.ones(num_seqs, np.int32), 0, np.zeros(num_seqs, bool), 0, 1.0,
                  keep_logical=keep_logical)


# FP8 cache scales of the FP8 workloads: with N(0,1) values the codes use
# the upper part of the E4M3FN range (|x| / scale up to ~180 < 448) and stay
# clear of its subnormals; deliberately not powers of two.  A cache scale is
# a float32 (the library's argument type), so these are the float32 values
# nearest 0.0312 and 0.0287: the oracle then divides by exactly the number
# the kernels receive (with the float64 0.0312 the two quotients differ by
# ~3e-8 relative, enough to move an occasional code across a rounding
# boundary).
FP8_K_SCALE = float(np.float32(0.0312))
FP8_V_SCALE = float(np.float32(0.0287))


def qwen2_long_decode_fp8(seed: int = 4, num_seqs: int = 64, keep_logical: bool = False) -> Batch:
    """The Qwen2-7B long-context decode with an FP8 (E4M3FN) KV cache: same
    lengths, rows and draws as the bf16 workload, the cache holding codes of
    value / scale (k_scale 0.0312, v_scale 0.0287)."""
    shape = AttnShape(num_heads=28, num_kv_heads=4, head_dim=128, cache_dtype="fp8",
                      k_scale=FP8_K_SCALE, v_scale=FP8_V_SCALE)
    rng = np.random.default_rng(seed)
    u = rng.uniform(math.log(2048), math.log(32768), size=num_seqs)
    ctx = np.clip(np.floor(np.exp(u)), 2048, 32768).astype(np.int32)
    return _build("qwen2_7b_decode_b64_ctx[2048,32768]_fp8kv", shape, seed, rng, ctx,
                  np.ones(num_seqs, np.int32), 0, np.zeros(num_seqs, bool), 0, 1.0,
                  keep_logical=keep_logical)


def qwen2_prefill_fp8(seed: int = 3, num_seqs: int = 8, keep_logical: bool = False) -> Batch:
    """The Qwen2-7B varlen causal prefill with an FP8 (E4M3FN) KV cache: same
    lengths, rows and draws as the bf16 workload, the cache written as codes
    of value / scale (k_scale 0.0312, v_scale 0.0287)."""
    shape = AttnShape(num_heads=28, num_kv_heads=4, head_dim=128, cache_dtype="fp8",
                      k_scale=FP8_K_SCALE, v_scale=FP8_V_SCALE)
    rng = np.random.default_rng(seed)
    n = rng.integers(128, 512, size=num_seqs, endpoint=True).astype(np.int32)
    return _build("qwen2_7b_prefill_8x[128,512]_fp8kv", shape, seed, rng, n.copy(), n.copy(),
                  num_seqs, np.zeros(num_seqs, bool), 0, 1.0, keep_logical=keep_logical)


def mixed_tp2(seed: int = 5, keep_logical: bool = False) -> Batch:
    """Mixed chunked batch at the TP=2 share of Qwen2-7B, bf16: 14 q heads,
    2 KV heads, head_dim 128.  4 prefill chunks of 512 tokens (2 continue a
    shared 1024-token prefix: positions 1024..1535; 2 start fresh: 0..511) plus
    96 decode tokens with contexts uniform in [256, 8192], 48 of which share
    the same 1024-token prefix (shared physical block ids)."""
    shape = AttnShape(num_heads=14, num_kv_heads=2, head_dim=128)
    rng = np.random.default_rng(seed)
    prefix = 1024
    dec_ctx = rng.integers(256, 8192, size=96, endpoint=True).astype(np.int32)
    eligible = np.flatnonzero(dec_ctx > prefix)
    share_dec = np.zeros(96, bool)
    share_dec[rng.choice(eligible, size=48, replace=False)] = True
    pre_ctx = np.array([1536, 1536, 512, 512], np.int32)
    pre_share = np.array([True, True, False, False])
    ctx = np.concatenate([pre_ctx, dec_ctx])
    qlen = np.concatenate([np.full(4, 512, np.int32), np.ones(96, np.int32)])
    share = np.concatenate([pre_share, share_dec])
    return _build("qwen2_7b_tp2_mixed_4x512+96", shape, seed, rng, ctx, qlen, 4, share, prefix, 1.0,
                  keep_logical=keep_logical)


def qwen2_131k_decode(seed: int = 6, num_seqs: int = 8, keep_logical: bool = False) -> Batch:
    """Qwen2-7B decode past the native window with dynamic-NTK rope scaling
    (factor 4 over 32768 positions: a 131072-row table), bf16: 28 q heads,
    4 KV heads, head_dim 128, block 16; batch 8, contexts uniform in
    [65536, 131072]."""
    shape = AttnShape(num_heads=28, num_kv_heads=4, head_dim=128, rope_scaling=(4.0, 32768),
                      max_position=131072)
    rng = np.random.default_rng(seed)
    ctx = rng.integers(65536, 131072, size=num_seqs, endpoint=True).astype(np.int32)
    return _build("qwen2_7b_131k_decode_b8", shape, seed, rng, ctx, np.ones(num_seqs, np.int32), 0,
                  np.zeros(num_seqs, bool), 0, 1.0, keep_logical=keep_logical)


def with_qk_norm(b: Batch, seed: int) -> Batch:
    """Attach Qwen3 q/k norm weights: N(1, 0.1^2) per element (learned RMSNorm
    weights sit around 1), drawn from their own generator so the batch's
    other draws are unchanged."""
    rng = np.random.default_rng([seed, 0x51CE])
    d, dt = b.shape.head_dim, b.shape.dtype
    b.q_norm_weight = normal_storage(rng, (d,), 0.1, "f32") + np.float32(1.0)
    b.k_norm_weight = normal_storage(rng, (d,), 0.1, "f32") + np.float32(1.0)
    if dt == "bf16":
        b.q_norm_weight = f32_to_bf16_bits(b.q_norm_weight)
        b.k_norm_weight = f32_to_bf16_bits(b.k_norm_weight)
    return b


def qwen3_decode_qknorm(seed: int = 2, num_seqs: int = 32, keep_logical: bool = False) -> Batch:
    """The Qwen3-0.6B decode with its q/k RMSNorm (weights N(1, 0.1^2), eps
    1e-6) fused into the cache write."""
    return with_qk_norm(qwen3_decode(seed, num_seqs, keep_logical), seed)


def with_prefix_groups(b: Batch, groups) -> Batch:
    """Make decode sequences share prefixes, as prefix caching does: groups
    is a list of (members, prefix_len) with members decode-local indices and
    prefix_len a multiple of the block size, below every member's context.
    Each member's first prefix_len / block_size block ids become those of
    the group's first member (the blocks they named before stay in the pool,
    unreferenced).  Records the grouping in b.prefix_groups."""
    B, P = b.shape.block_size, b.num_prefill
    ind, seqs, lens = [0], [], []
    for members, L in groups:
        assert L % B == 0
        members = [int(m) for m in members]
        first = b.block_tables[P + members[0], : L // B].copy()
        for m in members:
            assert L < int(b.context_lens[P + m])
            b.block_tables[P + m, : L // B] = first
        seqs.extend(members)
        lens.append(L)
        ind.append(len(seqs))
    b.prefix_groups = (np.array(ind, np.int32), np.array(seqs, np.int32), np.array(lens, np.int32))
    b.pre_k = b.pre_v = None
    return b


def shared_prompt_decode(seed: int = 7, num_groups: int = 4, members_per_group: int = 16,
                         prefix_len: int = 4096, keep_logical: bool = False) -> Batch:
    """Qwen2-7B decode, bf16, where sequences share long system prompts:
    num_groups groups of members_per_group sequences, each group holding one
    prefix_len-token prefix (shared block ids), private suffixes uniform in
    [256, 2048] tokens after it.  28 q heads, 4 KV heads, head_dim 128,
    block 16."""
    shape = AttnShape(num_heads=28, num_kv_heads=4, head_dim=128)
    rng = np.random.default_rng(seed)
    S = num_groups * members_per_group
    ctx = (prefix_len + rng.integers(256, 2048, size=S, endpoint=True)).astype(np.int32)
    b = _build(f"qwen2_7b_shared_prompt_{num_groups}x{members_per_group}_p{prefix_len}", shape,
               seed, rng, ctx, np.ones(S, np.int32), 0, np.zeros(S, bool), 0, 1.0,
               keep_logical=keep_logical)
    groups = [(list(range(g * members_per_group, (g + 1) * members_per_group)), prefix_len)
              for g in range(num_groups)]
    return with_prefix_groups(b, groups)


def small_case(seed: int, dtype: str, num_heads: int, num_kv_heads: int, head_dim: int,
               context_lens, query_lens, num_prefill: int, block_size: int = 16,
               value_scale: float = 1.0, keep_logical: bool = True, shares_prefix=None,
               shared_prefix_len: int = 0, cache_dtype=None, k_scale: float = 1.0,
               v_scale: float = 1.0, qk_norm: bool = False, rope_scaling=None) -> Batch:
    """A custom small batch (tests): explicit lengths, any head layout."""
    shape = AttnShape(num_heads=num_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                      block_size=block_size, dtype=dtype, cache_dtype=cache_dtype,
                      k_scale=k_scale, v_scale=v_scale)
    if rope_scaling is not None:
        shape.rope_scaling = (float(rope_scaling[0]), int(rope_scaling[1]))
        shape.max_position = int(rope_scaling[0] * rope_scaling[1])
    rng = np.random.default_rng(seed)
    ctx = np.asarray(context_lens, np.int32)
    ql = np.asarray(query_lens, np.int32)
    sh = np.zeros(len(ctx), bool) if shares_prefix is None else np.asarray(shares_prefix, bool)
    b = _build(f"small_{dtype}_s{seed}", shape, seed, rng, ctx, ql, num_prefill, sh,
               shared_prefix_len, value_scale, keep_logical=keep_logical)
    return with_qk_norm(b, seed) if qk_norm else b


WORKLOADS = {
    "tiny_f32": tiny_f32_steps,
    "qwen3_decode": qwen3_decode,
    "qwen2_prefill": qwen2_prefill,
    "qwen2_prefill_long_prefix": qwen2_prefill_long_prefix,
    "qwen2_long_decode": qwen2_long_decode,
    "mixed_tp2": mixed_tp2,
    "qwen2_long_decode_fp8": qwen2_long_decode_fp8,
    "qwen3_decode_qknorm": qwen3_decode_qknorm,
    "qwen2_131k_decode": qwen2_131k_decode,
    "shared_prompt_decode": shared_prompt_decode,
}
