"""Run one attention step of a workload batch through the C ABI.

Uploads a ``workloads.Batch`` to device memory (torch tensors) and calls
``qwen2_rope_cache_write`` over every token, then
``qwen2_attn_prefill_varlen`` over the prefill sequences and
``qwen2_attn_decode_paged`` (or, with cascade=True and prefix groups,
``qwen2_attn_decode_paged_cascade``) over the decode sequences, all on the
current stream.  Only marshalling: the arithmetic happens in the HIP library.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as B

_TABLES = {}


def to_device(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Storage array (uint16 bf16 bits, float32, or uint8 FP8 codes) -> device tensor."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    if dtype == "fp8":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def to_host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> storage array (uint16 bits for bf16)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def rope_table(head_dim: int, theta: float, max_position: int, device="cuda",
               rope_scaling=None) -> torch.Tensor:
    """The device cos/sin table; with rope_scaling = (factor, original) the
    dynamic-NTK table of floor(factor * original) rows."""
    key = (head_dim, float(theta), int(max_position), str(device),
           None if rope_scaling is None else tuple(rope_scaling))
    t = _TABLES.get(key)
    if t is None:
        if rope_scaling is None:
            t = torch.empty(max_position, head_dim, dtype=torch.float64, device=device)
            B.qwen2_rope_table_init(t, theta)
        else:
            factor, original = rope_scaling
            n = B.qwen2_rope_dynamic_ntk_positions(original, factor)
            if n != max_position:
                raise ValueError(f"max_position {max_position} != scaled table rows {n}")
            t = torch.empty(n, head_dim, dtype=torch.float64, device=device)
            B.qwen2_rope_table_init_dynamic_ntk(t, original, factor, theta)
        _TABLES[key] = t
    return t


def use_cascade(batch, cascade) -> bool:
    """Whether the decode of `batch` goes through the cascade entry point:
    never without prefix groups; always for cascade=True; for "auto", when
    the library expects it to pay (qwen2_attn_decode_cascade_worthwhile)."""
    if not cascade or batch.prefix_groups is None:
        return False
    if cascade != "auto":
        return True
    sh = batch.shape
    ind, seqs, lens = batch.prefix_groups
    return B.qwen2_attn_decode_cascade_worthwhile(
        len(lens), len(seqs), int(np.max(lens)) if len(lens) else 0, sh.num_kv_heads,
        sh.head_dim, sh.cache_storage == "fp8")


class DeviceStep:
    """Device copies of one batch plus the calls of the step."""

    def __init__(self, batch, device="cuda", k_cache=None, v_cache=None, cascade=False):
        """cascade: False (plain decode), True (the cascade entry point whenever
        the batch has prefix groups) or "auto" (the cascade where the library
        expects it to pay, qwen2_attn_decode_cascade_worthwhile)."""
        sh = batch.shape
        self.batch = batch
        self.sh = sh
        H, Hkv, d = sh.num_heads, sh.num_kv_heads, sh.head_dim
        self.tdtype = torch.bfloat16 if sh.dtype == "bf16" else torch.float32
        i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)
        self.qkv = to_device(batch.qkv, sh.dtype, device)
        self.q = self.qkv[:, : H * d]
        self.k = self.qkv[:, H * d:(H + Hkv) * d]
        self.v = self.qkv[:, (H + Hkv) * d:]
        T = batch.num_tokens
        self.q_out = torch.empty(T, H, d, dtype=self.tdtype, device=device)
        self.out = torch.full((T, H, d), float("nan"), dtype=self.tdtype, device=device)
        self.positions = i32(batch.positions)
        self.slots = i32(batch.slot_mapping)
        cdt = sh.cache_storage
        self.fp8 = cdt == "fp8"
        self.k_cache = k_cache if k_cache is not None else to_device(batch.k_cache, cdt, device)
        self.v_cache = v_cache if v_cache is not None else to_device(batch.v_cache, cdt, device)
        self.cos_sin = rope_table(d, sh.rope_theta, sh.max_position, device,
                                  getattr(sh, "rope_scaling", None))
        self.q_norm_w = self.k_norm_w = None
        if batch.q_norm_weight is not None:
            self.q_norm_w = to_device(batch.q_norm_weight, sh.dtype, device)
            self.k_norm_w = to_device(batch.k_norm_weight, sh.dtype, device)
        P = batch.num_prefill
        self.Tp = batch.num_prefill_tokens
        if P:
            cu, ctx, bt = batch.prefill_part()
            self.p_cu, self.p_ctx, self.p_bt = i32(cu), i32(ctx), i32(bt)
            self.p_max_q = int(batch.query_lens[:P].max())
            self.p_max_c = int(ctx.max())
        if batch.num_decode:
            ctx, bt = batch.decode_part()
            self.d_ctx, self.d_bt = i32(ctx), i32(bt)
            self.d_max_c = int(ctx.max())
            self.cascade = use_cascade(batch, cascade)
            if self.cascade:
                ind, seqs, lens = batch.prefix_groups
                self.pg = (i32(ind), i32(seqs), i32(lens))
                self.max_prefix = int(np.max(lens))
                ws = B.qwen2_attn_decode_cascade_workspace_size(
                    batch.num_decode, self.d_max_c, self.max_prefix, len(lens), len(seqs), H, Hkv,
                    d, sh.block_size, self.tdtype)
            else:
                ws = B.qwen2_attn_decode_workspace_size(batch.num_decode, self.d_max_c, H, Hkv, d,
                                                        sh.block_size, self.tdtype)
            self.workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=device) if ws else None

    # --- the three calls ---
    def rope_write(self, stream=None):
        sh = self.sh
        args = (self.q, self.q_out, self.k, self.v, self.positions, self.slots, self.cos_sin,
                self.k_cache, self.v_cache, sh.num_heads, sh.num_kv_heads, sh.head_dim,
                sh.block_size)
        if self.q_norm_w is not None:
            B.qwen3_rope_cache_write(*args, self.q_norm_w, self.k_norm_w, sh.rms_eps,
                                     sh.k_scale if self.fp8 else None,
                                     sh.v_scale if self.fp8 else None, stream)
        elif self.fp8:
            B.qwen2_rope_cache_write_fp8(*args, sh.k_scale, sh.v_scale, stream)
        else:
            B.qwen2_rope_cache_write(*args, stream)

    def prefill(self, stream=None):
        if not self.batch.num_prefill:
            return
        sh = self.sh
        args = (self.q_out[: self.Tp], self.k_cache, self.v_cache, self.p_cu, self.p_ctx,
                self.p_bt, self.out[: self.Tp], self.p_max_q, self.p_max_c, sh.num_heads,
                sh.num_kv_heads, sh.head_dim, sh.block_size, sh.scale)
        if self.fp8:
            B.qwen2_attn_prefill_varlen_fp8(*args, sh.k_scale, sh.v_scale, stream)
        else:
            B.qwen2_attn_prefill_varlen(*args, stream)

    def decode(self, stream=None):
        if not self.batch.num_decode:
            return
        sh = self.sh
        if self.cascade:
            B.qwen2_attn_decode_paged_cascade(
                self.q_out[self.Tp:], self.k_cache, self.v_cache, self.d_bt, self.d_ctx, *self.pg,
                self.max_prefix, self.out[self.Tp:], self.workspace, self.d_max_c, sh.num_heads,
                sh.num_kv_heads, sh.head_dim, sh.block_size, sh.scale,
                sh.k_scale if self.fp8 else None, sh.v_scale if self.fp8 else None, stream)
            return
        args = (self.q_out[self.Tp:], self.k_cache, self.v_cache, self.d_bt, self.d_ctx,
                self.out[self.Tp:], self.workspace, self.d_max_c, sh.num_heads, sh.num_kv_heads,
                sh.head_dim, sh.block_size, sh.scale)
        if self.fp8:
            B.qwen2_attn_decode_paged_fp8(*args, sh.k_scale, sh.v_scale, stream)
        else:
            B.qwen2_attn_decode_paged(*args, stream)

    def step(self, stream=None):
        self.rope_write(stream)
        self.prefill(stream)
        self.decode(stream)

    def step_overlapped(self):
        """The step with the prefill and the decode on two streams: both read
        only what the cache write produced, so after it the prefill runs on a
        side stream (default priority) while the decode runs on the current
        one, and the current stream then waits for the side stream.  A graph
        captured around this call records the same fork and join."""
        if not (self.batch.num_prefill and self.batch.num_decode):
            return self.step()
        cur = torch.cuda.current_stream()
        if getattr(self, "_side", None) is None:
            self._side = torch.cuda.Stream()
        side = self._side
        self.rope_write()
        side.wait_stream(cur)
        with torch.cuda.stream(side):
            self.prefill()
        self.decode()
        cur.wait_stream(side)

    def results(self):
        """Host copies: q_out, k_cache, v_cache, out (storage arrays)."""
        torch.cuda.synchronize()
        return {"q_out": to_host(self.q_out), "k_cache": to_host(self.k_cache),
                "v_cache": to_host(self.v_cache), "out": to_host(self.out)}
