"""ctypes binding of libqwen2attn.so (declared in include/qwen2_attn.h).

Argument marshalling only: each function takes torch tensors (device memory
owned by the caller), passes their data pointers, row strides and sizes to
the C entry point of the same name on the current HIP stream, and raises
``QwenAttnError`` on a nonzero status.  Every step of the computation runs
in the library's HIP kernels; there is no Python or CPU fallback.

Storage dtypes: ``torch.bfloat16`` (QW_BF16) and ``torch.float32`` (QW_F32).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqwen2attn.so")

QW_F32, QW_BF16 = 0, 1
STATUS = {0: "QW_OK", 1: "QW_ERR_NULL", 2: "QW_ERR_SHAPE", 3: "QW_ERR_UNSUPPORTED",
          4: "QW_ERR_ALIGN", 5: "QW_ERR_WORKSPACE", 6: "QW_ERR_METADATA", 7: "QW_ERR_HIP"}

# exported symbols and their C signatures (mirrors include/qwen2_attn.h)
_p, _i, _i64, _f, _d, _sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                            ctypes.c_double, ctypes.c_size_t)
SIGNATURES = {
    "qwen2_rope_table_init": (_i, [_p, _i, _i, _d, _p]),
    "qwen2_rope_dynamic_ntk_positions": (_i, [_i, _d]),
    "qwen2_rope_table_init_dynamic_ntk": (_i, [_p, _i, _d, _i, _d, _p]),
    "qwen2_rope_cache_write": (_i, [_p, _i64, _p, _i64, _p, _i64, _p, _i64, _p, _p, _p, _i,
                                    _p, _p, _i, _i, _i, _i, _i, _i, _i, _p]),
    "qwen2_attn_prefill_varlen": (_i, [_p, _i64, _p, _p, _i, _p, _p, _p, _i, _p, _i64, _i, _i,
                                       _i, _i, _i, _i, _i, _i, _f, _i, _p]),
    "qwen2_attn_decode_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "qwen2_attn_decode_paged": (_i, [_p, _i64, _p, _p, _i, _p, _i, _p, _p, _i64, _p, _sz, _i,
                                     _i, _i, _i, _i, _i, _f, _i, _p]),
    "qwen2_rope_cache_write_fp8": (_i, [_p, _i64, _p, _i64, _p, _i64, _p, _i64, _p, _p, _p, _i,
                                        _p, _p, _i, _i, _i, _i, _i, _i, _i, _f, _f, _p]),
    "qwen2_attn_prefill_varlen_fp8": (_i, [_p, _i64, _p, _p, _i, _p, _p, _p, _i, _p, _i64, _i,
                                           _i, _i, _i, _i, _i, _i, _i, _f, _i, _f, _f, _p]),
    "qwen2_attn_decode_paged_noalloc": (_i, [_p, _i64, _p, _p, _i, _p, _i, _p, _p, _i64, _i, _i,
                                             _i, _i, _i, _i, _f, _i, _p]),
    "qwen2_attn_decode_paged_fp8": (_i, [_p, _i64, _p, _p, _i, _p, _i, _p, _p, _i64, _p, _sz,
                                         _i, _i, _i, _i, _i, _i, _f, _i, _f, _f, _p]),
    "qwen3_rope_cache_write": (_i, [_p, _i64, _p, _i64, _p, _i64, _p, _i64, _p, _p, _p, _i,
                                    _p, _p, _i, _i, _i, _i, _i, _i, _i, _p, _p, _d, _p]),
    "qwen3_rope_cache_write_fp8": (_i, [_p, _i64, _p, _i64, _p, _i64, _p, _i64, _p, _p, _p, _i,
                                        _p, _p, _i, _i, _i, _i, _i, _i, _i, _p, _p, _d, _f, _f,
                                        _p]),
    "qwen2_attn_decode_cascade_worthwhile": (_i, [_i, _i, _i, _i, _i, _i]),
    "qwen2_attn_decode_cascade_workspace_size": (_sz, [_i, _i, _i, _i, _i, _i, _i, _i, _i, _i]),
    "qwen2_attn_decode_paged_cascade": (_i, [_p, _i64, _p, _p, _i, _p, _i, _p, _p, _p, _p, _i, _i,
                                             _i, _p, _i64, _p, _sz, _i, _i, _i, _i, _i, _i, _f,
                                             _i, _p]),
    "qwen2_attn_decode_paged_cascade_fp8": (_i, [_p, _i64, _p, _p, _i, _p, _i, _p, _p, _p, _p, _i,
                                                 _i, _i, _p, _i64, _p, _sz, _i, _i, _i, _i, _i,
                                                 _i, _f, _i, _f, _f, _p]),
    "qwen2_check_prefix_groups_host": (_i, [_p, _p, _p, _i, _i, _i, _p, _p, _i, _i, _i]),
    "qwen2_check_metadata_host": (_i, [_p, _p, _i, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i]),
    "qwen2_device_errors": (_i, [_p, _i]),
    "qwen2_status_string": (ctypes.c_char_p, [_i]),
    "qwen2_last_error": (ctypes.c_char_p, []),
}

# flags of qwen2_device_errors (QW_DEVICE_ERR_* in the header)
DEVICE_ERR_POSITION, DEVICE_ERR_SLOT, DEVICE_ERR_BLOCK, DEVICE_ERR_SEQUENCE = 1, 2, 4, 8

_lib: Optional[ctypes.CDLL] = None


class QwenAttnError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn}: {STATUS.get(status, status)}: {detail}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load the shared library (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m paged_gqa_attention_neox_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise QwenAttnError(fn, status, lib().qwen2_last_error().decode())


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return QW_BF16
    if t.dtype == torch.float32:
        return QW_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _rows(t: torch.Tensor, width: int):
    """(pointer, row stride in elements) of a [rows][width] or [rows][heads][d]
    view whose row elements are contiguous."""
    if t.dim() == 3:
        if t.stride(2) != 1 or t.stride(1) != t.shape[2]:
            raise ValueError("heads within a row must be contiguous")
    elif t.dim() == 2:
        if t.stride(1) != 1:
            raise ValueError("row elements must be contiguous")
    else:
        raise ValueError("expected a 2-D or 3-D tensor")
    if t.shape[0] > 0 and t[0].numel() != width:
        raise ValueError(f"row width {t[0].numel()} != {width}")
    return t.data_ptr(), t.stride(0)


def _i32(t: Optional[torch.Tensor]) -> int:
    if t is None:
        return 0
    if t.dtype != torch.int32 or not t.is_contiguous():
        raise TypeError("metadata tensors must be contiguous int32")
    return t.data_ptr()


# ---------------------------------------------------------------------------
def qwen2_rope_table_init(cos_sin: torch.Tensor, rope_theta: float, stream=None) -> None:
    """cos_sin: float64 [max_position][rotary_dim] on the device, filled."""
    if cos_sin.dtype != torch.float64 or not cos_sin.is_contiguous() or cos_sin.dim() != 2:
        raise TypeError("cos_sin must be a contiguous float64 [max_position][rotary_dim] tensor")
    _check("qwen2_rope_table_init",
           lib().qwen2_rope_table_init(cos_sin.data_ptr(), cos_sin.shape[0], cos_sin.shape[1],
                                       float(rope_theta), _stream(stream)))


def qwen2_rope_dynamic_ntk_positions(original_max_position: int, factor: float) -> int:
    """Rows of the dynamic-NTK table: floor(factor * original_max_position)."""
    n = lib().qwen2_rope_dynamic_ntk_positions(int(original_max_position), float(factor))
    if n < 1:
        raise ValueError("invalid original_max_position / factor")
    return n


def qwen2_rope_table_init_dynamic_ntk(cos_sin: torch.Tensor, original_max_position: int,
                                      factor: float, rope_theta: float, stream=None) -> None:
    """cos_sin: float64 [qwen2_rope_dynamic_ntk_positions(...)][rotary_dim], filled."""
    if cos_sin.dtype != torch.float64 or not cos_sin.is_contiguous() or cos_sin.dim() != 2:
        raise TypeError("cos_sin must be a contiguous float64 [positions][rotary_dim] tensor")
    if cos_sin.shape[0] != qwen2_rope_dynamic_ntk_positions(original_max_position, factor):
        raise ValueError("cos_sin rows must equal qwen2_rope_dynamic_ntk_positions(...)")
    _check("qwen2_rope_table_init_dynamic_ntk",
           lib().qwen2_rope_table_init_dynamic_ntk(cos_sin.data_ptr(), int(original_max_position),
                                                   float(factor), cos_sin.shape[1],
                                                   float(rope_theta), _stream(stream)))


def qwen2_rope_cache_write(q, q_out, k, v, positions, slot_mapping, cos_sin, k_cache, v_cache,
                           num_heads: int, num_kv_heads: int, head_dim: int, block_size: int,
                           stream=None) -> None:
    """q [T][H*d] (or [T][H][d]) view, q_out same shape (may be q), k and v
    [T][Hkv*d] views (e.g. column slices of the fused QKV tensor);
    positions, slot_mapping int32 [T]; cos_sin float64 [max_position][d];
    caches laid out as in include/qwen2_attn.h."""
    T = q.shape[0]
    if cos_sin.dim() != 2 or cos_sin.shape[1] != head_dim or cos_sin.dtype != torch.float64:
        raise ValueError("cos_sin must be float64 [max_position][head_dim]")
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        if t.dim() != 4 or t.shape[1] != num_kv_heads or t.dtype != q.dtype:
            raise ValueError(f"{name} must be [num_blocks][num_kv_heads][..] of the q dtype")
    qp, qs = _rows(q, num_heads * head_dim)
    op, os_ = _rows(q_out, num_heads * head_dim)
    kp, ks = _rows(k, num_kv_heads * head_dim)
    vp, vs = _rows(v, num_kv_heads * head_dim)
    _check("qwen2_rope_cache_write",
           lib().qwen2_rope_cache_write(qp, qs, op, os_, kp, ks, vp, vs, _i32(positions),
                                        _i32(slot_mapping), cos_sin.data_ptr(), cos_sin.shape[0],
                                        k_cache.data_ptr(), v_cache.data_ptr(), k_cache.shape[0],
                                        T, num_heads, num_kv_heads, head_dim, block_size,
                                        _dtype(q), _stream(stream)))


def qwen2_attn_prefill_varlen(q, k_cache, v_cache, cu_seqlens_q, context_lens, block_tables, out,
                              max_query_len: int, max_context_len: int, num_heads: int,
                              num_kv_heads: int, head_dim: int, block_size: int, scale: float,
                              stream=None) -> None:
    """q, out: [T][H][d] (or [T][H*d]); cu_seqlens_q int32 [S+1];
    context_lens int32 [S]; block_tables int32 [S][max_blocks]."""
    qp, qs = _rows(q, num_heads * head_dim)
    op, os_ = _rows(out, num_heads * head_dim)
    S = context_lens.shape[0]
    _check("qwen2_attn_prefill_varlen",
           lib().qwen2_attn_prefill_varlen(qp, qs, k_cache.data_ptr(), v_cache.data_ptr(),
                                           k_cache.shape[0], _i32(cu_seqlens_q), _i32(context_lens),
                                           _i32(block_tables), block_tables.shape[1], op, os_, S,
                                           q.shape[0], max_query_len, max_context_len, num_heads,
                                           num_kv_heads, head_dim, block_size, float(scale),
                                           _dtype(q), _stream(stream)))


def qwen2_attn_decode_workspace_size(num_seqs: int, max_context_len: int, num_heads: int,
                                     num_kv_heads: int, head_dim: int, block_size: int,
                                     dtype: torch.dtype) -> int:
    n = lib().qwen2_attn_decode_workspace_size(num_seqs, max_context_len, num_heads, num_kv_heads,
                                               head_dim, block_size,
                                               QW_BF16 if dtype == torch.bfloat16 else QW_F32)
    if n == ctypes.c_size_t(-1).value:
        raise QwenAttnError("qwen2_attn_decode_workspace_size", 3, lib().qwen2_last_error().decode())
    return n


def qwen2_attn_decode_paged(q, k_cache, v_cache, block_tables, context_lens, out, workspace,
                            max_context_len: int, num_heads: int, num_kv_heads: int, head_dim: int,
                            block_size: int, scale: float, stream=None) -> None:
    """q, out: [S][H][d] (or [S][H*d]); workspace: a device tensor of at
    least qwen2_attn_decode_workspace_size(...) bytes, or None when that is 0."""
    qp, qs = _rows(q, num_heads * head_dim)
    op, os_ = _rows(out, num_heads * head_dim)
    wp = workspace.data_ptr() if workspace is not None else 0
    wb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("qwen2_attn_decode_paged",
           lib().qwen2_attn_decode_paged(qp, qs, k_cache.data_ptr(), v_cache.data_ptr(),
                                         k_cache.shape[0], _i32(block_tables), block_tables.shape[1],
                                         _i32(context_lens), op, os_, wp, wb, q.shape[0],
                                         max_context_len, num_heads, num_kv_heads, head_dim,
                                         block_size, float(scale), _dtype(q), _stream(stream)))


def qwen2_attn_decode_paged_noalloc(q, k_cache, v_cache, block_tables, context_lens, out,
                                    max_context_len: int, num_heads: int, num_kv_heads: int,
                                    head_dim: int, block_size: int, scale: float,
                                    stream=None) -> None:
    """As qwen2_attn_decode_paged, with the library's per-GPU static scratch
    as the workspace (the call allocates nothing; overlapping calls on one
    GPU race)."""
    qp, qs = _rows(q, num_heads * head_dim)
    op, os_ = _rows(out, num_heads * head_dim)
    _check("qwen2_attn_decode_paged_noalloc",
           lib().qwen2_attn_decode_paged_noalloc(qp, qs, k_cache.data_ptr(), v_cache.data_ptr(),
                                                 k_cache.shape[0], _i32(block_tables),
                                                 block_tables.shape[1], _i32(context_lens), op,
                                                 os_, q.shape[0], max_context_len, num_heads,
                                                 num_kv_heads, head_dim, block_size, float(scale),
                                                 _dtype(q), _stream(stream)))


# ---------------------------------------------------------------------------
# FP8 (E4M3FN) KV cache: the caches are uint8 code tensors of the same layouts
def _fp8_caches(k_cache, v_cache, num_kv_heads):
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        if t.dim() != 4 or t.shape[1] != num_kv_heads or t.dtype != torch.uint8:
            raise ValueError(f"{name} must be a uint8 [num_blocks][num_kv_heads][..] code tensor")


def qwen2_rope_cache_write_fp8(q, q_out, k, v, positions, slot_mapping, cos_sin, k_cache, v_cache,
                               num_heads: int, num_kv_heads: int, head_dim: int, block_size: int,
                               k_scale: float, v_scale: float, stream=None) -> None:
    """As qwen2_rope_cache_write; the caches receive E4M3FN codes of
    rot(k) / k_scale and v / v_scale."""
    T = q.shape[0]
    if cos_sin.dim() != 2 or cos_sin.shape[1] != head_dim or cos_sin.dtype != torch.float64:
        raise ValueError("cos_sin must be float64 [max_position][head_dim]")
    _fp8_caches(k_cache, v_cache, num_kv_heads)
    qp, qs = _rows(q, num_heads * head_dim)
    op, os_ = _rows(q_out, num_heads * head_dim)
    kp, ks = _rows(k, num_kv_heads * head_dim)
    vp, vs = _rows(v, num_kv_heads * head_dim)
    _check("qwen2_rope_cache_write_fp8",
           lib().qwen2_rope_cache_write_fp8(qp, qs, op, os_, kp, ks, vp, vs, _i32(positions),
                                            _i32(slot_mapping), cos_sin.data_ptr(),
                                            cos_sin.shape[0], k_cache.data_ptr(),
                                            v_cache.data_ptr(), k_cache.shape[0], T, num_heads,
                                            num_kv_heads, head_dim, block_size, _dtype(q),
                                            float(k_scale), float(v_scale), _stream(stream)))


def qwen2_attn_prefill_varlen_fp8(q, k_cache, v_cache, cu_seqlens_q, context_lens, block_tables,
                                  out, max_query_len: int, max_context_len: int, num_heads: int,
                                  num_kv_heads: int, head_dim: int, block_size: int, scale: float,
                                  k_scale: float, v_scale: float, stream=None) -> None:
    """As qwen2_attn_prefill_varlen over FP8 code caches."""
    _fp8_caches(k_cache, v_cache, num_kv_heads)
    qp, qs = _rows(q, num_heads * head_dim)
    op, os_ = _rows(out, num_heads * head_dim)
    S = context_lens.shape[0]
    _check("qwen2_attn_prefill_varlen_fp8",
           lib().qwen2_attn_prefill_varlen_fp8(qp, qs, k_cache.data_ptr(), v_cache.data_ptr(),
                                               k_cache.shape[0], _i32(cu_seqlens_q),
                                               _i32(context_lens), _i32(block_tables),
                                               block_tables.shape[1], op, os_, S, q.shape[0],
                                               max_query_len, max_context_len, num_heads,
                                               num_kv_heads, head_dim, block_size, float(scale),
                                               _dtype(q), float(k_scale), float(v_scale),
                                               _stream(stream)))


def qwen2_attn_decode_paged_fp8(q, k_cache, v_cache, block_tables, context_lens, out, workspace,
                                max_context_len: int, num_heads: int, num_kv_heads: int,
                                head_dim: int, block_size: int, scale: float, k_scale: float,
                                v_scale: float, stream=None) -> None:
    """As qwen2_attn_decode_paged over FP8 code caches."""
    _fp8_caches(k_cache, v_cache, num_kv_heads)
    qp, qs = _rows(q, num_heads * head_dim)
    op, os_ = _rows(out, num_heads * head_dim)
    wp = workspace.data_ptr() if workspace is not None else 0
    wb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("qwen2_attn_decode_paged_fp8",
           lib().qwen2_attn_decode_paged_fp8(qp, qs, k_cache.data_ptr(), v_cache.data_ptr(),
                                             k_cache.shape[0], _i32(block_tables),
                                             block_tables.shape[1], _i32(context_lens), op, os_,
                                             wp, wb, q.shape[0], max_context_len, num_heads,
                                             num_kv_heads, head_dim, block_size, float(scale),
                                             _dtype(q), float(k_scale), float(v_scale),
                                             _stream(stream)))


def qwen3_rope_cache_write(q, q_out, k, v, positions, slot_mapping, cos_sin, k_cache, v_cache,
                           num_heads: int, num_kv_heads: int, head_dim: int, block_size: int,
                           q_norm_weight, k_norm_weight, rms_eps: float = 1e-6,
                           k_scale: Optional[float] = None, v_scale: Optional[float] = None,
                           stream=None) -> None:
    """Qwen3: per-head RMSNorm of q and k (weights [head_dim] of the q dtype)
    before the rotation; with k_scale/v_scale the caches are FP8 code tensors
    (qwen3_rope_cache_write_fp8)."""
    T = q.shape[0]
    if cos_sin.dim() != 2 or cos_sin.shape[1] != head_dim or cos_sin.dtype != torch.float64:
        raise ValueError("cos_sin must be float64 [max_position][head_dim]")
    for name, w in (("q_norm_weight", q_norm_weight), ("k_norm_weight", k_norm_weight)):
        if w.dtype != q.dtype or w.numel() != head_dim or not w.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [head_dim] tensor of the q dtype")
    fp8 = k_scale is not None
    if fp8:
        _fp8_caches(k_cache, v_cache, num_kv_heads)
    qp, qs = _rows(q, num_heads * head_dim)
    op, os_ = _rows(q_out, num_heads * head_dim)
    kp, ks = _rows(k, num_kv_heads * head_dim)
    vp, vs = _rows(v, num_kv_heads * head_dim)
    common = (qp, qs, op, os_, kp, ks, vp, vs, _i32(positions), _i32(slot_mapping),
              cos_sin.data_ptr(), cos_sin.shape[0], k_cache.data_ptr(), v_cache.data_ptr(),
              k_cache.shape[0], T, num_heads, num_kv_heads, head_dim, block_size, _dtype(q),
              q_norm_weight.data_ptr(), k_norm_weight.data_ptr(), float(rms_eps))
    if fp8:
        _check("qwen3_rope_cache_write_fp8",
               lib().qwen3_rope_cache_write_fp8(*common, float(k_scale), float(v_scale),
                                                _stream(stream)))
    else:
        _check("qwen3_rope_cache_write", lib().qwen3_rope_cache_write(*common, _stream(stream)))


def qwen2_check_metadata_host(positions, slot_mapping, cu_seqlens_q, context_lens, block_tables,
                              num_blocks: int, block_size: int, max_position: int,
                              max_context_len: int, max_query_len: int = 0) -> None:
    """Host-side contract check on numpy int32 arrays (any may be None except
    context_lens and block_tables).  Raises QwenAttnError on a violation."""
    def ptr(a):
        if a is None:
            return 0, None
        a = np.ascontiguousarray(a, dtype=np.int32)
        return a.ctypes.data, a
    pp, keep1 = ptr(positions)
    sp, keep2 = ptr(slot_mapping)
    cp, keep3 = ptr(cu_seqlens_q)
    lp, keep4 = ptr(context_lens)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    T = len(positions) if positions is not None else (len(slot_mapping) if slot_mapping is not None else 0)
    _check("qwen2_check_metadata_host",
           lib().qwen2_check_metadata_host(pp, sp, T, cp, lp, bt.ctypes.data, len(context_lens),
                                           bt.shape[1], num_blocks, block_size, max_position,
                                           max_context_len, max_query_len))
    del keep1, keep2, keep3, keep4


# ---------------------------------------------------------------------------
# shared-prefix (cascade) decode
def qwen2_attn_decode_cascade_worthwhile(num_prefixes: int, num_prefix_members: int,
                                         max_prefix_len: int, num_kv_heads: int, head_dim: int,
                                         cache_fp8: bool = False) -> bool:
    """The library's estimate of whether the cascade decode beats the plain one."""
    return bool(lib().qwen2_attn_decode_cascade_worthwhile(num_prefixes, num_prefix_members,
                                                           max_prefix_len, num_kv_heads, head_dim,
                                                           int(bool(cache_fp8))))


def qwen2_attn_decode_cascade_workspace_size(num_seqs: int, max_context_len: int,
                                             max_prefix_len: int, num_prefixes: int,
                                             num_prefix_members: int, num_heads: int,
                                             num_kv_heads: int, head_dim: int, block_size: int,
                                             dtype: torch.dtype) -> int:
    n = lib().qwen2_attn_decode_cascade_workspace_size(
        num_seqs, max_context_len, max_prefix_len, num_prefixes, num_prefix_members, num_heads,
        num_kv_heads, head_dim, block_size, QW_BF16 if dtype == torch.bfloat16 else QW_F32)
    if n == ctypes.c_size_t(-1).value:
        raise QwenAttnError("qwen2_attn_decode_cascade_workspace_size", 3,
                            lib().qwen2_last_error().decode())
    return n


def qwen2_attn_decode_paged_cascade(q, k_cache, v_cache, block_tables, context_lens,
                                    prefix_indptr, prefix_seqs, prefix_lens, max_prefix_len: int,
                                    out, workspace, max_context_len: int, num_heads: int,
                                    num_kv_heads: int, head_dim: int, block_size: int,
                                    scale: float, k_scale=None, v_scale=None,
                                    stream=None) -> None:
    """As qwen2_attn_decode_paged, with the decode sequences' shared prefixes
    given as device int32 prefix_indptr [P+1], prefix_seqs [members],
    prefix_lens [P] (tokens); k_scale and v_scale select the FP8-cache call."""
    qp, qs = _rows(q, num_heads * head_dim)
    op, os_ = _rows(out, num_heads * head_dim)
    wp = workspace.data_ptr() if workspace is not None else 0
    wb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    P = prefix_lens.shape[0] if prefix_lens is not None else 0
    M = prefix_seqs.shape[0] if prefix_seqs is not None else 0
    args = [qp, qs, k_cache.data_ptr(), v_cache.data_ptr(), k_cache.shape[0], _i32(block_tables),
            block_tables.shape[1], _i32(context_lens), _i32(prefix_indptr), _i32(prefix_seqs),
            _i32(prefix_lens), P, M, int(max_prefix_len), op, os_, wp, wb, q.shape[0],
            max_context_len, num_heads, num_kv_heads, head_dim, block_size, float(scale),
            _dtype(q)]
    if k_scale is None:
        _check("qwen2_attn_decode_paged_cascade",
               lib().qwen2_attn_decode_paged_cascade(*args, _stream(stream)))
    else:
        _fp8_caches(k_cache, v_cache, num_kv_heads)
        _check("qwen2_attn_decode_paged_cascade_fp8",
               lib().qwen2_attn_decode_paged_cascade_fp8(*args, float(k_scale), float(v_scale),
                                                         _stream(stream)))


def qwen2_check_prefix_groups_host(prefix_indptr, prefix_seqs, prefix_lens, max_prefix_len: int,
                                   context_lens, block_tables, block_size: int) -> None:
    """Host-side check of the cascade's prefix-group contract on numpy int32
    arrays.  Raises QwenAttnError on a violation."""
    ind = np.ascontiguousarray(prefix_indptr, dtype=np.int32)
    seqs = np.ascontiguousarray(prefix_seqs, dtype=np.int32)
    lens = np.ascontiguousarray(prefix_lens, dtype=np.int32)
    ctx = np.ascontiguousarray(context_lens, dtype=np.int32)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    _check("qwen2_check_prefix_groups_host",
           lib().qwen2_check_prefix_groups_host(ind.ctypes.data, seqs.ctypes.data, lens.ctypes.data,
                                                len(lens), len(seqs), int(max_prefix_len),
                                                ctx.ctypes.data, bt.ctypes.data, len(ctx),
                                                bt.shape[1], block_size))


def qwen2_device_errors(clear: bool = False) -> int:
    """The current GPU's device error word (QW_DEVICE_ERR_* flags gathered
    since it was last cleared); clear=True resets it.  Synchronises."""
    flags = ctypes.c_uint(0)
    _check("qwen2_device_errors", lib().qwen2_device_errors(ctypes.addressof(flags), int(clear)))
    return int(flags.value)


def status_string(status: int) -> str:
    return lib().qwen2_status_string(status).decode()
