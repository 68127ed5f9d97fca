"""The C-ABI library without a GPU: it loads, exports every declared entry
point, and its host-side validation returns the documented status before any
launch.  Every call here fails validation (or is host-only), so nothing is
enqueued on a device."""
import ctypes
import os
import re

import numpy as np
import pytest

from paged_gqa_attention_neox_amd import binding as B
from paged_gqa_attention_neox_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qwen2_attn.h")

QW_OK, QW_ERR_NULL, QW_ERR_SHAPE, QW_ERR_UNSUPPORTED, QW_ERR_ALIGN, QW_ERR_WORKSPACE, \
    QW_ERR_METADATA, QW_ERR_HIP = range(8)

# fake, 256-byte aligned "device" addresses: validation only looks at them
P = 0x10000
P2 = 0x20000
P3 = 0x30000
MIS = 0x10008   # 8-byte aligned only


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libqwen2attn.so not built")
    return B.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qwen[23]_\w+)\s*\(", text)))


def test_header_declares_the_three_path_calls():
    names = declared_functions()
    for n in ("qwen2_rope_cache_write", "qwen2_attn_prefill_varlen", "qwen2_attn_decode_paged"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(lib, n), n
        assert n in B.SIGNATURES, f"binding lacks {n}"


def test_exported_dynamic_symbols_match_header(lib):
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (qwen[23]_\w+)", out))
    assert exported == set(declared_functions())
    # every exported symbol of the library is a declared entry point (no
    # other external names leak out of the C ABI)
    assert "qwen3_rope_cache_write" in exported and "qwen3_rope_cache_write_fp8" in exported
    assert set(B.SIGNATURES) == exported
    others = set(re.findall(r"\bT (\S+)", out)) - exported
    assert not others, f"internal symbols exported: {sorted(others)[:5]}"


def test_status_strings(lib):
    for s in range(8):
        assert B.status_string(s) and B.status_string(s) != "unknown status"
    assert B.status_string(99) == "unknown status"


def _decode(lib, **kw):
    a = dict(q=P, qs=28 * 128, kc=P2, vc=P3, nb=100, bt=P, mb=64, ctx=P, out=P2, os=28 * 128,
             ws=P3, wsb=1 << 30, S=4, maxc=1024, H=28, Hkv=4, d=128, B=16, scale=0.0884, dt=1)
    a.update(kw)
    return lib.qwen2_attn_decode_paged(a["q"], a["qs"], a["kc"], a["vc"], a["nb"], a["bt"], a["mb"],
                                       a["ctx"], a["out"], a["os"], a["ws"], a["wsb"], a["S"],
                                       a["maxc"], a["H"], a["Hkv"], a["d"], a["B"], a["scale"],
                                       a["dt"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), QW_ERR_NULL),
    (dict(out=0), QW_ERR_NULL),
    (dict(kc=0), QW_ERR_NULL),
    (dict(ctx=0), QW_ERR_NULL),
    (dict(bt=0), QW_ERR_NULL),
    (dict(H=30), QW_ERR_SHAPE),                    # not a multiple of Hkv
    (dict(d=96, qs=28 * 96, os=28 * 96), QW_ERR_UNSUPPORTED),
    (dict(B=48), QW_ERR_UNSUPPORTED),              # block sizes: 16, 32 or 64 tokens
    (dict(B=8), QW_ERR_UNSUPPORTED),
    (dict(B=128), QW_ERR_UNSUPPORTED),
    (dict(dt=5), QW_ERR_UNSUPPORTED),
    (dict(H=68, Hkv=4, qs=68 * 128, os=68 * 128), QW_ERR_UNSUPPORTED),   # group 17
    (dict(q=MIS), QW_ERR_ALIGN),
    (dict(qs=28 * 128 + 4), QW_ERR_ALIGN),
    (dict(qs=100), QW_ERR_SHAPE),
    (dict(mb=8), QW_ERR_SHAPE),                    # 8 blocks cannot hold 1024 tokens
    (dict(maxc=0), QW_ERR_SHAPE),
    (dict(nb=0), QW_ERR_SHAPE),
    (dict(scale=float("nan")), QW_ERR_SHAPE),
    (dict(S=-1), QW_ERR_SHAPE),
    (dict(ws=0), QW_ERR_WORKSPACE),
    (dict(wsb=16), QW_ERR_WORKSPACE),
    (dict(ws=MIS), QW_ERR_ALIGN),
])
def test_decode_validation(lib, kw, status):
    assert _decode(lib, **kw) == status
    assert lib.qwen2_last_error().decode()


def test_zero_work_is_ok_without_launch(lib):
    assert _decode(lib, S=0, q=0, out=0) == QW_OK
    assert lib.qwen2_rope_cache_write(0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 1, 0, 0, 0, 0, 28, 4, 128, 16, 1,
                                      None) == QW_OK


def test_workspace_size(lib):
    bf16 = __import__("torch").bfloat16
    # long contexts: partial states of at most two pieces per wave (a few MB,
    # far below one partial per 512-token partition)
    n = B.qwen2_attn_decode_workspace_size(64, 32768, 28, 4, 128, 16, bf16)
    assert 0 < n < 64 * 28 * (32768 // 512) * 128 * 4 // 2
    assert n >= 2 * 256 * 2 * 7 * 130 * 4       # at least two partial states per range of a full round
    # small batches are spread over a few ranges and need little workspace
    small = B.qwen2_attn_decode_workspace_size(1, 16, 28, 4, 128, 16, bf16)
    assert 0 < small <= 1024 + 3 * 2 * 7 * 130 * 4
    assert B.qwen2_attn_decode_workspace_size(8, 512, 28, 4, 128, 16, bf16) > small
    assert lib.qwen2_attn_decode_workspace_size(8, 100, 28, 4, 96, 16, 1) == ctypes.c_size_t(-1).value
    # 32- and 64-token cache blocks are streamed as 16-token blocks: the same plan
    for bs in (32, 64):
        assert B.qwen2_attn_decode_workspace_size(64, 32768, 28, 4, 128, bs, bf16) == n
    assert lib.qwen2_attn_decode_workspace_size(8, 100, 28, 4, 128, 48, 1) == ctypes.c_size_t(-1).value


def _rope(lib, **kw):
    W_ = (28 + 8) * 128
    a = dict(q=P, qs=W_, qo=P2, qos=28 * 128, k=P + 28 * 256, ks=W_, v=P + 32 * 256, vs=W_, pos=P,
             slot=P, cs=P3, maxp=32768, kc=P, vc=P2, nb=10, T=5, H=28, Hkv=4, d=128, B=16, dt=1)
    a.update(kw)
    return lib.qwen2_rope_cache_write(a["q"], a["qs"], a["qo"], a["qos"], a["k"], a["ks"], a["v"],
                                      a["vs"], a["pos"], a["slot"], a["cs"], a["maxp"], a["kc"], a["vc"],
                                      a["nb"], a["T"], a["H"], a["Hkv"], a["d"], a["B"], a["dt"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), QW_ERR_NULL), (dict(pos=0), QW_ERR_NULL), (dict(slot=0), QW_ERR_NULL),
    (dict(cs=0), QW_ERR_NULL), (dict(kc=0), QW_ERR_NULL),
    (dict(T=-1), QW_ERR_SHAPE), (dict(maxp=0), QW_ERR_SHAPE),
    (dict(qs=128), QW_ERR_SHAPE), (dict(Hkv=3), QW_ERR_SHAPE),
    (dict(k=MIS), QW_ERR_ALIGN), (dict(cs=MIS), QW_ERR_ALIGN),
    (dict(qo=P + 64), QW_ERR_SHAPE),            # overlaps q without being q
    (dict(d=80), QW_ERR_UNSUPPORTED), (dict(B=48), QW_ERR_UNSUPPORTED), (dict(B=8), QW_ERR_UNSUPPORTED),
])
def test_rope_validation(lib, kw, status):
    assert _rope(lib, **kw) == status


def _rope_qkn(lib, fp8=False, **kw):
    W_ = (28 + 8) * 128
    a = dict(q=P, qs=W_, qo=P2, qos=28 * 128, k=P + 28 * 256, ks=W_, v=P + 32 * 256, vs=W_, pos=P,
             slot=P, cs=P3, maxp=32768, kc=P, vc=P2, nb=10, T=5, H=28, Hkv=4, d=128, B=16, dt=1,
             qw=P3, kw=P3 + 256, eps=1e-6, ksc=0.03, vsc=0.03)
    a.update(kw)
    args = (a["q"], a["qs"], a["qo"], a["qos"], a["k"], a["ks"], a["v"], a["vs"], a["pos"],
            a["slot"], a["cs"], a["maxp"], a["kc"], a["vc"], a["nb"], a["T"], a["H"], a["Hkv"],
            a["d"], a["B"], a["dt"], a["qw"], a["kw"], a["eps"])
    if fp8:
        return lib.qwen3_rope_cache_write_fp8(*args, a["ksc"], a["vsc"], None)
    return lib.qwen3_rope_cache_write(*args, None)


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("kw,status", [
    (dict(qw=0), QW_ERR_NULL), (dict(kw=0), QW_ERR_NULL), (dict(qw=0, kw=0), QW_ERR_NULL),
    (dict(qw=MIS), QW_ERR_ALIGN), (dict(kw=MIS), QW_ERR_ALIGN),
    (dict(eps=-1e-6), QW_ERR_SHAPE), (dict(eps=float("nan")), QW_ERR_SHAPE),
    (dict(eps=float("inf")), QW_ERR_SHAPE), (dict(q=0), QW_ERR_NULL), (dict(d=80), QW_ERR_UNSUPPORTED),
])
def test_qwen3_rope_validation(lib, fp8, kw, status):
    assert _rope_qkn(lib, fp8=fp8, **kw) == status
    assert lib.qwen2_last_error().decode()


def test_qwen3_rope_fp8_scale_validation(lib):
    assert _rope_qkn(lib, fp8=True, ksc=0.0) == QW_ERR_SHAPE
    assert _rope_qkn(lib, fp8=True, vsc=float("nan")) == QW_ERR_SHAPE


def _prefill(lib, **kw):
    a = dict(q=P, qs=28 * 128, kc=P2, vc=P3, nb=100, cu=P, ctx=P, bt=P, mb=64, out=P2, os=28 * 128,
             S=4, T=100, maxq=50, maxc=1024, H=28, Hkv=4, d=128, B=16, scale=0.0884, dt=1)
    a.update(kw)
    return lib.qwen2_attn_prefill_varlen(a["q"], a["qs"], a["kc"], a["vc"], a["nb"], a["cu"], a["ctx"],
                                         a["bt"], a["mb"], a["out"], a["os"], a["S"], a["T"], a["maxq"],
                                         a["maxc"], a["H"], a["Hkv"], a["d"], a["B"], a["scale"],
                                         a["dt"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(cu=0), QW_ERR_NULL), (dict(q=0), QW_ERR_NULL), (dict(vc=0), QW_ERR_NULL),
    (dict(maxq=2000), QW_ERR_SHAPE), (dict(S=70000), QW_ERR_UNSUPPORTED),
    (dict(out=MIS), QW_ERR_ALIGN), (dict(H=0), QW_ERR_SHAPE), (dict(scale=-1.0), QW_ERR_SHAPE),
])
def test_prefill_validation(lib, kw, status):
    assert _prefill(lib, **kw) == status


def test_dynamic_ntk_positions_and_validation(lib):
    assert lib.qwen2_rope_dynamic_ntk_positions(4096, 2.0) == 8192
    assert lib.qwen2_rope_dynamic_ntk_positions(32768, 4.0) == 131072
    assert lib.qwen2_rope_dynamic_ntk_positions(1000, 1.5) == 1500
    assert lib.qwen2_rope_dynamic_ntk_positions(0, 2.0) == -1
    assert lib.qwen2_rope_dynamic_ntk_positions(4096, 0.5) == -1
    assert lib.qwen2_rope_dynamic_ntk_positions(4096, float("nan")) == -1
    assert lib.qwen2_rope_dynamic_ntk_positions(1 << 30, 4.0) == -1
    f = lib.qwen2_rope_table_init_dynamic_ntk
    assert f(0, 4096, 2.0, 128, 1e6, None) == QW_ERR_NULL
    assert f(P, 0, 2.0, 128, 1e6, None) == QW_ERR_SHAPE
    assert f(P, 4096, 0.9, 128, 1e6, None) == QW_ERR_SHAPE
    assert f(P, 4096, 2.0, 127, 1e6, None) == QW_ERR_SHAPE
    assert f(P, 4096, 2.0, 2, 1e6, None) == QW_ERR_SHAPE
    assert f(P, 4096, 2.0, 128, -1.0, None) == QW_ERR_SHAPE
    assert lib.qwen2_last_error().decode()


def test_rope_table_validation(lib):
    assert lib.qwen2_rope_table_init(0, 10, 128, 1e6, None) == QW_ERR_NULL
    assert lib.qwen2_rope_table_init(P, 0, 128, 1e6, None) == QW_ERR_SHAPE
    assert lib.qwen2_rope_table_init(P, 10, 127, 1e6, None) == QW_ERR_SHAPE
    assert lib.qwen2_rope_table_init(P, 10, 128, 0.0, None) == QW_ERR_SHAPE


# ---------------------------------------------------------------------------
# host metadata checker
# ---------------------------------------------------------------------------
def _meta(b, **over):
    a = dict(positions=b.positions, slot_mapping=b.slot_mapping, cu_seqlens_q=b.cu_seqlens_q,
             context_lens=b.context_lens, block_tables=b.block_tables, num_blocks=b.num_blocks,
             block_size=16, max_position=32768, max_context_len=int(b.context_lens.max()),
             max_query_len=int(b.query_lens.max()))
    a.update(over)
    return a


@pytest.mark.parametrize("maker", [W.mixed_tp2, W.qwen2_prefill, W.qwen3_decode])
def test_metadata_of_workloads_is_valid(lib, maker):
    b = maker()
    B.qwen2_check_metadata_host(**_meta(b))


def test_metadata_violations(lib):
    b = W.small_case(3, "bf16", 4, 2, 16, context_lens=[40, 17, 5], query_lens=[8, 1, 5],
                     num_prefill=1)
    B.qwen2_check_metadata_host(**_meta(b))

    def bad(**over):
        with pytest.raises(B.QwenAttnError) as ei:
            B.qwen2_check_metadata_host(**_meta(b, **over))
        assert ei.value.status == QW_ERR_METADATA

    pos = b.positions.copy(); pos[2] += 1
    bad(positions=pos)
    pos = b.positions.copy(); pos[0] = 40000
    bad(positions=pos)
    sl = b.slot_mapping.copy(); sl[1] = sl[0]
    bad(slot_mapping=sl)                                   # duplicate slot
    sl = b.slot_mapping.copy(); sl[3] = b.num_blocks * 16
    bad(slot_mapping=sl)
    sl = b.slot_mapping.copy(); sl[4] = (sl[4] + 1) % (b.num_blocks * 16)
    bad(slot_mapping=sl)                                   # disagrees with the block table
    ctx = b.context_lens.copy(); ctx[2] = 4
    bad(context_lens=ctx)                                  # context < rows
    bt = b.block_tables.copy(); bt[0, 1] = -3
    bad(block_tables=bt)
    cu = b.cu_seqlens_q.copy(); cu[0] = 1
    bad(cu_seqlens_q=cu)
    bad(max_context_len=30)
    bad(max_query_len=4)
    # slot -1 (skip) is allowed
    sl = b.slot_mapping.copy(); sl[0] = -1
    B.qwen2_check_metadata_host(**_meta(b, slot_mapping=sl))


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        B.lib()


# ---------------------------------------------------------------------------
# shared-prefix (cascade) decode: argument checks, workspace, host contract
def _cascade(lib, fp8=False, **kw):
    a = dict(q=P, qs=28 * 128, kc=P2, vc=P3, nb=100, bt=P, mb=64, ctx=P, ind=P, seqs=P2, lens=P3,
             np_=1, nm=3, maxp=512, out=P2, os=28 * 128, ws=P3, wsb=1 << 30, S=4, maxc=1024, H=28,
             Hkv=4, d=128, B=16, scale=0.0884, dt=1)
    a.update(kw)
    args = [a["q"], a["qs"], a["kc"], a["vc"], a["nb"], a["bt"], a["mb"], a["ctx"], a["ind"],
            a["seqs"], a["lens"], a["np_"], a["nm"], a["maxp"], a["out"], a["os"], a["ws"], a["wsb"],
            a["S"], a["maxc"], a["H"], a["Hkv"], a["d"], a["B"], a["scale"], a["dt"]]
    if fp8:
        return lib.qwen2_attn_decode_paged_cascade_fp8(*args, a.get("ksc", 1.0), a.get("vsc", 1.0),
                                                       None)
    return lib.qwen2_attn_decode_paged_cascade(*args, None)


@pytest.mark.parametrize("kw,status", [
    (dict(np_=-1), QW_ERR_SHAPE),
    (dict(nm=-2), QW_ERR_SHAPE),
    (dict(maxp=-16), QW_ERR_SHAPE),
    (dict(ind=0), QW_ERR_NULL),
    (dict(lens=0), QW_ERR_NULL),
    (dict(seqs=0), QW_ERR_NULL),
    (dict(q=0), QW_ERR_NULL),
    (dict(H=30), QW_ERR_SHAPE),
    (dict(mb=8), QW_ERR_SHAPE),
    (dict(ws=0), QW_ERR_WORKSPACE),
    (dict(wsb=4096), QW_ERR_WORKSPACE),
    (dict(ws=MIS), QW_ERR_ALIGN),
    (dict(S=-1), QW_ERR_SHAPE),
])
def test_cascade_validation(lib, kw, status):
    assert _cascade(lib, **kw) == status
    assert lib.qwen2_last_error().decode()


def test_cascade_validation_fp8_and_zero_work(lib):
    assert _cascade(lib, fp8=True, ksc=0.0) == QW_ERR_SHAPE
    assert _cascade(lib, fp8=True, vsc=float("inf")) == QW_ERR_SHAPE
    assert _cascade(lib, S=0, q=0, out=0) == QW_OK
    assert _cascade(lib, S=0, q=0, out=0, fp8=True) == QW_OK


def test_cascade_workspace_size(lib):
    bf16 = __import__("torch").bfloat16
    plain = B.qwen2_attn_decode_workspace_size(96, 8192, 14, 2, 128, 16, bf16)
    # no group, or a prefix shorter than a block: the plain decode's workspace
    assert B.qwen2_attn_decode_cascade_workspace_size(96, 8192, 0, 0, 0, 14, 2, 128, 16, bf16) == plain
    assert B.qwen2_attn_decode_cascade_workspace_size(96, 8192, 8, 1, 48, 14, 2, 128, 16, bf16) == plain
    # a 1024-token prefix: 8 chunks of 8 blocks, one state row per (chunk, sequence, head)
    n = B.qwen2_attn_decode_cascade_workspace_size(96, 8192, 1024, 1, 48, 14, 2, 128, 16, bf16)
    assert n >= plain + 8 * 96 * 14 * 130 * 4
    assert n <= plain + 8 * 96 * 14 * 130 * 4 + 96 * 8 + 4 * 256
    # chunks stay about 16 for long prefixes, 8..64 blocks each
    m = B.qwen2_attn_decode_cascade_workspace_size(64, 8192, 4096, 4, 64, 28, 4, 128, 16, bf16)
    plain64 = B.qwen2_attn_decode_workspace_size(64, 8192, 28, 4, 128, 16, bf16)
    assert m - plain64 >= 16 * 64 * 28 * 130 * 4
    assert m - plain64 <= 16 * 64 * 28 * 130 * 4 + 64 * 8 + 4 * 256
    assert lib.qwen2_attn_decode_cascade_workspace_size(8, 100, -1, 1, 1, 28, 4, 128, 16, 1) == \
        ctypes.c_size_t(-1).value


def test_cascade_host_checker_agrees_with_oracle_contract(lib):
    """The C host checker and the oracle's check_prefix_groups accept the
    workloads' groupings and refuse the same broken ones."""
    import oracle.reference as R
    for b in (W.mixed_tp2(), W.shared_prompt_decode(num_groups=2, members_per_group=4,
                                                        prefix_len=512)):
        ctx, bt = b.decode_part()
        ind, seqs, lens = b.prefix_groups
        B.qwen2_check_prefix_groups_host(ind, seqs, lens, int(lens.max()), ctx, bt, 16)
        R.check_prefix_groups(bt, ctx, ind, seqs, lens, 16)
    b = W.shared_prompt_decode(num_groups=2, members_per_group=4, prefix_len=512)
    ctx, bt = b.decode_part()
    ind, seqs, lens = b.prefix_groups
    bt_bad = bt.copy()
    bt_bad[5, 3] = bt_bad[5, 3] + 1 if bt_bad[5, 3] + 1 != bt_bad[4, 3] else bt_bad[5, 3] + 2
    broken = [
        (ind, seqs, lens, bt_bad),                                         # member 5 holds another block
        (ind, np.array([0, 1, 2, 3, 4, 5, 6, 6], np.int32), lens, bt),     # listed twice
        (ind, seqs, np.array([512, 520], np.int32), bt),                   # partial block
        (ind, seqs, np.array([512, 4096], np.int32), bt),                  # prefix reaches the context
        (np.array([0, 3, 8], np.int32), seqs, lens, bt),                   # member 3 in group 0's ids
    ]
    for ind_, seqs_, lens_, bt_ in broken:
        with pytest.raises(B.QwenAttnError):
            B.qwen2_check_prefix_groups_host(ind_, seqs_, lens_, 4096, ctx, bt_, 16)
        with pytest.raises(ValueError):
            R.check_prefix_groups(bt_, ctx, ind_, seqs_, lens_, 16)


# ---------------------------------------------------------------------------
# qwen2_attn_decode_paged_noalloc: validation happens before the per-device
# scratch lookup, so every refused call below touches no device state
NOALLOC_SCRATCH = 9 << 20


def _decode_noalloc(lib, **kw):
    a = dict(q=P, qs=28 * 128, kc=P2, vc=P3, nb=100, bt=P, mb=64, ctx=P, out=P2, os=28 * 128,
             S=4, maxc=1024, H=28, Hkv=4, d=128, B=16, scale=0.0884, dt=1)
    a.update(kw)
    return lib.qwen2_attn_decode_paged_noalloc(a["q"], a["qs"], a["kc"], a["vc"], a["nb"], a["bt"],
                                               a["mb"], a["ctx"], a["out"], a["os"], a["S"],
                                               a["maxc"], a["H"], a["Hkv"], a["d"], a["B"],
                                               a["scale"], a["dt"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), QW_ERR_NULL),
    (dict(out=0), QW_ERR_NULL),
    (dict(bt=0), QW_ERR_NULL),
    (dict(H=30), QW_ERR_SHAPE),
    (dict(B=48), QW_ERR_UNSUPPORTED),
    (dict(q=MIS), QW_ERR_ALIGN),
    (dict(mb=8), QW_ERR_SHAPE),
    (dict(S=-1), QW_ERR_SHAPE),
])
def test_decode_noalloc_validation(lib, kw, status):
    assert _decode_noalloc(lib, **kw) == status
    assert lib.qwen2_last_error().decode()


def test_decode_noalloc_zero_work_and_scratch_bound(lib):
    assert _decode_noalloc(lib, S=0, q=0, out=0) == QW_OK
    # the largest decode plans (most ranges, group 8) fit the static scratch
    bf16 = __import__("torch").bfloat16
    for S, c, H, Hkv in ((65535, 131072, 32, 4), (64, 32768, 28, 4), (1, 1, 8, 1)):
        n = B.qwen2_attn_decode_workspace_size(S, c, H, Hkv, 128, 16, bf16)
        assert 0 < n <= NOALLOC_SCRATCH, (S, c, H, Hkv, n)
    text = open(HEADER).read()
    assert "#define QWEN2_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)9 << 20)" in text


def test_cascade_worthwhile_rule(lib):
    """The library's estimate of when the cascade pays: saved prefix KV bytes
    of at least 96 MiB (host-only function)."""
    f = lib.qwen2_attn_decode_cascade_worthwhile
    mixed = W.mixed_tp2()
    ind, seqs, lens = mixed.prefix_groups
    # the TP=2 mixed batch: 48 members of one 1024-token prefix over 2 KV heads (~49 MB)
    assert f(len(lens), len(seqs), int(max(lens)), 2, 128, 0) == 0
    # 4 groups of 16 sequences over 4096-token prefixes, 4 KV heads (~503 MB)
    assert f(4, 64, 4096, 4, 128, 0) == 1
    assert f(4, 64, 4096, 4, 128, 1) == 1                  # FP8: half the bytes, still above
    # the threshold itself: 96 MiB exactly
    n = 96 * 1024 * 1024 // (2 * 128 * 2)                  # tokens x heads x members saved
    assert f(1, 1 + n // 1024, 1024, 1, 128, 0) == 1
    assert f(1, n // 1024, 1024, 1, 128, 0) == 0
    for bad in ((0, 5, 1024, 2, 128, 0), (2, 2, 1024, 2, 128, 0), (1, 5, 0, 2, 128, 0),
                (-1, 5, 1024, 2, 128, 0), (1, 5, 1024, 0, 128, 0)):
        assert f(*bad) == 0
