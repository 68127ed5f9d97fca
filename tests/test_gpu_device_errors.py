"""The device error word (qwen2_device_errors), through the C ABI.

Device metadata that breaks the contract (a position outside the rope
table, a slot outside the cache, a block id outside the pool, a context
length or row range that no valid batch has) must never make a kernel
access memory out of bounds; the kernel skips the write or produces NaN and
ORs a flag into the GPU's error word.  Each case corrupts one device array
of an otherwise valid step, from the host, and checks the flag it sets, that
the rows it spoils are NaN (or untouched), and that every other result is
bitwise the result of the same step with valid metadata (or, where the
corruption changes how the decode splits its work, within the oracle
tolerance).
"""
import numpy as np
import pytest
import torch

import oracle.reference as R
from paged_gqa_attention_neox_amd import binding as B
from paged_gqa_attention_neox_amd import runner
from paged_gqa_attention_neox_amd import workloads as W
from gpu_common import check_out, require_gpu, run_oracle, say

pytestmark = pytest.mark.gpu

POS, SLOT, BLOCK, SEQ = (B.DEVICE_ERR_POSITION, B.DEVICE_ERR_SLOT, B.DEVICE_ERR_BLOCK,
                         B.DEVICE_ERR_SEQUENCE)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.fixture(autouse=True)
def _clear():
    B.qwen2_device_errors(clear=True)
    yield
    B.qwen2_device_errors(clear=True)


def _nan_rows(out, dtype):
    return np.isnan(R.to_f64(out, dtype)).reshape(out.shape[0], -1).all(axis=1)


def _batch(seed, dtype="bf16", d=128, ctx=(40, 300, 9, 1700, 70, 1), ql=(40, 17, 1, 1, 1, 1),
           npf=2, **kw):
    return W.small_case(seed, dtype, 28 if d == 128 else 8, 4 if d == 128 else 2, d,
                        context_lens=list(ctx), query_lens=list(ql), num_prefill=npf,
                        keep_logical=False, **kw)


def _clean(b, **kw):
    dev = runner.DeviceStep(b, **kw)
    dev.step()
    res = dev.results()
    assert B.qwen2_device_errors() == 0, "a valid step set device error flags"
    return res


def _spoiled(b, corrupt, **kw):
    """The step with `corrupt(dev)` applied to the device metadata first."""
    dev = runner.DeviceStep(b, **kw)
    corrupt(dev)
    dev.step()
    return dev.results(), B.qwen2_device_errors()


def _rows_of(b, seqs):
    cu = np.concatenate([[0], np.cumsum(b.query_lens)])
    return np.concatenate([np.arange(cu[s], cu[s + 1]) for s in seqs]).astype(np.int64)


def _others_equal(b, res, ref, bad_rows):
    keep = np.setdiff1d(np.arange(b.num_tokens), bad_rows)
    assert np.array_equal(res["out"][keep], ref["out"][keep])


def _others_match_oracle(b, res, bad_seqs, label):
    """The other sequences against the oracle.  A decode context length
    that changes its sequence's block count changes how the decode splits
    the whole batch's work, and with it the summation order (not the
    result) of the other sequences: bitwise equality does not hold."""
    seqs = [s for s in range(b.num_seqs) if s not in bad_seqs]
    ora = run_oracle(b, seqs=seqs)
    check_out(res["out"], ora["out"], b.shape.dtype, rows=_rows_of(b, seqs), what=label)


def test_valid_step_leaves_zero_and_clear_resets():
    b = _batch(900)
    _clean(b)
    dev = runner.DeviceStep(b)
    dev.positions[0] = b.shape.max_position
    dev.rope_write()
    assert B.qwen2_device_errors() == POS
    assert B.qwen2_device_errors(clear=True) == POS
    assert B.qwen2_device_errors() == 0


@pytest.mark.parametrize("bad_pos", [-1, -1000, "max"])
def test_position_out_of_range(bad_pos):
    b = _batch(901)
    ref = _clean(b)
    t = 5
    pos = b.shape.max_position if bad_pos == "max" else bad_pos
    say(f"position {pos} at token {t}")

    def corrupt(dev):
        dev.positions[t] = pos
    res, flags = _spoiled(b, corrupt)
    assert flags == POS
    assert _nan_rows(res["q_out"], "bf16")[t]
    keep = np.arange(b.num_tokens) != t
    assert np.array_equal(res["q_out"][keep], ref["q_out"][keep])
    blk, off = divmod(int(b.slot_mapping[t]), 16)
    assert np.array_equal(res["k_cache"][blk, :, off, :], b.k_cache[blk, :, off, :])
    assert np.array_equal(res["v_cache"][blk, :, :, off], b.v_cache[blk, :, :, off])


@pytest.mark.parametrize("bad_slot", [-2, "pool"])
def test_slot_out_of_range(bad_slot):
    b = _batch(902)
    ref = _clean(b)
    t = 3
    slot = b.k_cache.shape[0] * 16 if bad_slot == "pool" else bad_slot
    say(f"slot {slot} at token {t}")

    def corrupt(dev):
        dev.slots[t] = slot
    res, flags = _spoiled(b, corrupt)
    assert flags == SLOT
    assert np.array_equal(res["q_out"], ref["q_out"])      # q is rotated as usual
    blk, off = divmod(int(b.slot_mapping[t]), 16)
    assert np.array_equal(res["k_cache"][blk, :, off, :], b.k_cache[blk, :, off, :])
    assert np.array_equal(res["v_cache"][blk, :, :, off], b.v_cache[blk, :, :, off])


def test_slot_minus_one_is_no_error():
    b = _batch(903)

    def corrupt(dev):
        dev.slots[3] = -1
    _, flags = _spoiled(b, corrupt)
    assert flags == 0


@pytest.mark.parametrize("which,dtype,d,fp8", [
    ("decode", "bf16", 128, False), ("decode", "bf16", 128, True),
    ("prefill", "bf16", 128, False), ("prefill", "bf16", 128, True),
    ("decode", "f32", 128, False), ("prefill", "bf16", 64, False)])
def test_block_id_out_of_range(which, dtype, d, fp8):
    kw = dict(cache_dtype="fp8", k_scale=W.FP8_K_SCALE, v_scale=W.FP8_V_SCALE) if fp8 else {}
    b = _batch(904, dtype, d, **kw)
    ref = _clean(b)
    pool = b.k_cache.shape[0]
    # decode: sequence 3 (1700 keys, several split ranges), an entry in the
    # middle; prefill: sequence 0, entry 0 (every row attends to it)
    s, e, bad_id = (3, 50, pool) if which == "decode" else (0, 0, -7)
    say(f"{which} {dtype} d{d} fp8={fp8}: block id {bad_id} at sequence {s} entry {e}")

    def corrupt(dev):
        if which == "decode":
            dev.d_bt[s - b.num_prefill, e] = bad_id
        else:
            dev.p_bt[s, e] = bad_id
    res, flags = _spoiled(b, corrupt)
    assert flags == BLOCK
    rows = _rows_of(b, [s])
    assert _nan_rows(res["out"], dtype)[rows].all()
    _others_equal(b, res, ref, rows)


@pytest.mark.parametrize("which,value", [("decode", 0), ("decode", "max+1"), ("decode", -3),
                                         ("prefill", "rows-1"), ("prefill", "max+1")])
def test_context_length_out_of_range(which, value):
    b = _batch(905)
    ref = _clean(b)
    s = 4 if which == "decode" else 1
    n = int(b.query_lens[s])
    maxc = int(b.context_lens[b.num_prefill:].max() if which == "decode"
               else b.context_lens[:b.num_prefill].max())
    c = {"max+1": maxc + 1, "rows-1": n - 1}.get(value, value)
    say(f"{which}: context length {c} at sequence {s}")

    def corrupt(dev):
        if which == "decode":
            dev.d_ctx[s - b.num_prefill] = c
        else:
            dev.p_ctx[s] = c
    res, flags = _spoiled(b, corrupt)
    assert flags == SEQ
    rows = _rows_of(b, [s])
    assert _nan_rows(res["out"], "bf16")[rows].all()
    if which == "prefill":
        _others_equal(b, res, ref, rows)
    else:
        _others_match_oracle(b, res, [s], f"device errors: decode context {c}")


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 128)])
def test_prefill_rows_outside_batch(dtype, d):
    """cu_seqlens ending past num_tokens: the last prefill sequence's rows
    are not written (they keep what the output held)."""
    b = _batch(906, dtype, d)
    ref = _clean(b)
    P = b.num_prefill
    say(f"{dtype}: cu_seqlens[{P}] past the prefill rows")

    def corrupt(dev):
        dev.p_cu[P] = b.num_prefill_tokens + 3
    res, flags = _spoiled(b, corrupt)
    assert flags == SEQ
    rows = _rows_of(b, [P - 1])
    assert _nan_rows(res["out"], dtype)[rows].all()   # untouched: the runner fills out with NaN
    _others_equal(b, res, ref, rows)


def test_prefill_negative_row_count():
    b = _batch(907)
    ref = _clean(b)

    def corrupt(dev):
        dev.p_cu[1] = b.num_prefill_tokens + 1     # sequence 1 gets a negative row count
    res, flags = _spoiled(b, corrupt)
    assert flags & SEQ
    _others_equal(b, res, ref, _rows_of(b, [0, 1]))


def test_cascade_prefix_block_out_of_range():
    ctx = [1100, 1200, 1300, 700, 90]
    b = W.small_case(908, "bf16", 28, 4, 128, context_lens=ctx, query_lens=[1] * len(ctx),
                     num_prefill=0, keep_logical=False)
    W.with_prefix_groups(b, [([0, 1, 2], 1024)])
    ref = _clean(b, cascade=True)
    pool = b.k_cache.shape[0]
    say("cascade: prefix block id out of the pool")

    def corrupt(dev):
        dev.d_bt[0, 10] = pool + 5                 # inside the shared prefix
    res, flags = _spoiled(b, corrupt, cascade=True)
    assert flags == BLOCK
    assert _nan_rows(res["out"], "bf16")[0]
    assert np.array_equal(res["out"][3:], ref["out"][3:])   # outside the group: unchanged


def test_flags_accumulate_across_calls():
    b = _batch(909)
    dev = runner.DeviceStep(b)
    dev.positions[1] = -1
    dev.d_bt[0, 0] = b.k_cache.shape[0]
    dev.step()
    torch.cuda.synchronize()
    assert B.qwen2_device_errors() == POS | BLOCK
