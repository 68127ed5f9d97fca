"""Shared helpers of the GPU parity tests: run a batch on the HIP path and on
the CPU oracle, and compare element by element."""
from __future__ import annotations

import json
import os
import sys

import numpy as np
import torch

import oracle.reference as R
from paged_gqa_attention_neox_amd import binding as B
from paged_gqa_attention_neox_amd import runner

# tolerances the attention outputs must meet against the float64 oracle:
# the stated absolute bars (max-abs, mean-abs) ...
TOL = {"bf16": (2e-2, 2e-3), "f32": (1e-5, 1e-6)}
# ... and, per (row, head), the largest error over head_dim relative to the
# RMS of that oracle output row.  The absolute bars lose their power where
# outputs are small (a long context averages thousands of values: |o| ~ 0.01).
# The relative bar follows from the arithmetic.  The GPU rounds the output
# once: at most half a bf16 step, 2^-8 of |o_e|, and |o_e| is rarely more
# than ~4x the row RMS over 128 dims (2^-6 of the RMS).  It also rounds each
# probability to bf16 before the PV product: relative errors of at most
# 2^-8 with mean zero; over many keys they average out (~2^-8/sqrt(3) of
# the row's own scale, a few times that at the largest of ~1e7 elements),
# over a handful of keys (the first rows of a prefill) they do not, and
# their effect reaches ~2^-8 of max |V_e| again.  The sum of both stays
# below ~2^-5 (the largest ratio observed over the GPU suite is 0.030); the
# bar is 2^-4, which still holds a long-context output to ~6e-4 where the
# absolute bar allows 2e-2.  Two GPU results of the same rows (each rounded
# once) differ by at most the same amount twice over the rounding step, and
# are held to the same bar.  fp32 storage rounds nothing but the output
# (2^-24) and the fp32 sums, so 2^-16 is ample.
REL_RMS = {"bf16": 2.0 ** -4, "f32": 2.0 ** -16}


def say(msg: str) -> None:
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


def require_gpu():
    import pytest
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def run_gpu(batch, k_cache=None, v_cache=None, repeat=1, cascade=False):
    dev = runner.DeviceStep(batch, k_cache=k_cache, v_cache=v_cache, cascade=cascade)
    for _ in range(repeat):
        dev.step()
    return dev.results(), dev


def run_oracle(batch, seqs=None):
    """Oracle step.  ``seqs`` restricts the attention to those sequence ids
    (the cache write always covers every token)."""
    sh = batch.shape
    fp8 = dict(cache_dtype=sh.cache_dtype, k_scale=sh.k_scale, v_scale=sh.v_scale)
    theta = sh.rope_theta
    if sh.rope_scaling is not None:
        theta, rows = R.rope_dynamic_ntk(sh.rope_theta, sh.head_dim, *sh.rope_scaling)
        assert rows == sh.max_position
    q_out, kc, vc = R.rope_cache_write(batch.qkv, sh.dtype, batch.positions, batch.slot_mapping,
                                       batch.k_cache, batch.v_cache, sh.num_heads, sh.num_kv_heads,
                                       sh.head_dim, sh.block_size, theta, **fp8,
                                       q_norm_weight=batch.q_norm_weight,
                                       k_norm_weight=batch.k_norm_weight, rms_eps=sh.rms_eps)
    cu = batch.cu_seqlens_q
    out = np.full((batch.num_tokens, sh.num_heads, sh.head_dim), np.nan)
    ids = range(batch.num_seqs) if seqs is None else seqs
    for s in ids:
        r0, r1 = int(cu[s]), int(cu[s + 1])
        o = R.attention_varlen(q_out[r0:r1], kc, vc, np.array([0, r1 - r0]),
                               batch.context_lens[s:s + 1], batch.block_tables[s:s + 1],
                               sh.num_heads, sh.num_kv_heads, sh.head_dim, sh.block_size, sh.dtype,
                               **fp8)
        out[r0:r1] = o
    return {"q_out": q_out, "k_cache": kc, "v_cache": vc, "out": out}


def bits(a):
    a = np.asarray(a)
    return a.view(np.uint16) if a.dtype == np.uint16 else a.view(np.uint32)


def ulp_bf16(x):
    """Spacing of bf16 at |x| (normal range)."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    _, e = np.frexp(ax)
    return np.ldexp(1.0, e - 8)


def check_rotated(gpu, ora, dtype, what):
    """Rotated q/k in the storage dtype.  The GPU rotates in float64 and rounds
    once, like the oracle, so the stored values are expected bit for bit.
    The two float64 results can differ in the last place (device vs host
    libm), which can move a value across a rounding boundary with a
    probability of order 1e-13 per element: at most one element in a million
    may differ, and then by one unit in the last place only."""
    g = R.to_f64(gpu, dtype)
    o = R.to_f64(ora, dtype)
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    neq = bits(gpu) != bits(ora)
    n_bad = int(neq.sum())
    assert n_bad <= max(0, neq.size // 1_000_000), f"{what}: {n_bad} of {neq.size} elements differ"
    if n_bad:
        d = np.abs(g - o)[neq]
        lim = (ulp_bf16(o[neq]) if dtype == "bf16" else np.abs(o[neq]) * 2.0 ** -23) * 1.0001
        assert np.all(d <= lim), f"{what}: a differing element is off by more than one ulp"


def _log_parity(rec: dict) -> None:
    """Append one record to the JSON-lines file named by QW_PARITY_LOG, if set
    (the observed errors of every output comparison)."""
    path = os.environ.get("QW_PARITY_LOG")
    if not path:
        return
    rec["test"] = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
    with open(path, "a") as f:
        f.write(json.dumps(rec) + "\n")


def check_out(gpu, ora64, dtype, rows=None, what="out"):
    """Attention outputs [T][H][d] against the float64 oracle: the stated
    max-abs / mean-abs bars over all elements, and the per-(row, head) bar
    relative to the RMS of the oracle row.  Returns (max abs, mean abs)."""
    g = R.to_f64(gpu, dtype)
    o = ora64
    if rows is not None:
        g, o = g[rows], o[rows]
    assert np.all(np.isfinite(o)), f"{what}: oracle rows not computed"
    assert np.all(np.isfinite(g)), f"{what}: GPU output has {int((~np.isfinite(g)).sum())} non-finite values"
    d = np.abs(g - o)
    mx, mean = TOL[dtype]
    rms = np.sqrt((o * o).mean(axis=-1))
    rel = d.max(axis=-1) / np.maximum(rms, 1e-30)
    _log_parity({"what": what, "dtype": dtype, "elements": int(d.size), "max_abs": float(d.max()),
                 "mean_abs": float(d.mean()), "max_rel_rms": float(rel.max()),
                 "p99_rel_rms": float(np.quantile(rel, 0.99)),
                 "min_row_rms": float(rms.min()), "bar_rel_rms": REL_RMS[dtype]})
    assert d.max() <= mx, f"{what}: max abs {d.max():.3e} > {mx} (at {np.unravel_index(d.argmax(), d.shape)})"
    assert d.mean() <= mean, f"{what}: mean abs {d.mean():.3e} > {mean}"
    assert rel.max() <= REL_RMS[dtype], (
        f"{what}: error {rel.max():.3e} x the row RMS > {REL_RMS[dtype]:.3e} "
        f"(at row/head {np.unravel_index(rel.argmax(), rel.shape)})")
    return float(d.max()), float(d.mean())


def key_groups(ctx, ql, hkv, h):
    """The prefill launcher's layout choice (one or two key groups), restated
    from its cost estimate so that each case that names a layout is known to
    exercise it.  Two query heads per KV head always take one group."""
    if h == 2 * hkv:
        return 1
    c, n, rows = max(ctx), max(ql), hkv * sum(ql)
    avg = c - 0.5 * n
    t1 = max(4 + c / 32, rows / 32 * (4 + avg / 32) / 256)
    t2 = max(5 + 1.5 * c / 64, rows / 16 * (5 + 1.5 * avg / 64) / 256)
    return 2 if t2 < t1 else 1


def written_mask(batch):
    """Boolean per (block, offset): slots this step writes."""
    B_ = batch.shape.block_size
    m = np.zeros((batch.num_blocks, B_), bool)
    for sl in batch.slot_mapping:
        if sl >= 0:
            m[sl // B_, sl % B_] = True
    return m


def check_caches(batch, res, ora):
    """V cache bitwise equal everywhere; K cache bitwise equal at every slot
    the step does not write and within rounding at the written ones.  FP8
    caches: every code equal, except that at most one written K code in a
    million may be its neighbour (the float64 rotation can differ in the last
    place between device and host, which moves a value across a rounding
    boundary with a probability of order 1e-13)."""
    dt = batch.shape.dtype
    if batch.shape.cache_dtype == "fp8":
        assert np.array_equal(res["v_cache"], ora["v_cache"]), "V codes differ"
        wm = written_mask(batch)
        kg, ko = res["k_cache"], ora["k_cache"]
        diff = np.nonzero(kg != ko)
        assert wm[diff[0], diff[2]].all(), "K codes changed at slots the step does not write"
        n_bad = len(diff[0])
        assert n_bad <= kg.size // 1_000_000, f"K codes: {n_bad} differ"
        if n_bad:
            a = kg[diff].astype(np.int64)
            b = ko[diff].astype(np.int64)
            assert np.all((np.abs(a - b) == 1) & ((a ^ b) < 128)), "K codes differ by more than a step"
        return
    assert np.array_equal(bits(res["v_cache"]), bits(ora["v_cache"])), "V cache differs"
    wm = written_mask(batch)
    kc_g, kc_o = res["k_cache"], ora["k_cache"]
    diff = np.nonzero(bits(kc_g) != bits(kc_o))
    assert wm[diff[0], diff[2]].all(), "K cache changed at slots the step does not write"
    blk, off = np.nonzero(wm)
    check_rotated(kc_g[blk, :, off, :], kc_o[blk, :, off, :], dt, "K cache (written slots)")


def full_check(batch, seqs=None, label=""):
    say(f"{label or batch.name}: GPU step")
    res, _ = run_gpu(batch)
    say(f"{label or batch.name}: oracle")
    ora = run_oracle(batch, seqs=seqs)
    dt = batch.shape.dtype
    check_rotated(res["q_out"], ora["q_out"], dt, "q_out")
    check_caches(batch, res, ora)
    if seqs is None:
        rows = None
    else:
        cu = batch.cu_seqlens_q
        rows = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in seqs])
    mx, mean = check_out(res["out"], ora["out"], dt, rows=rows)
    say(f"{label or batch.name}: out max abs {mx:.3e} mean abs {mean:.3e}")
    return res, ora
