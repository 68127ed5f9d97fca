"""Benchmark of the paged GQA attention path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]

Headline workload: Qwen2-7B-shaped long-context paged decode, bf16 (28 query
heads, 4 KV heads, head_dim 128, block 16, batch 64, contexts log-uniform in
[2048, 32768]).  One step = qwen2_rope_cache_write of the 64 new tokens (rotate
q/k, write k/v into the paged cache) + qwen2_attn_decode_paged (counter
reset + stream kernel, which also merges shared segments).  ``value`` is KV bytes read per step divided
by the step time (GB/s), inputs resident in HBM.  The K timed steps are
captured in one HIP graph and replayed once between HIP events on the
launching stream, so the figures are GPU time without the Python call cost;
per-call figures come from graphs of K calls of that call alone.  The KV pool (~2.2 GB) is far
larger than the 256 MB last-level cache, so every step streams KV from HBM.

Also reported on the same line: Qwen2-7B varlen causal prefill (8 sequences
of 128..512 tokens) TFLOP/s over a bf16 and over an FP8 cache, the mixed
TP=2-share batch in tokens/s, the long
decode over an FP8 E4M3FN cache, the Qwen3 q/k-norm cache write, the
shared-prefix (cascade) decode against the plain decode, plus the
roofline of the decode call and the CPU oracle baseline.
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")
DECODE_SOURCES = ("decode.hip", "common.h", "kernels.h")
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix-core peak


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _events(n):
    import torch
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def _graph(fn, reps):
    """Capture `reps` back-to-back calls of fn (on a side stream, as torch
    requires) into one HIP graph.  The library calls allocate nothing and
    record no memsets, so a replay re-runs exactly the captured kernels."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                                     # warm the call path outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    torch.cuda.synchronize()
    return g


def _time(fn, steps, warmup):
    """Mean GPU ms per call of fn: `warmup` eager calls, then one replay of a
    graph holding `steps` calls, bracketed by HIP events on the launching
    stream (the graph amortizes its launch over the steps and the replay
    carries no Python call cost).  Also returns the wall ms per call."""
    import torch
    for _ in range(warmup):
        fn()
    g = _graph(fn, steps)
    g.replay()                                   # first replay uploads the graph
    torch.cuda.synchronize()
    e0, e1 = _events(2)
    t0 = time.perf_counter()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps * 1e3
    return e0.elapsed_time(e1) / steps, wall


def bench_decode(steps, warmup):
    from paged_gqa_attention_neox_amd import runner
    from paged_gqa_attention_neox_amd import workloads as W

    log("generating the long-context decode workload")
    b = W.qwen2_long_decode()
    dev = runner.DeviceStep(b)

    def step():
        dev.rope_write()
        dev.decode()
    step_ms, wall = _time(step, steps, warmup)
    rope_ms, _ = _time(dev.rope_write, steps, warmup)
    dec_ms, _ = _time(dev.decode, steps, warmup)
    return dict(batch=b, wall_ms=wall, step_ms=step_ms, rope_ms=rope_ms, decode_ms=dec_ms,
                kv_bytes=b.decode_kv_bytes(), decode_alg_bytes=b.decode_bytes(),
                rope_bytes=b.rope_write_bytes())


def _time_cold(fn, reps, flush):
    """GPU ms of fn with the last-level cache flushed before each call: a
    read of all of `flush` (larger than the 256 MB cache) is enqueued first,
    then fn between HIP events on the launching stream; the read keeps the
    GPU busy while the call is enqueued, so the events see no launch gap.
    The flush reads rather than writes: a write fill leaves the cache full of
    dirty lines whose write-back would then compete with fn's reads (on the
    long decode that adds ~64 us that belong to the fill).  Returns the
    median and the per-call list."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    fn()
    for e0, e1 in ev:
        flush.sum(dtype=torch.int64)
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    t = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    return t[len(t) // 2], t


def bench_achievable():
    """Streaming references measured on this GPU, context beside the published
    8 TB/s peak (the roofline peak stays the published one): a read-only
    reduction over 2 GiB (torch's sum) and a 1 GiB device-to-device copy
    (read + write bytes), each timed eagerly between HIP events over 10
    launches after 3 warm-up launches (the reduction records memsets, so it
    is not captured in a graph)."""
    import torch
    x = torch.ones(1 << 29, dtype=torch.float32, device="cuda")     # 2 GiB
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB
    dst = torch.empty_like(src)

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = _events(2)
        e0.record()
        for _ in range(10):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 10

    read_ms = timed(lambda: x.sum())
    copy_ms = timed(lambda: dst.copy_(src))
    res = {"read_2GiB_sum_GB/s": round(x.numel() * 4 / (read_ms * 1e-3) / 1e9, 1),
           "copy_1GiB_read_plus_write_GB/s": round(2 * src.numel() * 4 / (copy_ms * 1e-3) / 1e9, 1)}
    del x, src, dst
    torch.cuda.empty_cache()
    return res


def bench_cold(reps):
    """Decode with a cold last-level cache: the Qwen3-0.6B-shaped decode
    (batch 32, contexts U[128, 2048]: 143 MB of KV, which a warm 256 MB cache
    would hold) and the Qwen2-7B long decode (a cross-check of the
    graph-timed headline)."""
    import torch
    from paged_gqa_attention_neox_amd import runner
    from paged_gqa_attention_neox_amd import workloads as W

    flush = torch.ones(512 << 20, dtype=torch.uint8, device="cuda")
    out = {}
    for name, mk in (("qwen3_decode", W.qwen3_decode), ("qwen2_long_decode", W.qwen2_long_decode)):
        b = mk()
        dev = runner.DeviceStep(b)
        dev.rope_write()
        med, _ = _time_cold(dev.decode, reps, flush)
        out[name] = dict(decode_ms=med, alg_bytes=b.decode_bytes(), kv_bytes=b.decode_kv_bytes(),
                         seqs=b.num_seqs)
        del dev
    del flush
    return out


def bench_decode_fp8(steps, warmup):
    """The long-context decode with an FP8 (E4M3FN) KV cache: half the KV bytes."""
    from paged_gqa_attention_neox_amd import runner
    from paged_gqa_attention_neox_amd import workloads as W

    log("generating the long-context decode workload with an FP8 cache")
    b = W.qwen2_long_decode_fp8()
    dev = runner.DeviceStep(b)

    def step():
        dev.rope_write()
        dev.decode()
    step_ms, _ = _time(step, steps, warmup)
    dec_ms, _ = _time(dev.decode, steps, warmup)
    return dict(step_ms=step_ms, decode_ms=dec_ms, kv_bytes=b.decode_kv_bytes(),
                alg_bytes=b.decode_bytes(), seqs=b.num_seqs)


def bench_qknorm(steps, warmup):
    """Qwen3 q/k RMSNorm fused into the rope + cache write, on the prefill
    batch (the largest token count): its cost over the plain write."""
    from paged_gqa_attention_neox_amd import runner
    from paged_gqa_attention_neox_amd import workloads as W

    b = W.with_qk_norm(W.qwen2_prefill(), 3)
    dev = runner.DeviceStep(b)
    ms, _ = _time(dev.rope_write, steps, warmup)
    return dict(tokens=b.num_tokens, ms=ms, bytes=b.rope_write_bytes())


def bench_decode_131k(steps, warmup):
    """Qwen2-7B decode at 65k-131k contexts with the dynamic-NTK (factor 4)
    rope table: the same kernels over positions past the native window."""
    from paged_gqa_attention_neox_amd import runner
    from paged_gqa_attention_neox_amd import workloads as W

    log("generating the 131k-context decode workload")
    b = W.qwen2_131k_decode()
    dev = runner.DeviceStep(b)

    def step():
        dev.rope_write()
        dev.decode()
    step_ms, _ = _time(step, steps, warmup)
    dec_ms, _ = _time(dev.decode, steps, warmup)
    res = dict(step_ms=step_ms, decode_ms=dec_ms, kv_bytes=b.decode_kv_bytes(),
               alg_bytes=b.decode_bytes(), seqs=b.num_seqs, mean_ctx=float(b.context_lens.mean()))
    del dev
    return res


def bench_prefill(steps, warmup):
    from paged_gqa_attention_neox_amd import runner
    from paged_gqa_attention_neox_amd import workloads as W

    b = W.qwen2_prefill()
    dev = runner.DeviceStep(b)
    rope_ms, _ = _time(dev.rope_write, steps, warmup)
    pf_ms, _ = _time(dev.prefill, steps, warmup)
    return dict(tokens=b.num_tokens, flops=b.prefill_flops(), prefill_ms=pf_ms, rope_ms=rope_ms,
                rope_bytes=b.rope_write_bytes())


def bench_prefill_qwen3(steps, warmup):
    """Qwen3-0.6B-shaped prefill (16 q / 8 KV heads: two query heads per KV
    head), 8 sequences of 128..512 tokens."""
    from paged_gqa_attention_neox_amd import runner
    from paged_gqa_attention_neox_amd import workloads as W

    b = W.qwen3_prefill()
    dev = runner.DeviceStep(b)
    dev.rope_write()
    pf_ms, _ = _time(dev.prefill, steps, warmup)
    return dict(tokens=b.num_tokens, flops=b.prefill_flops(), prefill_ms=pf_ms)


def bench_prefill_long_prefix(steps, warmup):
    """Chunked prefill with long key loops: 8 chunks of 256 rows after
    8192-token prefixes (Qwen2-7B heads).  Its work items are long, so it
    shows the kernel's steady-state matrix-core rate, which the short items
    of the headline prefill batch do not reach."""
    from paged_gqa_attention_neox_amd import runner
    from paged_gqa_attention_neox_amd import workloads as W

    b = W.qwen2_prefill_long_prefix()
    dev = runner.DeviceStep(b)
    dev.rope_write()
    # median of three timings: a 0.25 ms call varies by ~5% from one timing
    # to the next (the first is usually the slowest)
    runs = sorted(_time(dev.prefill, steps, warmup)[0] for _ in range(3))
    return dict(tokens=b.num_tokens, flops=b.prefill_flops(), prefill_ms=runs[1], runs_ms=runs)


def bench_prefill_fp8(steps, warmup):
    """The Qwen2-7B prefill over an FP8 (E4M3FN) cache: the same batch, the
    cache written as codes by the FP8 rope + cache write."""
    from paged_gqa_attention_neox_amd import runner
    from paged_gqa_attention_neox_amd import workloads as W

    b = W.qwen2_prefill_fp8()
    dev = runner.DeviceStep(b)
    rope_ms, _ = _time(dev.rope_write, steps, warmup)
    pf_ms, _ = _time(dev.prefill, steps, warmup)
    return dict(tokens=b.num_tokens, flops=b.prefill_flops(), prefill_ms=pf_ms, rope_ms=rope_ms)


def bench_mixed(steps, warmup):
    from paged_gqa_attention_neox_amd import runner
    from paged_gqa_attention_neox_amd import workloads as W

    b = W.mixed_tp2()
    dev = runner.DeviceStep(b)
    ms, _ = _time(dev.step, steps, warmup)
    ov_ms, _ = _time(dev.step_overlapped, steps, warmup)
    rope_ms, _ = _time(dev.rope_write, steps, warmup)
    pf_ms, _ = _time(dev.prefill, steps, warmup)
    dec_ms, _ = _time(dev.decode, steps, warmup)
    return dict(tokens=b.num_tokens, step_ms=ms, overlapped_ms=ov_ms, rope_ms=rope_ms,
                prefill_ms=pf_ms, decode_ms=dec_ms, prefill_flops=b.prefill_flops(),
                decode_kv_bytes=b.decode_kv_bytes(), decode_alg_bytes=b.decode_bytes())


def bench_cascade(steps, warmup):
    """Shared-prefix (cascade) decode against the plain decode on the same
    batches: the shared-system-prompt decode (4 groups x 16 sequences over one
    4096-token prefix each) and the mixed TP=2 step (48 of its 96 decodes
    share a 1024-token prefix)."""
    from paged_gqa_attention_neox_amd import runner
    from paged_gqa_attention_neox_amd import workloads as W

    out = {}
    b = W.shared_prompt_decode()
    plain = runner.DeviceStep(b)
    plain_ms, _ = _time(plain.decode, steps, warmup)
    casc = runner.DeviceStep(b, k_cache=plain.k_cache, v_cache=plain.v_cache, cascade=True)
    casc_ms, _ = _time(casc.decode, steps, warmup)
    out["shared_prompt"] = dict(plain_ms=plain_ms, cascade_ms=casc_ms,
                                logical_bytes=b.decode_bytes(),
                                unique_bytes=b.decode_cascade_bytes())
    del plain, casc
    m = W.mixed_tp2()
    plain = runner.DeviceStep(m)
    plain_ms, _ = _time(plain.step, steps, warmup)
    casc = runner.DeviceStep(m, k_cache=plain.k_cache, v_cache=plain.v_cache, cascade=True)
    casc_ms, _ = _time(casc.step, steps, warmup)
    auto = runner.DeviceStep(m, k_cache=plain.k_cache, v_cache=plain.v_cache, cascade="auto")
    auto_ms, _ = _time(auto.step, steps, warmup)
    out["mixed"] = dict(plain_ms=plain_ms, cascade_ms=casc_ms, auto_ms=auto_ms,
                        auto_uses_cascade=bool(auto.cascade), tokens=m.num_tokens)
    return out


def _host_info():
    """Host CPU facts for the baseline: logical CPUs, the CPUs this process
    may run on, and the CPU model."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "cpu_model": model}


_CPU_JOB = {}


def _oracle_seq(s):
    """Decode attention of sequence s by the oracle (worker of the all-cores
    timing; the prepared cache lives in _CPU_JOB, inherited at fork)."""
    import oracle.reference as R
    from threadpoolctl import threadpool_limits
    b, q_out, kc, vc = (_CPU_JOB[k] for k in ("batch", "q_out", "kc", "vc"))
    sh = b.shape
    with threadpool_limits(1):
        R.attention_decode(q_out[s:s + 1], kc, vc, b.block_tables[s:s + 1],
                           b.context_lens[s:s + 1], sh.num_heads, sh.num_kv_heads, sh.head_dim,
                           sh.block_size, sh.dtype)
    return s


def cpu_baseline_child(budget_s=10.0):
    """The CPU oracle (as it stands) on the headline decode workload, run in a
    process that never touches the GPU.  Setup (not timed): the workload's
    draws and the oracle's rope + cache write of the new tokens.  Then (a) one
    thread (BLAS limited to 1) takes whole sequences in batch order until
    about budget_s of work is done; (b) all host CPUs this process may use
    (at most 16) each run the same oracle call on whole sequences of the
    batch (a fork pool over sequences, BLAS at 1 thread per worker), timed
    over the whole batch.  Returns the baseline record."""
    import multiprocessing as mp
    import oracle.reference as R
    from threadpoolctl import threadpool_limits
    from paged_gqa_attention_neox_amd import workloads as W
    b = W.qwen2_long_decode()
    sh = b.shape
    q_out, kc, vc = R.rope_cache_write(b.qkv, sh.dtype, b.positions, b.slot_mapping, b.k_cache,
                                       b.v_cache, sh.num_heads, sh.num_kv_heads, sh.head_dim,
                                       sh.block_size, sh.rope_theta)
    kv_of = lambda s: int(b.context_lens[s]) * 2 * sh.num_kv_heads * sh.head_dim * sh.elem_bytes
    t1, kv1, n1 = 0.0, 0, 0
    with threadpool_limits(1):
        for s in range(b.num_seqs):
            t0 = time.perf_counter()
            R.attention_decode(q_out[s:s + 1], kc, vc, b.block_tables[s:s + 1],
                               b.context_lens[s:s + 1], sh.num_heads, sh.num_kv_heads,
                               sh.head_dim, sh.block_size, sh.dtype)
            t1 += time.perf_counter() - t0
            kv1 += kv_of(s)
            n1 += 1
            if t1 >= budget_s:
                break
    host = _host_info()
    workers = max(1, min(16, host["affinity_cpus"]))
    _CPU_JOB.update(batch=b, q_out=q_out, kc=kc, vc=vc)
    order = list(np.argsort(-b.context_lens))          # longest first: even finish
    ctx = mp.get_context("fork")
    with ctx.Pool(workers) as pool:
        pool.map(_oracle_seq, order[:workers])          # start-up outside the timing
        t0 = time.perf_counter()
        pool.map(_oracle_seq, order, chunksize=1)
        tn = time.perf_counter() - t0
    kvn = sum(kv_of(s) for s in range(b.num_seqs))
    total_tokens = int(b.context_lens.sum())
    return {"value": round(kvn / tn / 1e9, 4), "unit": "GB/s", "cores": int(workers),
            "kind": "oracle",
            "sample": f"decode attention of all {b.num_seqs} sequences ({total_tokens} context "
                      f"tokens, {kvn / 1e6:.1f} MB of KV) on {workers} worker processes in "
                      f"{tn:.2f} s, float64 numpy oracle, one BLAS thread per worker",
            "single_thread": {"value": round(kv1 / t1 / 1e9, 4), "unit": "GB/s",
                              "sample": f"the first {n1} of {b.num_seqs} sequences "
                                        f"({kv1 / 1e6:.1f} MB of KV) in {t1:.2f} s"},
            "host": host}


def cpu_baseline():
    """Run cpu_baseline_child in a fresh interpreter (a child process that
    does not inherit this process's GPU state) and return its record."""
    import subprocess
    r = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-baseline-only"],
                       capture_output=True, text=True, timeout=600)
    if r.returncode != 0:
        raise RuntimeError(f"CPU baseline failed ({r.returncode}): {r.stderr[-2000:]}")
    return json.loads(r.stdout.strip().splitlines()[-1])


def decode_traffic():
    """HBM bytes per decode call measured with FETCH_SIZE / WRITE_SIZE counter
    runs (scaled by a plain-copy calibration), as recorded under profiles/;
    None once the decode kernel sources differ from the ones profiled."""
    import hashlib
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(os.path.join(ROOT, "paged_gqa_attention_neox_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return int(rec["traffic_bytes_per_launch"]) if rec.get("sources_sha256") == h.hexdigest() else None


# --profile targets: (workload builder, the DeviceStep call repeated)
PROFILE_CALLS = {
    "prefill": ("qwen2_prefill", "prefill"),
    "prefill_fp8": ("qwen2_prefill_fp8", "prefill"),
    "rope_write": ("qwen2_prefill", "rope_write"),
    "decode": ("qwen2_long_decode", "decode"),
    "decode_fp8": ("qwen2_long_decode_fp8", "decode"),
    "decode_qwen3": ("qwen3_decode", "decode"),
    "mixed_overlapped": ("mixed_tp2", "step_overlapped"),
}


def profile_call(name, reps):
    """Upload one workload, write its cache once, then run one of its calls
    `reps` times eagerly: a short program whose kernels a profiler counts."""
    import torch
    from paged_gqa_attention_neox_amd import runner
    from paged_gqa_attention_neox_amd import workloads as W
    wl, call = PROFILE_CALLS[name]
    dev = runner.DeviceStep(getattr(W, wl)())
    dev.rope_write()
    fn = getattr(dev, call)
    for _ in range(reps):
        fn()
    torch.cuda.synchronize()
    log(f"profile {name}: {reps} calls of {call} on {wl}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only-decode", action="store_true", help="time the decode workload only")
    ap.add_argument("--profile", choices=sorted(PROFILE_CALLS),
                    help="only run one workload's call --steps times, eagerly (no graphs, no "
                         "timing): the target of rocprofv3 counter passes")
    ap.add_argument("--cpu-baseline-only", action="store_true",
                    help="only time the CPU oracle baseline (no GPU use) and print its record")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (3 times), the reference "
                         "for scaling FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.cpu_baseline_only:
        print(json.dumps(cpu_baseline_child()), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the path has no "
              "multi-GPU mode in this build.", file=sys.stderr)
        sys.exit(2)

    import torch
    from paged_gqa_attention_neox_amd import binding
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    binding.lib()
    if args.profile:
        profile_call(args.profile, args.steps)
        return
    if args.copy_calibration:
        src = torch.ones(1 << 29, dtype=torch.int16, device="cuda")     # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": src.numel() * 2, "launches": 3}), flush=True)
        return

    dec = bench_decode(args.steps, args.warmup)
    log(f"decode: step {dec['step_ms']:.3f} ms (rope {dec['rope_ms']:.3f}, decode {dec['decode_ms']:.3f})")
    res = {}
    if not args.only_decode:
        res["prefill"] = bench_prefill(args.steps, args.warmup)
        log(f"prefill: {res['prefill']['prefill_ms']:.3f} ms")
        res["prefill_qwen3"] = bench_prefill_qwen3(args.steps, args.warmup)
        log(f"qwen3 prefill: {res['prefill_qwen3']['prefill_ms']:.3f} ms")
        res["prefill_long"] = bench_prefill_long_prefix(args.steps, args.warmup)
        log(f"long-prefix prefill: {res['prefill_long']['prefill_ms']:.3f} ms")
        res["prefill_fp8"] = bench_prefill_fp8(args.steps, args.warmup)
        log(f"fp8 prefill: {res['prefill_fp8']['prefill_ms']:.3f} ms")
        res["mixed"] = bench_mixed(args.steps, args.warmup)
        log(f"mixed: {res['mixed']['step_ms']:.3f} ms serial, {res['mixed']['overlapped_ms']:.3f} ms overlapped")
        res["fp8"] = bench_decode_fp8(args.steps, args.warmup)
        log(f"fp8 decode: step {res['fp8']['step_ms']:.3f} ms (decode {res['fp8']['decode_ms']:.3f})")
        res["qknorm"] = bench_qknorm(args.steps, args.warmup)
        log(f"q/k-norm rope + cache write: {res['qknorm']['ms']:.4f} ms")
        res["cascade"] = bench_cascade(args.steps, args.warmup)
        log(f"cascade: shared-prompt decode {res['cascade']['shared_prompt']['cascade_ms']:.3f} ms "
            f"(plain {res['cascade']['shared_prompt']['plain_ms']:.3f}), mixed step "
            f"{res['cascade']['mixed']['cascade_ms']:.3f} ms (plain {res['cascade']['mixed']['plain_ms']:.3f})")
        res["ctx131k"] = bench_decode_131k(args.steps, args.warmup)
        log(f"131k decode: step {res['ctx131k']['step_ms']:.3f} ms (decode {res['ctx131k']['decode_ms']:.3f})")
        res["achievable"] = bench_achievable()
        log(f"streaming references: {res['achievable']}")
        res["cold"] = bench_cold(max(5, args.steps))
        log(f"cold-cache decode: qwen3 {res['cold']['qwen3_decode']['decode_ms']:.4f} ms, "
            f"qwen2 long {res['cold']['qwen2_long_decode']['decode_ms']:.4f} ms")

    b = dec["batch"]
    value = dec["kv_bytes"] / (dec["step_ms"] * 1e-3) / 1e9
    achieved = dec["decode_alg_bytes"] / (dec["decode_ms"] * 1e-3) / 1e9
    out = {
        "metric": "paged GQA decode KV-read GB/s (%HBM peak); prefill TFLOP/s; Qwen2-7B shape",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["step_ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "qwen2-7b paged decode: 28 q / 4 kv heads, head_dim 128, block 16, "
                        "batch 64, contexts log-uniform [2048, 32768], seed 4",
            "global_batch": int(b.num_seqs),
            "seq_len": int(b.context_lens.max()),
            "mean_context": float(b.context_lens.mean()),
            "kv_bytes_per_step": int(dec["kv_bytes"]),
            "parallelism": "single-gpu",
        },
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "tokens_per_s": round(b.num_seqs / (dec["step_ms"] * 1e-3), 1),
        "wall_ms_per_step": round(dec["wall_ms"], 4),
        "roofline": {
            "kernel": "qwen2_attn_decode_paged (counter reset + stream kernel with its merges)",
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": decode_traffic(),
            "alg_bytes_per_launch": int(dec["decode_alg_bytes"]),
            "avg_launch_ms": round(dec["decode_ms"], 4),
        },
        "rope_cache_write": {"ms": round(dec["rope_ms"], 4), "bytes": dec["rope_bytes"],
                             "GB/s": round(dec["rope_bytes"] / (dec["rope_ms"] * 1e-3) / 1e9, 2)},
    }
    if "prefill" in res:
        p = res["prefill"]
        tf = p["flops"] / (p["prefill_ms"] * 1e-3) / 1e12
        out["prefill"] = {
            "workload": "qwen2-7b varlen causal prefill: 8 seqs, lengths U[128,512], 28 q / 4 kv, seed 3",
            "tokens": p["tokens"], "causal_gflop": round(p["flops"] / 1e9, 3),
            "prefill_ms": round(p["prefill_ms"], 4), "TFLOP/s": round(tf, 2),
            "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4),
            "rope_cache_write_ms": round(p["rope_ms"], 4),
            "rope_cache_write_GB/s": round(p["rope_bytes"] / (p["rope_ms"] * 1e-3) / 1e9, 2),
            "tokens_per_s": round(p["tokens"] / ((p["prefill_ms"] + p["rope_ms"]) * 1e-3), 1),
        }
    if "prefill_qwen3" in res:
        p = res["prefill_qwen3"]
        tf = p["flops"] / (p["prefill_ms"] * 1e-3) / 1e12
        out["qwen3_0.6b_prefill"] = {
            "workload": "qwen3-0.6b-shaped varlen causal prefill: 8 seqs, lengths U[128,512], "
                        "16 q / 8 kv heads, seed 8",
            "tokens": p["tokens"], "causal_gflop": round(p["flops"] / 1e9, 3),
            "prefill_ms": round(p["prefill_ms"], 4), "TFLOP/s": round(tf, 2),
            "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4),
        }
    if "prefill_long" in res:
        p = res["prefill_long"]
        tf = p["flops"] / (p["prefill_ms"] * 1e-3) / 1e12
        out["long_prefix_prefill"] = {
            "workload": "qwen2-7b chunked prefill: 8 chunks of 256 rows after 8192-token "
                        "prefixes, 28 q / 4 kv, seed 9",
            "tokens": p["tokens"], "causal_gflop": round(p["flops"] / 1e9, 3),
            "prefill_ms": round(p["prefill_ms"], 4), "TFLOP/s": round(tf, 2),
            "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4),
            "timings_ms": [round(x, 4) for x in p["runs_ms"]],
        }
    if "prefill_fp8" in res:
        p = res["prefill_fp8"]
        tf = p["flops"] / (p["prefill_ms"] * 1e-3) / 1e12
        out["fp8_kv_prefill"] = {
            "workload": "the same qwen2-7b varlen causal prefill over an FP8 E4M3FN KV cache "
                        "(k_scale 0.0312, v_scale 0.0287), seed 3",
            "prefill_ms": round(p["prefill_ms"], 4), "TFLOP/s": round(tf, 2),
            "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4),
            "fp8_rope_cache_write_ms": round(p["rope_ms"], 4),
        }
    if "mixed" in res:
        m = res["mixed"]
        best = min(m["step_ms"], m["overlapped_ms"])
        # roofline time of the step: prefill at the MFMA peak plus decode at
        # the HBM peak (the cache write is not counted)
        roof_ms = (m["prefill_flops"] / (BF16_PEAK_TFLOPS * 1e12)
                   + m["decode_alg_bytes"] / (HBM_PEAK_GBS * 1e9)) * 1e3
        out["mixed"] = {
            "workload": "qwen2-7b tp=2 share mixed step: 4x512 prefill chunks + 96 decodes, seed 5",
            "step_ms": round(best, 4),
            "serial_step_ms": round(m["step_ms"], 4),
            "overlapped_step_ms": round(m["overlapped_ms"], 4),
            "rope_cache_write_ms": round(m["rope_ms"], 4),
            "prefill_ms": round(m["prefill_ms"], 4),
            "decode_ms": round(m["decode_ms"], 4),
            "tokens_per_s": round(m["tokens"] / (best * 1e-3), 1),
            "roofline_ms": round(roof_ms, 4),
            "roofline_frac": round(roof_ms / best, 4),
        }
    if "fp8" in res:
        f = res["fp8"]
        out["fp8_kv_decode"] = {
            "workload": "the same qwen2-7b long-context decode with an FP8 E4M3FN KV cache "
                        "(k_scale 0.0312, v_scale 0.0287), seed 4",
            "kv_bytes_per_step": int(f["kv_bytes"]),
            "ms_per_step": round(f["step_ms"], 4),
            "decode_ms": round(f["decode_ms"], 4),
            "kv_read_GB/s": round(f["kv_bytes"] / (f["step_ms"] * 1e-3) / 1e9, 2),
            "decode_alg_GB/s": round(f["alg_bytes"] / (f["decode_ms"] * 1e-3) / 1e9, 2),
            "hbm_frac": round(f["alg_bytes"] / (f["decode_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "tokens_per_s": round(f["seqs"] / (f["step_ms"] * 1e-3), 1),
            "speedup_vs_bf16_cache": round(dec["step_ms"] / f["step_ms"], 3),
        }
    if "qknorm" in res:
        qn = res["qknorm"]
        out["qk_norm_cache_write"] = {
            "workload": "the qwen2-7b prefill batch (seed 3) through the Qwen3 q/k RMSNorm + rope "
                        "+ cache write (weights N(1, 0.1^2), eps 1e-6)",
            "tokens": qn["tokens"],
            "ms": round(qn["ms"], 4),
            "GB/s": round(qn["bytes"] / (qn["ms"] * 1e-3) / 1e9, 2),
            "plain_write_ms": round(res["prefill"]["rope_ms"], 4),
        }
    if "cascade" in res:
        sp, mx = res["cascade"]["shared_prompt"], res["cascade"]["mixed"]
        out["cascade_decode"] = {
            "workload": "qwen2-7b decode, 4 groups x 16 sequences sharing a 4096-token prefix "
                        "each, private suffixes U[256, 2048], seed 7",
            "plain_decode_ms": round(sp["plain_ms"], 4),
            "cascade_decode_ms": round(sp["cascade_ms"], 4),
            "speedup": round(sp["plain_ms"] / sp["cascade_ms"], 3),
            "logical_kv_GB/s": round(sp["logical_bytes"] / (sp["cascade_ms"] * 1e-3) / 1e9, 2),
            "unique_bytes_GB/s": round(sp["unique_bytes"] / (sp["cascade_ms"] * 1e-3) / 1e9, 2),
            "unique_bytes_hbm_frac": round(sp["unique_bytes"] / (sp["cascade_ms"] * 1e-3) / 1e9
                                           / HBM_PEAK_GBS, 4),
            "mixed_step_plain_ms": round(mx["plain_ms"], 4),
            "mixed_step_cascade_ms": round(mx["cascade_ms"], 4),
            "mixed_step_library_choice_ms": round(mx["auto_ms"], 4),
            "mixed_step_library_chooses_cascade": mx["auto_uses_cascade"],
            "mixed_tokens_per_s_cascade": round(mx["tokens"] / (mx["cascade_ms"] * 1e-3), 1),
        }
    if "ctx131k" in res:
        c = res["ctx131k"]
        out["dynamic_ntk_131k_decode"] = {
            "workload": "qwen2-7b decode, batch 8, contexts U[65536, 131072], dynamic-NTK rope "
                        "table (factor 4 over 32768 positions), seed 6",
            "mean_context": round(c["mean_ctx"], 1),
            "kv_bytes_per_step": int(c["kv_bytes"]),
            "ms_per_step": round(c["step_ms"], 4),
            "decode_ms": round(c["decode_ms"], 4),
            "kv_read_GB/s": round(c["kv_bytes"] / (c["step_ms"] * 1e-3) / 1e9, 2),
            "hbm_frac": round(c["alg_bytes"] / (c["decode_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        }
    if "cold" in res:
        q3, q2 = res["cold"]["qwen3_decode"], res["cold"]["qwen2_long_decode"]
        gbs = lambda r: r["alg_bytes"] / (r["decode_ms"] * 1e-3) / 1e9
        out["cold_cache_decode"] = {
            "method": "each call timed alone between HIP events after a 512 MiB read that "
                      "evicts the 256 MB last-level cache (a read leaves no dirty lines to "
                      "write back); median of the calls",
            "qwen3_0.6b_decode": {
                "workload": "qwen3-0.6b-shaped decode: 16 q / 8 kv heads, head_dim 128, block 16, "
                            "batch 32, contexts U[128, 2048], values N(0,1)*0.5, seed 2",
                "kv_bytes": int(q3["kv_bytes"]), "decode_ms": round(q3["decode_ms"], 4),
                "alg_GB/s": round(gbs(q3), 2), "hbm_frac": round(gbs(q3) / HBM_PEAK_GBS, 4),
                "tokens_per_s": round(q3["seqs"] / (q3["decode_ms"] * 1e-3), 1)},
            "qwen2_7b_long_decode": {
                "decode_ms": round(q2["decode_ms"], 4), "alg_GB/s": round(gbs(q2), 2),
                "hbm_frac": round(gbs(q2) / HBM_PEAK_GBS, 4)},
        }
        out["achievable_streaming"] = dict(res["achievable"], note=(
            "torch's generic reduction and copy kernels measured on this GPU: context only, "
            "lower bounds on what a tuned streaming kernel reaches (the decode's stream kernel "
            "runs above both); roofline fractions use the published 8 TB/s peak"))
    if not args.no_cpu:
        log("CPU oracle baseline")
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
