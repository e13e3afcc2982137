"""Benchmark: paged decode tokens/s and achieved KV GB/s at 128K context.

One step is one pass of the decode hot path over one batch: kv_append of one
new token per sequence, the split-KV partial decode over every stored key
(the appended one included), and the log-sum-exp merge.  The new tokens are
stored by the decode launch itself (pkv_paged_attn_decode_append_partials:
the workgroup that reads a sequence's last page writes the row first), so a
step is two launches; --separate-append times kv_append as a launch of its
own instead (three launches, the same results bit for bit).  The default workload
is Llama-3-70B's per-GPU head share at 128K context: batch 8, 16 query / 2 KV
heads, head_dim 128, fp16 K/V in 16-token pages, 131072 keys per sequence.

Prints one JSON line.  `value` is decode tokens/s (batch / step time) with
every input resident in HBM before the timed region.  Steps are eager
launches; with --graph the step's calls are captured once in a HIP graph and
the timed steps are graph replays (on this stack no faster: the graph
launches each kernel node at about the cost of an eager launch).  `roofline` reports the
partial-decode kernel: algorithmic KV bytes per launch over its mean launch
time measured with HIP events on the stream it runs on.  `cpu_baseline` is
the CPU oracle timed on this host's cores on a bounded sample of the same
workload.

`measured_ceilings` holds what the library's probe kernels measure on the
same GPU (1 GiB read sequentially and as randomly placed 4 KiB blocks; bf16
MFMAs on random operands, alone and with the prefill kernel's vector work;
the prefill kernel's tile loop with its LDS operand reads, with and without
that vector work); each roofline carries the matching one as `measured_peak`
beside the nominal peak, and the prefill's also its tile loop's rate.  `system` records the ROCm and runtime versions and amd-smi's clocks.

Extra objects (--extras, all by default) measure the other rows of the hot
path on their own workloads, each with the roofline of its dominant kernel
and a parity check against the oracle (every row, except where noted):
  llama8b_decode the Llama-3-8B decode step (64 sequences, 513..4097 keys)
  tiny_decode    the tiny fp32 decode: latency (p10/p50/p90)
  prefill_chunk  chunked prefill on the matrix cores (MFMA TFLOP/s); parity
                 on one whole (sequence, KV head) pair and rows of the rest
  fp8_prefill    the same prefill over fp8 (e5m2) pools (MFMA TFLOP/s)
  fp8_decode     the 128K decode over fp8 (e4m3) pools (HBM GB/s)
  window_decode  the 128K decode with a 4096-key window and a 128-key sink
  mixed_batch    an 8192-token batch of decode rows and prefill chunks
                 (parity on the decode rows and sampled chunk rows)
  shared_prefix  256 sequences sharing 2048 tokens of pages: the one-pass decode
                 and the shared-prefix (cascade) decode, on logical and unique bytes
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode tokens/s and achieved KV GB/s (fraction of HBM peak) at 128K ctx"

WORKLOAD_TEXT = {
    "llama70b_128k": "Llama-3-70B per-GPU share at 128K: batch 8, 16 q / 2 kv heads, head_dim 128, "
                     "fp16 K/V, page 16, 131072 keys per sequence (131071 stored + 1 appended), "
                     "pages randomly permuted",
    "llama8b": "Llama-3-8B decode: batch 64, 32 q / 8 kv heads, head_dim 128, bf16, page 16, "
               "context 513..4097 (uniform history + 1 appended), pool +10%, pages permuted",
    "prefix": "prefix sharing: 256 sequences over one 2048-token shared prefix + 32..512 unique "
              "tokens, 32 q / 8 kv heads, head_dim 128, bf16, page 16",
    "tiny": "tiny decode: batch 4, 8 q = 8 kv heads, head_dim 64, fp32, page 16, "
            "lengths 37/128/200/511",
}
# Traffic factors measured for a plain copy kernel with the same counters
# (FETCH_SIZE and WRITE_SIZE in KiB per dispatch versus known bytes).


def progress(msg: str) -> None:
    """One progress line on stderr (stdout carries only the JSON line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def host_cores() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except Exception:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except Exception:
        pass
    return platform.processor() or "unknown"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="llama70b_128k", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--split-tokens", type=int, default=0,
                    help="keys per split (multiple of 16); 0 = library rule")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="lower bound on the CPU oracle sample's wall time")
    ap.add_argument("--extras", default="llama8b,tiny,prefill,fp8prefill,fp8,window,mixed,prefix",
                    help="comma-separated extra rows to measure: llama8b, tiny, prefill, "
                         "fp8prefill, fp8, window, mixed, prefix ('' or 'none' for none)")
    ap.add_argument("--prefill", action="store_true", help="same as --extras prefill")
    ap.add_argument("--separate-append", action="store_true",
                    help="store the new tokens with their own kv_append launch")
    ap.add_argument("--graph", action="store_true",
                    help="time the steps as HIP graph replays instead of eager launches")
    ap.add_argument("--no-smi", action="store_true",
                    help="do not query amd-smi for clocks (for runs under a profiler that "
                         "initialises the GPU before this process starts: a child process "
                         "cannot be started then)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one plain copy of this many MiB first (counter calibration)")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="measured HBM traffic per launch (from rocprofv3 counters), if present")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(--gpus must be 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import paged_kv_cache_04_amd as pkv
    from paged_kv_cache_04_amd import accounting as A
    from paged_kv_cache_04_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)          # reads n bytes, writes n bytes
        torch.cuda.synchronize()
        del src, dst

    t_gen = time.time()
    progress(f"generating {args.config}")
    w = W.make(args.config)
    gen_s = time.time() - t_gen
    kc, vc = w.k_cache.to(dev), w.v_cache.to(dev)
    q, bt, cl = w.q.to(dev), w.block_table.to(dev), w.context_lens.to(dev)
    has_append = w.k_new is not None
    if has_append:
        k_new, v_new, slots = w.k_new.to(dev), w.v_new.to(dev), w.slots.to(dev)
    desc = pkv.cache_desc(kc)
    n_split, _ = pkv.decode_plan(desc, w.batch, w.num_q_heads, w.max_context_len,
                                 args.split_tokens)
    ob, total = pkv.binding.partials_bytes(w.batch, w.num_q_heads, n_split, w.head_dim)
    workspace = torch.empty(total, dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device=dev)
    dargs = (q, kc, vc, bt, cl, w.max_context_len, w.scale)

    # one call to each entry point per step, arguments marshalled once
    o_parts, l_parts, _ = pkv.paged_attn_decode_partials(
        *dargs, split_tokens=args.split_tokens, workspace=workspace)
    fused = has_append and not args.separate_append
    call_append = (pkv.binding.prepare_kv_append(kc, vc, k_new, v_new, slots)
                   if has_append and not fused else None)
    # a plan of one split needs no partials and no merge: the decode launch
    # writes the output itself (one launch per step)
    direct = fused and n_split == 1
    if direct:
        call_partials = pkv.binding.prepare_decode_append(
            q, kc, vc, k_new, v_new, bt, cl, w.max_context_len, w.scale, args.split_tokens,
            out, lse)
    elif fused:
        call_partials = pkv.binding.prepare_decode_append_partials(
            q, kc, vc, k_new, v_new, bt, cl, w.max_context_len, w.scale, args.split_tokens,
            workspace)
    else:
        call_partials = pkv.binding.prepare_decode_partials(*dargs, args.split_tokens,
                                                            workspace)
    call_merge = (None if direct else
                  pkv.binding.prepare_merge_states(o_parts, l_parts, out, lse))

    def step(ev=None):
        if call_append is not None:
            call_append()
        if ev is not None:
            ev[0].record()
        call_partials()
        if ev is not None:
            ev[1].record()
        if call_merge is not None:
            call_merge()

    progress(f"timing {args.steps} steps after {args.warmup} warm-up steps")
    for _ in range(args.warmup):
        step()
    _warm(step)          # and at least 40 ms of them: clocks at their steady state
    torch.cuda.synchronize()

    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t_begin.record()
    for i in range(args.steps):
        step()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = t_begin.elapsed_time(t_end)
    eager_ms_per_step = total_ms / args.steps
    ms_per_step = eager_ms_per_step
    # the same K steps again with an event pair around each partial launch
    # (kept out of the timed region: the event packets sit between the kernels)
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    if args.graph:
        # the same three calls per step, replayed as one HIP graph: no launch gaps
        def issue_step():
            if direct:
                pkv.binding.prepare_decode_append(
                    q, kc, vc, k_new, v_new, bt, cl, w.max_context_len, w.scale,
                    args.split_tokens, out, lse)()
                return
            if fused:
                pkv.binding.prepare_decode_append_partials(
                    q, kc, vc, k_new, v_new, bt, cl, w.max_context_len, w.scale,
                    args.split_tokens, workspace)()
            else:
                if has_append:
                    pkv.binding.prepare_kv_append(kc, vc, k_new, v_new, slots)()
                pkv.binding.prepare_decode_partials(*dargs, args.split_tokens, workspace)()
            pkv.binding.prepare_merge_states(o_parts, l_parts, out, lse)()
        t0 = time.perf_counter()
        ms_per_step = _graph_us(issue_step, args.steps, args.warmup) / 1e3
        wall = time.perf_counter() - t0
    kern_us = [e0.elapsed_time(e1) * 1e3 for e0, e1 in events]
    step_kern_us = float(np.mean(kern_us))
    kern_spread = _spread(kern_us)
    # the kernel's own duration: back-to-back launches between one event pair
    # on its stream, so that the per-call event overhead does not count
    kern_avg_us = _back_to_back_us(call_partials, args.steps)
    # the same launch with L2 and the Infinity Cache evicted before it, against
    # the same launch timed warm by its own event pair
    cold_us = _cold_event_us(call_partials, 10)
    _, warm_event_us = _event_times(call_partials, 10)

    system = system_info(query_smi=not args.no_smi)
    progress("measured ceilings (read and matrix-core probes)")
    ceilings = measure_ceilings(dev)

    kv_bytes = A.decode_kv_bytes(w.context_lens.tolist(), w.num_kv_heads, w.head_dim, w.dtype)
    # the fused launch also reads the new rows and stores them in the pools
    kern_bytes = kv_bytes + (A.append_bytes(w.batch, w.num_kv_heads, w.head_dim, w.dtype)
                             if fused else 0)
    achieved = kern_bytes / (kern_avg_us * 1e-6) / 1e9
    tokens_per_s = w.batch / (ms_per_step * 1e-3)

    traffic = None
    if os.path.exists(args.traffic_json):
        try:
            with open(args.traffic_json) as f:
                tj = json.load(f)
            entry = tj.get(args.config)
            if entry and entry.get("kernel_source_sha") == _kernel_sha():
                traffic = entry.get("bytes_per_launch")
        except Exception:
            traffic = None

    # parity of this run's output on sampled rows against the oracle
    parity = None
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import pkvref
        torch.cuda.synchronize()
        got = out.float().cpu().double().numpy().reshape(w.batch * w.num_q_heads, w.head_dim)
        host_k, host_v = w.k_cache, w.v_cache
        cores = host_cores()
        progress(f"CPU oracle baseline on {cores} threads")
        # CPU oracle on the same workload: one full step (append + decode of
        # every row), repeated until at least --cpu-seconds have passed.
        reps, t_cpu = 0, 0.0
        ref = None
        while reps == 0 or (t_cpu < args.cpu_seconds and reps < 50):
            t1 = time.perf_counter()
            if has_append:
                pkvref.kv_append(w.dtype, host_k, host_v, w.k_new, w.v_new, w.slots)
            ref, _ = pkvref.decode(w.dtype, host_k, host_v, w.q, w.block_table, w.context_lens,
                                   w.scale, n_threads=cores)
            t_cpu += time.perf_counter() - t1
            reps += 1
        cpu = {"value": round(w.batch * reps / t_cpu, 3), "unit": "tokens/s", "cores": cores,
               "kind": "oracle",
               "sample": f"{reps} full step(s) of the same workload (kv_append of {w.batch} "
                         f"tokens + fp64 decode of all {w.batch * w.num_q_heads} query rows), "
                         f"{t_cpu:.1f} s on {cores} threads of {cpu_model()}"}
        err = np.abs(got - ref)
        tol = 2e-2 + 1e-2 * np.abs(ref) if w.dtype != "f32" else 1e-5
        parity = {"rows": int(ref.shape[0]), "max_abs_err": float(np.nanmax(err)),
                  "within_tolerance": bool(np.all(err <= tol))}

    line = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "step_launch": "hip graph" if args.graph else "eager",
        "eager_ms_per_step": round(eager_ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) K/V/Q, random page permutation)",
        "config": {"workload": WORKLOAD_TEXT[args.config], "name": args.config,
                   "batch": w.batch, "context_max": w.max_context_len,
                   "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "page_size": w.page_size, "n_split": n_split,
                   "split_tokens": args.split_tokens},
        "kv_gbps": round(kv_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "roofline": {"bound": "hbm",
                     "kernel": f"{_decode_kernel_name(w)} (split-KV partials"
                               f"{', storing the new tokens' if fused else ''})",
                     "achieved": round(achieved, 1), "peak": A.HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / A.HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": kern_bytes,
                     "kernel_avg_us": round(kern_avg_us, 2),
                     "in_step_event_us": round(step_kern_us, 2),
                     "event_us_spread": kern_spread,
                     "measured_peak": ceilings["random_4k_block_read"]["gbps"],
                     "frac_of_measured": round(achieved / ceilings["random_4k_block_read"]["gbps"],
                                               4)},
        "step_launches": (1 if direct else 2 if fused or not has_append else 3),
        "cold_cache": {"event_us": round(cold_us, 2), "warm_event_us": round(warm_event_us, 2),
                       "achieved_gbps": round(kern_bytes / (cold_us * 1e-6) / 1e9, 1)},
        "cpu_baseline": cpu,
        "parity": parity,
        "host_wall_s": round(wall, 4),
        "gen_s": round(gen_s, 1),
        "measured_ceilings": ceilings,
        "system": system,
    }

    extras = [e for e in args.extras.split(",") if e and e != "none"]
    if args.prefill and "prefill" not in extras:
        extras.append("prefill")
    sample = not args.no_cpu_baseline
    if "window" in extras:
        reuse = ((w, (q, kc, vc, bt, cl, k_new, v_new)) if args.config == "llama70b_128k"
                 else None)
        line["window_decode"] = bench_window(args, dev, sample, reuse)
    del kc, vc, workspace
    torch.cuda.empty_cache()
    if "llama8b" in extras:
        line["llama8b_decode"] = bench_llama8b(args, dev, sample, ceilings)
    if "tiny" in extras:
        line["tiny_decode"] = bench_tiny(args, dev, sample)
    if "prefill" in extras:
        line["prefill_chunk"] = bench_prefill(args, dev, sample, ceilings=ceilings)
    if "fp8prefill" in extras:
        line["fp8_prefill"] = bench_prefill(args, dev, sample, "prefill_fp8", ceilings)
    if "fp8" in extras:
        line["fp8_decode"] = bench_fp8(args, dev, sample)
    if "mixed" in extras:
        line["mixed_batch"] = bench_mixed(args, dev, sample)
    if "prefix" in extras:
        line["shared_prefix"] = bench_shared_prefix(args, dev, sample)

    print(json.dumps(line), flush=True)


def _decode_kernel_name(w) -> str:
    """The decode kernel the library runs for this workload: the matrix-core
    kernel for 4, 8 or 16 query heads per KV head, else the vector kernel."""
    g = w.num_q_heads // w.num_kv_heads
    mfma = w.head_dim == 128 and w.dtype in ("f16", "bf16") and g in (4, 8, 16)
    return "decode_mfma_kernel" if mfma else "decode_kernel"


def _kernel_sha() -> str:
    """Hash of the sources the partial-decode kernel is built from; a stored
    traffic figure is reported only while it matches."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_cache_04_amd", "csrc")
    for name in ("decode.hip", "decode_mfma.hip", "pkv_device.h", "pkv_internal.h",
                 "pkv_append.h"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _back_to_back_us(fn, n):
    """Mean microseconds per call of n back-to-back calls of fn() bracketed by
    one pair of HIP events on the current stream."""
    import torch
    _warm(fn)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / n


def _graph_us(issue, n, warmup=5):
    """Mean microseconds per replay of a HIP graph that holds one issue() --
    the step's library calls, prepared and made on torch's capture stream --
    over n back-to-back replays between one event pair."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        issue()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / n


def _cold_event_us(fn, n, scratch_bytes=1 << 30):
    """Mean microseconds of fn() bracketed by HIP events, each call preceded
    (untimed) by a read of a 1 GiB scratch buffer on the same stream, which
    evicts L2 and the 256 MB Infinity Cache and leaves them holding clean
    lines (a write would leave dirty ones to be written back during fn)."""
    import torch
    scratch = torch.ones(scratch_bytes // 4, dtype=torch.float32, device="cuda")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    fn()
    for i, (e0, e1) in enumerate(ev):
        scratch.sum()
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    us = [e0.elapsed_time(e1) * 1e3 for e0, e1 in ev]
    del scratch
    return sum(us) / len(us)


def _event_times(fn, n, warmup=3):
    """Mean and median microseconds of fn() bracketed by HIP events on the
    current stream (the stream the library enqueues on)."""
    import numpy as np
    import torch
    for _ in range(warmup):
        fn()
    _warm(fn)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    for e0, e1 in ev:
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    us = [e0.elapsed_time(e1) * 1e3 for e0, e1 in ev]
    return float(np.mean(us)), float(np.median(us))


def _warm(fn, ms: float = 40.0):
    """Call fn() until at least `ms` of GPU-busy wall time has passed: the
    chip raises its clocks over the first ~25 ms of sustained work (a
    prefill launch settles from 1.1-1.3 ms to ~0.95-1.0 ms), so every row is
    timed at its steady state."""
    import time
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while True:
        fn()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
            if (time.perf_counter() - t0) * 1e3 >= ms:
                return


def _spread(us):
    """Mean and the 10th, 50th and 90th percentiles of per-launch times (us)."""
    import numpy as np
    a = np.asarray(us, dtype=np.float64)
    return {"mean": round(float(a.mean()), 2), "p10": round(float(np.percentile(a, 10)), 2),
            "p50": round(float(np.percentile(a, 50)), 2),
            "p90": round(float(np.percentile(a, 90)), 2), "n": int(a.size)}


def _event_list(fn, n, warmup=3):
    """Per-call microseconds of n calls of fn(), each between its own pair of
    HIP events on the current stream."""
    import torch
    for _ in range(warmup):
        fn()
    _warm(fn)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    for e0, e1 in ev:
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) * 1e3 for e0, e1 in ev]


def system_info(query_smi: bool = True):
    """ROCm and runtime versions, the device, and the clocks amd-smi reports
    (sampled after the timed steps; the maxima are the chip's limits)."""
    import subprocess
    import torch
    info = {"torch": torch.__version__, "hip_runtime": torch.version.hip}
    try:
        with open("/opt/rocm/.info/version") as f:
            info["rocm"] = f.read().strip()
    except OSError:
        info["rocm"] = None
    p = torch.cuda.get_device_properties(0)
    info["device"] = {"arch": p.gcnArchName, "compute_units": p.multi_processor_count,
                      "memory_gib": round(p.total_memory / 2 ** 30, 1),
                      "l2_bytes_per_xcd": getattr(p, "L2_cache_size", None)}
    try:
        if not query_smi:
            raise RuntimeError("amd-smi not queried (--no-smi)")
        r = subprocess.run(["amd-smi", "metric", "--clock", "--json"], capture_output=True,
                           text=True, timeout=30)
        data = json.loads(r.stdout)
        gpu = data["gpu_data"][0] if isinstance(data, dict) else data[0]
        clk = gpu["clock"]
    except Exception:
        clk = None
    if isinstance(clk, dict):
        gfx = [v for k, v in sorted(clk.items()) if k.startswith("gfx_") and isinstance(v, dict)]
        mem = next((v for k, v in sorted(clk.items())
                    if k.startswith("mem") and isinstance(v, dict)), None)
        def mhz(d, key):
            try:
                return d[key]["value"]
            except Exception:
                return None
        info["amd_smi_clock_mhz"] = {
            "gfx_current_per_xcd": [mhz(g, "clk") for g in gfx],
            "gfx_max": mhz(gfx[0], "max_clk") if gfx else None,
            "mem_current": mhz(mem, "clk") if isinstance(mem, dict) else None,
            "sampled": "after the timed steps (idle)"}
    else:
        info["amd_smi_clock_mhz"] = None
    return info


def measure_ceilings(dev):
    """Measured ceilings on this GPU with the library's probe kernels: 1 GiB
    read sequentially and as randomly placed 4 KiB blocks (the decode's
    pattern), best of a few grid sizes; 32x32x16 bf16 MFMAs on random
    operands alone and with the prefill kernel's vector work per MFMA, with
    the shader clock under that load."""
    import torch

    import paged_kv_cache_04_amd as pkv
    nbytes = 1 << 30
    buf = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=dev)
    res = {}
    best = None
    for grid in (4096, 8192, 16384):
        us = _back_to_back_us(lambda: pkv.binding.probe_read(buf, grid=grid), 10)
        best = us if best is None else min(best, us)
    res["sequential_read"] = {"gbps": round(nbytes / (best * 1e-6) / 1e9, 1),
                              "us_per_gib": round(best, 2)}
    gen = torch.Generator(device="cpu").manual_seed(11)
    order = torch.randperm(nbytes // 4096, generator=gen).to(torch.int32).to(dev)
    best = None
    for grid in (8192, 16384):
        us = _back_to_back_us(lambda: pkv.binding.probe_read(buf, order, 4096, grid=grid), 10)
        best = us if best is None else min(best, us)
    res["random_4k_block_read"] = {"gbps": round(nbytes / (best * 1e-6) / 1e9, 1),
                                   "us_per_gib": round(best, 2)}
    del buf, order
    ops = torch.randn(2048, generator=gen).to(torch.bfloat16).to(dev)
    clocks = torch.zeros(2, dtype=torch.int64, device=dev)
    iters, grid = 4000, 256
    flops = grid * 8 * iters * 4 * 32768
    for key, vec in (("mfma_bf16_random", False), ("mfma_bf16_random_with_prefill_vector_work", True)):
        us = _back_to_back_us(lambda: pkv.binding.probe_mfma(ops, iters, vec, grid, clocks), 5)
        c = clocks.tolist()
        res[key] = {"tflops": round(flops / (us * 1e-6) / 1e12, 1),
                    "shader_clock_ghz": round(c[0] / max(c[1], 1) * 0.1, 3)}
    # the prefill kernel's tile loop alone (its MFMAs, LDS operand reads and,
    # second, its vector work; no copies or barriers), after ~50 ms of load so
    # that the clock has settled as it has for the kernel
    iters, grid = 1000, 256
    flops = grid * 8 * iters * 2 * 32 * 32768
    for key, vec in (("prefill_tile_loop_lds_operands", False),
                     ("prefill_tile_loop_lds_operands_with_vector_work", True)):
        def run():
            pkv.binding.probe_prefill_loop(ops, iters, vec, grid, clocks)
        for _ in range(15):
            run()
        us = _back_to_back_us(run, 5)
        c = clocks.tolist()
        res[key] = {"tflops": round(flops / (us * 1e-6) / 1e12, 1),
                    "shader_clock_ghz": round(c[0] / max(c[1], 1) * 0.1, 3)}
    torch.cuda.empty_cache()
    return res


def bench_llama8b(args, dev, sample, ceilings):
    """The Llama-3-8B decode step (64 sequences of 513..4097 keys, GQA 4):
    the new token stored by the decode launch, split by the batch's lengths
    as a scheduler that holds them would (pkv_decode_split_for_lens), then
    the merge; the automatic plan (one split, a single launch writing the
    output) beside it."""
    progress("llama8b_decode")
    import torch

    import paged_kv_cache_04_amd as pkv
    from paged_kv_cache_04_amd import accounting as A
    from paged_kv_cache_04_amd import workloads as W

    w = W.make("llama8b")
    kc, vc = w.k_cache.to(dev), w.v_cache.to(dev)
    q, bt, cl = w.q.to(dev), w.block_table.to(dev), w.context_lens.to(dev)
    k_new, v_new = w.k_new.to(dev), w.v_new.to(dev)
    desc = pkv.cache_desc(kc)
    lens = w.context_lens.tolist()
    split = pkv.decode_split_for_lens(desc, w.num_q_heads, lens)
    n_split, _ = pkv.decode_plan(desc, w.batch, w.num_q_heads, w.max_context_len, split)
    _, total = pkv.binding.partials_bytes(w.batch, w.num_q_heads, n_split, w.head_dim)
    ws = torch.empty(total, dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty((w.batch, w.num_q_heads), dtype=torch.float32, device=dev)
    o_parts, l_parts, _ = pkv.paged_attn_decode_partials(
        q, kc, vc, bt, cl, w.max_context_len, w.scale, split_tokens=split, workspace=ws)
    c_part = pkv.binding.prepare_decode_append_partials(q, kc, vc, k_new, v_new, bt, cl,
                                                        w.max_context_len, w.scale, split, ws)
    c_merge = pkv.binding.prepare_merge_states(o_parts, l_parts, out, lse)

    def step():
        c_part()
        c_merge()

    for _ in range(10):
        step()
    step_us = _back_to_back_us(step, 50)
    part_us = _back_to_back_us(c_part, 50)
    part_ev = _spread(_event_list(c_part, 50))
    cold_us = _cold_event_us(c_part, 10)
    out1 = torch.empty_like(q)
    c_direct = pkv.binding.prepare_decode_append(q, kc, vc, k_new, v_new, bt, cl,
                                                 w.max_context_len, w.scale, 0, out1)
    direct_us = _back_to_back_us(c_direct, 50)
    kv_bytes = A.decode_kv_bytes(lens, w.num_kv_heads, w.head_dim, w.dtype)
    kern_bytes = kv_bytes + A.append_bytes(w.batch, w.num_kv_heads, w.head_dim, w.dtype)
    roof = _hbm_roofline("decode_mfma_kernel (split-KV partials, storing the new tokens)",
                         kern_bytes, part_us)
    meas = ceilings["random_4k_block_read"]["gbps"]
    roof["measured_peak"] = meas
    roof["frac_of_measured"] = round(roof["achieved"] / meas, 4)
    roof["event_us_spread"] = part_ev
    res = {"workload": WORKLOAD_TEXT["llama8b"],
           "kv_bytes": int(kv_bytes), "split_tokens": split, "n_split": n_split,
           "tokens_per_s": round(w.batch / (step_us * 1e-6), 1),
           "step_us": round(step_us, 2), "step_launches": 2,
           "kv_gbps_per_step": round(kv_bytes / (step_us * 1e-6) / 1e9, 1),
           "roofline": roof,
           "cold_cache": {"kernel_us": round(cold_us, 2),
                          "achieved_gbps": round(kern_bytes / (cold_us * 1e-6) / 1e9, 1)},
           "automatic_plan_one_launch": {
               "n_split": 1, "call_us": round(direct_us, 2),
               "tokens_per_s": round(w.batch / (direct_us * 1e-6), 1),
               "achieved_gbps": round(kern_bytes / (direct_us * 1e-6) / 1e9, 1)}}
    if sample:
        from oracle import pkvref
        torch.cuda.synchronize()
        pkvref.kv_append(w.dtype, w.k_cache, w.v_cache, w.k_new, w.v_new, w.slots)
        ref, ref_lse = pkvref.decode(w.dtype, w.k_cache, w.v_cache, w.q, w.block_table,
                                     w.context_lens, w.scale, n_threads=host_cores())
        got = out.float().cpu().double().numpy().reshape(ref.shape)
        res["parity"] = _parity(got, ref, w.dtype)
        res["parity"]["lse_max_abs_err"] = float(abs(lse.cpu().double().numpy().reshape(-1)
                                                     - ref_lse).max())
        got1 = out1.float().cpu().double().numpy().reshape(ref.shape)
        res["automatic_plan_one_launch"]["parity"] = _parity(got1, ref, w.dtype)
    return res


def bench_tiny(args, dev, sample):
    """The tiny fp32 decode (4 sequences of 37..511 keys, head_dim 64): a
    launch-bound call, reported as latency; parity of every row."""
    progress("tiny_decode")
    import torch

    import paged_kv_cache_04_amd as pkv
    from paged_kv_cache_04_amd import workloads as W

    w = W.make("tiny")
    kc, vc = w.k_cache.to(dev), w.v_cache.to(dev)
    q, bt, cl = w.q.to(dev), w.block_table.to(dev), w.context_lens.to(dev)
    n_split, ws_bytes = pkv.decode_plan(pkv.cache_desc(kc), w.batch, w.num_q_heads,
                                        w.max_context_len, 0)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)

    def call():
        pkv.paged_attn_decode(q, kc, vc, bt, cl, w.max_context_len, w.scale, out=out,
                              workspace=ws)

    # the C call with its arguments marshalled once, as a serving loop makes it;
    # the Python call above adds its argument checks between the event pair
    prepared = pkv.binding.prepare_decode(q, kc, vc, bt, cl, w.max_context_len, w.scale, 0,
                                          out, workspace=ws)
    spread = _spread(_event_list(prepared, 50, warmup=10))
    res = {"workload": WORKLOAD_TEXT["tiny"], "n_split": n_split,
           "launches": 1 if n_split == 1 else 2,
           "call_event_us": spread,
           "python_call_event_us": _spread(_event_list(call, 50, warmup=10)),
           "back_to_back_us": round(_back_to_back_us(prepared, 50), 2),
           "tokens_per_s": round(w.batch / (spread["p50"] * 1e-6), 1),
           "note": "3.6 MB of K/V, cache resident: latency, no roofline claim"}
    if sample:
        from oracle import pkvref
        torch.cuda.synchronize()
        ref, _ = pkvref.decode(w.dtype, w.k_cache, w.v_cache, w.q, w.block_table,
                               w.context_lens, w.scale, n_threads=host_cores())
        got = out.double().cpu().numpy().reshape(ref.shape)
        res["parity"] = _parity(got, ref, w.dtype)
    return res


def _parity(got, ref, dtype):
    import numpy as np
    err = np.abs(got - ref)
    tol = 2e-2 + 1e-2 * np.abs(ref) if dtype != "f32" else 1e-5
    return {"rows": int(ref.shape[0]), "max_abs_err": float(np.nanmax(err)),
            "within_tolerance": bool(np.all(err <= tol))}


def _hbm_roofline(kernel, nbytes, us):
    from paged_kv_cache_04_amd import accounting as A
    gbps = nbytes / (us * 1e-6) / 1e9
    return {"bound": "hbm", "kernel": kernel, "achieved": round(gbps, 1),
            "peak": A.HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(gbps / A.HBM_PEAK_GBPS, 4),
            "algorithmic_bytes_per_launch": int(nbytes), "kernel_avg_us": round(us, 2)}


def _mfma_roofline(kernel, flops, us, dtype):
    from paged_kv_cache_04_amd import accounting as A
    tf = flops / (us * 1e-6) / 1e12
    peak = A.MFMA_PEAK_TFLOPS[dtype]
    return {"bound": "mfma", "kernel": kernel, "achieved": round(tf, 1), "peak": peak,
            "unit": "TFLOP/s", "frac": round(tf / peak, 4),
            "algorithmic_flops_per_launch": int(flops), "kernel_avg_us": round(us, 2)}


def bench_prefill(args, dev, sample, config="prefill", ceilings=None):
    fp8 = config == "prefill_fp8"
    progress("fp8_prefill" if fp8 else "prefill_chunk")
    import numpy as np
    import torch

    import paged_kv_cache_04_amd as pkv
    from paged_kv_cache_04_amd import accounting as A
    from paged_kv_cache_04_amd import workloads as W

    w = W.make(config)
    kc, vc = w.k_cache.to(dev), w.v_cache.to(dev)
    q, bt, kl = w.q.to(dev), w.block_table.to(dev), w.context_lens.to(dev)
    qi = w.q_indptr.to(dev)
    sc = dict(k_scale=w.k_scale, v_scale=w.v_scale) if fp8 else {}
    if fp8:
        pkv.kv_append_quant(kc, vc, w.k_new.to(dev), w.v_new.to(dev), w.slots.to(dev), **sc)
    else:
        pkv.kv_append(kc, vc, w.k_new.to(dev), w.v_new.to(dev), w.slots.to(dev))
    out = torch.empty_like(q)
    chunk = w.meta["chunk_lens"]

    def run():
        pkv.paged_attn_prefill_chunk(q, kc, vc, qi, bt, kl, max(chunk), w.max_context_len,
                                     w.scale, out=out, **sc)

    us, us_med = _event_times(run, 30)
    flops = A.prefill_flops(w.context_lens.tolist(), chunk, w.num_q_heads, w.head_dim)
    text = ("batch 4, 32768-token paged history + 512-row causal chunk, 32 q / 8 kv heads, "
            "head_dim 128, bf16")
    if fp8:
        text += (" queries over fp8 e5m2 pools with fp32 scales (page 4, section 3.1's "
                 "serving setup), each page widened exactly to bf16 in the kernel")
    res = {"workload": text,
           "kernel_avg_us": round(us, 2), "kernel_median_us": round(us_med, 2),
           "query_tokens_per_s": round(sum(chunk) / (us * 1e-6), 1),
           "roofline": _mfma_roofline("prefill_kernel" + ("<bf16 q, fp8 e5m2 cache>" if fp8 else ""),
                                      flops, us, "bf16")}
    res["kernel_event_us_spread"] = _spread(_event_list(run, 20))
    if ceilings is not None:
        # the matrix cores' measured rate on random operands with the vector
        # work this kernel does per MFMA (no memory traffic, no barriers)
        meas = ceilings["mfma_bf16_random_with_prefill_vector_work"]["tflops"]
        res["roofline"]["measured_peak"] = meas
        res["roofline"]["frac_of_measured"] = round(res["roofline"]["achieved"] / meas, 4)
        # and this kernel's own tile loop, LDS operand reads included, without
        # the page copies and barriers around it
        loop = ceilings["prefill_tile_loop_lds_operands_with_vector_work"]["tflops"]
        res["roofline"]["tile_loop_tflops"] = loop
        res["roofline"]["frac_of_tile_loop"] = round(res["roofline"]["achieved"] / loop, 4)
    if sample:
        from oracle import pkvref
        hq = w.num_q_heads
        g_size = hq // w.num_kv_heads
        # one whole (sequence, KV head) pair -- sequence 0, KV head 0: every
        # chunk row of its query heads -- plus rows of the other sequences
        q0, q1 = int(w.q_indptr[0]), int(w.q_indptr[1])
        rows = [t * hq + h for t in range(q0, q1) for h in range(g_size)]
        toks = [int(w.q_indptr[b]) + i for b in range(1, w.batch) for i in (0, 255, 511)]
        rows += [t * hq + h for t in toks for h in (5, 13, 31)]
        if fp8:
            f8 = W.DTYPES[w.kv_dtype]
            kq = torch.from_numpy(pkvref.quant_fp8(w.kv_dtype, w.dtype, w.k_new, w.k_scale))
            vq = torch.from_numpy(pkvref.quant_fp8(w.kv_dtype, w.dtype, w.v_new, w.v_scale))
            pkvref.kv_append(w.kv_dtype, w.k_cache, w.v_cache, kq.view(f8), vq.view(f8), w.slots)
        else:
            pkvref.kv_append(w.dtype, w.k_cache, w.v_cache, w.k_new, w.v_new, w.slots)
        ref, _ = pkvref.prefill_ex(w.dtype, w.kv_dtype, w.k_cache, w.v_cache, w.q, w.q_indptr,
                                   w.block_table, w.context_lens, w.scale, rows=rows,
                                   n_threads=host_cores(), **sc)
        got = out.float().cpu().double().numpy().reshape(-1, w.head_dim)[rows]
        res["parity"] = _parity(got, ref, w.dtype)
    return res


def bench_fp8(args, dev, sample):
    progress("fp8_decode")
    import torch

    import paged_kv_cache_04_amd as pkv
    from paged_kv_cache_04_amd import workloads as W

    w = W.make("llama70b_128k_fp8")
    kc, vc = w.k_cache.to(dev), w.v_cache.to(dev)
    q, bt, cl = w.q.to(dev), w.block_table.to(dev), w.context_lens.to(dev)
    k_new, v_new, slots = w.k_new.to(dev), w.v_new.to(dev), w.slots.to(dev)
    desc = pkv.cache_desc(kc)
    opts = pkv.decode_opts(q.dtype, kc.dtype, w.k_scale, w.v_scale)
    n_split, _ = pkv.decode_plan(desc, w.batch, w.num_q_heads, w.max_context_len, 0, opts)
    _, total = pkv.binding.partials_bytes(w.batch, w.num_q_heads, n_split, w.head_dim)
    ws = torch.empty(total, dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    o_parts, l_parts, _ = pkv.paged_attn_decode_partials(
        q, kc, vc, bt, cl, w.max_context_len, w.scale, workspace=ws, k_scale=w.k_scale,
        v_scale=w.v_scale)
    # the step: the decode launch that also quantizes and stores the new
    # tokens (or, with --separate-append, kv_append_quant before it), the merge
    sep = args.separate_append

    def parts():
        if sep:
            return pkv.binding.prepare_decode_partials(q, kc, vc, bt, cl, w.max_context_len,
                                                       w.scale, 0, ws, w.k_scale, w.v_scale)
        return pkv.binding.prepare_decode_append_partials(q, kc, vc, k_new, v_new, bt, cl,
                                                          w.max_context_len, w.scale, 0, ws,
                                                          w.k_scale, w.v_scale)

    def app():
        return pkv.binding.prepare_kv_append_quant(kc, vc, k_new, v_new, slots, w.k_scale,
                                                   w.v_scale)

    c_app = app() if sep else None
    c_part = parts()
    c_merge = pkv.binding.prepare_merge_states(o_parts, l_parts, out)

    def step():
        if c_app is not None:
            c_app()
        c_part()
        c_merge()

    def issue_step():
        if sep:
            app()()
        parts()()
        pkv.binding.prepare_merge_states(o_parts, l_parts, out)()

    # steps back to back between one event pair (as the main row's total is
    # taken); an event pair around every step would add its host cost, which
    # exceeds a short step's GPU time
    event_us, _ = _event_times(step, 30, warmup=10)
    eager_us = _back_to_back_us(step, 30)
    step_us = _graph_us(issue_step, 30) if args.graph else eager_us
    _, part_med = _event_times(c_part, 30)
    part_us = _back_to_back_us(c_part, 30)
    cold_us = _cold_event_us(c_part, 20)
    kv_bytes = sum(w.context_lens.tolist()) * 2 * w.num_kv_heads * w.head_dim * 1
    if not sep:   # f16 rows read, fp8 rows stored
        kv_bytes += w.batch * w.num_kv_heads * w.head_dim * 2 * (2 + 1)
    res = {"workload": "Llama-3-70B per-GPU share at 128K over fp8 (OCP e4m3) pools with fp32 "
                       "scales: batch 8, 16 q / 2 kv heads, head_dim 128, f16 queries, page 16, "
                       "131072 keys per sequence (131071 stored + 1 quantized on append)",
           "tokens_per_s": round(w.batch / (step_us * 1e-6), 1), "ms_per_step": round(
               step_us / 1e3, 5), "eager_ms_per_step": round(eager_us / 1e3, 5),
           "per_step_event_ms": round(event_us / 1e3, 5),
           "n_split": n_split, "kernel_median_us": round(part_med, 2),
           "roofline": _hbm_roofline("decode_mfma_kernel<f16 q, fp8 e4m3 cache> (split-KV partials)",
                                     kv_bytes, part_us),
           # 512 MB of fp8 K/V is twice the 256 MB Infinity Cache, which serves part of a
           # warm launch: the same launch with L2 and that cache evicted before it (its own
           # event pair per launch; compare with kernel_median_us)
           "cold_cache": {"kernel_us": round(cold_us, 2),
                          "achieved_gbps": round(kv_bytes / (cold_us * 1e-6) / 1e9, 1)}}
    if sample:
        from oracle import pkvref
        kq = torch.from_numpy(pkvref.quant_fp8(w.kv_dtype, w.dtype, w.k_new, w.k_scale))
        vq = torch.from_numpy(pkvref.quant_fp8(w.kv_dtype, w.dtype, w.v_new, w.v_scale))
        pkvref.kv_append(w.kv_dtype, w.k_cache, w.v_cache, kq.view(W.DTYPES[w.kv_dtype]),
                         vq.view(W.DTYPES[w.kv_dtype]), w.slots)
        rows = list(range(w.batch * w.num_q_heads))      # every row
        ref, _ = pkvref.decode_ex(w.dtype, w.kv_dtype, w.k_cache, w.v_cache, w.q, w.block_table,
                                  w.context_lens, w.scale, k_scale=w.k_scale,
                                  v_scale=w.v_scale, rows=rows, n_threads=host_cores())
        got = out.float().cpu().double().numpy().reshape(-1, w.head_dim)[rows]
        res["parity"] = _parity(got, ref, w.dtype)
    return res


def bench_window(args, dev, sample, reuse=None):
    progress("window_decode")
    import torch

    import paged_kv_cache_04_amd as pkv
    from paged_kv_cache_04_amd import accounting as A
    from paged_kv_cache_04_amd import workloads as W

    window, sink = 4096, 128
    if reuse is not None:      # the main 128K workload, its append already applied
        w, (q, kc, vc, bt, cl, k_new, v_new) = reuse
    else:
        w = W.make("llama70b_128k")
        kc, vc = w.k_cache.to(dev), w.v_cache.to(dev)
        q, bt, cl = w.q.to(dev), w.block_table.to(dev), w.context_lens.to(dev)
        k_new, v_new = w.k_new.to(dev), w.v_new.to(dev)
        pkv.kv_append(kc, vc, k_new, v_new, w.slots.to(dev))
        if sample:
            from oracle import pkvref
            pkvref.kv_append(w.dtype, w.k_cache, w.v_cache, w.k_new, w.v_new, w.slots)
    desc = pkv.cache_desc(kc)
    opts = pkv.decode_opts(q.dtype, kc.dtype, window=window, sink=sink)
    n_split, _ = pkv.decode_plan(desc, w.batch, w.num_q_heads, w.max_context_len, 0, opts)
    _, total = pkv.binding.partials_bytes(w.batch, w.num_q_heads, n_split, w.head_dim)
    ws = torch.empty(total, dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    o_parts, l_parts, _ = pkv.paged_attn_decode_partials(
        q, kc, vc, bt, cl, w.max_context_len, w.scale, workspace=ws, window=window, sink=sink)
    # a decode step as in the main row: the partial launch also stores the new
    # tokens (the same rows again: the pools keep their bits)
    def parts():
        if args.separate_append:
            return pkv.binding.prepare_decode_partials(q, kc, vc, bt, cl, w.max_context_len,
                                                       w.scale, 0, ws, window=window, sink=sink)
        return pkv.binding.prepare_decode_append_partials(q, kc, vc, k_new, v_new, bt, cl,
                                                          w.max_context_len, w.scale, 0, ws,
                                                          window=window, sink=sink)

    c_part = parts()
    c_merge = pkv.binding.prepare_merge_states(o_parts, l_parts, out)

    def step():
        c_part()
        c_merge()

    def issue_step():
        parts()()
        pkv.binding.prepare_merge_states(o_parts, l_parts, out)()

    # steps back to back between one event pair (as the main row's total is
    # taken); an event pair around every step would add its host cost, which
    # exceeds a short step's GPU time
    event_us, _ = _event_times(step, 30, warmup=10)
    eager_us = _back_to_back_us(step, 30)
    step_us = _graph_us(issue_step, 30) if args.graph else eager_us
    _, part_med = _event_times(c_part, 30)
    part_us = _back_to_back_us(c_part, 30)
    cold_us = _cold_event_us(c_part, 20)
    es = 4 if w.dtype == "f32" else 2
    vis = [min(L, window) + min(sink, max(0, L - window)) for L in w.context_lens.tolist()]
    kv_bytes = sum(vis) * 2 * w.num_kv_heads * w.head_dim * es
    if not args.separate_append:
        kv_bytes += A.append_bytes(w.batch, w.num_kv_heads, w.head_dim, w.dtype)
    res = {"workload": "the 128K decode workload with a sliding window: each query sees its "
                       "4096 most recent keys and the first 128 (page 4, section 2.3's local "
                       "window + global tokens); pages wholly outside are not read; the step "
                       "stores the new tokens in its partial launch",
           "tokens_per_s": round(w.batch / (step_us * 1e-6), 1),
           "ms_per_step": round(step_us / 1e3, 5), "eager_ms_per_step": round(eager_us / 1e3, 5),
           "per_step_event_ms": round(event_us / 1e3, 5),
           "n_split": n_split,
           "kernel_median_us": round(part_med, 2),
           "roofline": _hbm_roofline("decode_mfma_kernel (windowed split-KV partials)", kv_bytes,
                                     part_us),
           # the visible K/V (35 MB) fits in the 256 MB Infinity Cache: the same kernel with
           # L2 and that cache evicted before each launch (its own event pair per launch)
           "cold_cache": {"kernel_us": round(cold_us, 2),
                          "achieved_gbps": round(kv_bytes / (cold_us * 1e-6) / 1e9, 1)}}
    if sample:
        from oracle import pkvref
        rows = list(range(w.batch * w.num_q_heads))      # every row
        ref, _ = pkvref.decode_ex(w.dtype, w.dtype, w.k_cache, w.v_cache, w.q, w.block_table,
                                  w.context_lens, w.scale, window=window, sink=sink, rows=rows,
                                  n_threads=host_cores())
        got = out.float().cpu().double().numpy().reshape(-1, w.head_dim)[rows]
        res["parity"] = _parity(got, ref, w.dtype)
    return res


def bench_shared_prefix(args, dev, sample):
    progress("shared_prefix")
    import torch

    import paged_kv_cache_04_amd as pkv
    from paged_kv_cache_04_amd import accounting as A
    from paged_kv_cache_04_amd import workloads as W

    w = W.make("prefix")
    kc, vc = w.k_cache.to(dev), w.v_cache.to(dev)
    q, bt, cl = w.q.to(dev), w.block_table.to(dev), w.context_lens.to(dev)
    prefix = w.meta["shared_prefix"]
    pp = prefix // w.page_size
    prefix_table = bt[0, :pp].contiguous()
    own = bt[:, pp:]
    suffix_lens = (cl - prefix).contiguous()
    max_suffix = w.max_context_len - prefix
    desc = pkv.cache_desc(kc)
    n_parts, ws_bytes = pkv.shared_prefix_plan(desc, w.batch, w.num_q_heads, prefix, max_suffix)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    out1 = torch.empty_like(q)
    n1, ws1_bytes = pkv.decode_plan(desc, w.batch, w.num_q_heads, w.max_context_len, 0)
    ws1 = torch.empty(max(ws1_bytes, 16), dtype=torch.uint8, device=dev)

    def one_pass():
        pkv.paged_attn_decode(q, kc, vc, bt, cl, w.max_context_len, w.scale, out=out1,
                              workspace=ws1)

    def cascade():
        pkv.paged_attn_decode_shared_prefix(q, kc, vc, prefix_table, prefix, own, suffix_lens,
                                            max_suffix, w.scale, out=out, workspace=ws)

    lens = w.context_lens.tolist()
    logical = A.decode_kv_bytes(lens, w.num_kv_heads, w.head_dim, w.dtype)
    unique = A.decode_kv_bytes([prefix] + [L - prefix for L in lens], w.num_kv_heads,
                               w.head_dim, w.dtype)
    one_us, _ = _event_times(one_pass, 30, warmup=5)
    cas_us, cas_med = _event_times(cascade, 30, warmup=5)
    cold_us = _cold_event_us(cascade, 10)
    res = {"workload": "256 sequences sharing 2048 tokens (128 physical pages in every table) "
                       "+ U{32..512} own tokens, 32 q / 8 kv heads, head_dim 128, bf16 (page 2, "
                       "section 3.2: identical prefixes share physical pages)",
           "logical_kv_bytes": int(logical), "unique_kv_bytes": int(unique),
           "one_pass_decode": {"call_us": round(one_us, 2), "n_split": n1,
                               "tokens_per_s": round(w.batch / (one_us * 1e-6), 1),
                               "logical_gbps": round(logical / (one_us * 1e-6) / 1e9, 1),
                               "unique_gbps": round(unique / (one_us * 1e-6) / 1e9, 1)},
           "cascade": {"call_us": round(cas_us, 2), "call_median_us": round(cas_med, 2),
                       "n_parts": n_parts,
                       "tokens_per_s": round(w.batch / (cas_us * 1e-6), 1),
                       "logical_gbps": round(logical / (cas_us * 1e-6) / 1e9, 1),
                       "cold_call_us": round(cold_us, 2)},
           # the cascade reads each unique byte once: its roofline is HBM on unique bytes
           "roofline": _hbm_roofline("shared-prefix decode (3 launches: shared pages on MFMA, "
                                     "own pages split-KV, merge)", unique, cas_us)}
    if sample:
        from oracle import pkvref
        torch.cuda.synchronize()
        rows = list(range(w.batch * w.num_q_heads))      # every row
        ref, _ = pkvref.decode(w.dtype, w.k_cache, w.v_cache, w.q, w.block_table,
                               w.context_lens, w.scale, rows=rows, n_threads=host_cores())
        got = out.float().cpu().double().numpy().reshape(-1, w.head_dim)[rows]
        res["parity"] = _parity(got, ref, w.dtype)
    del kc, vc
    torch.cuda.empty_cache()
    return res


def bench_mixed(args, dev, sample):
    progress("mixed_batch")
    import torch

    import paged_kv_cache_04_amd as pkv
    from paged_kv_cache_04_amd import accounting as A
    from paged_kv_cache_04_amd import workloads as W

    w = W.make("mixed")
    kc, vc = w.k_cache.to(dev), w.v_cache.to(dev)
    q, bt, kl, qi = w.q.to(dev), w.block_table.to(dev), w.context_lens.to(dev), w.q_indptr.to(dev)
    pkv.kv_append(kc, vc, w.k_new.to(dev), w.v_new.to(dev), w.slots.to(dev))
    nd = w.meta["num_decode"]
    chunk = w.meta["chunk_lens"]
    max_q = max(chunk[nd:])
    # the scheduler knows the decode rows' lengths: split them by the batch's pages
    split = pkv.decode_split_for_lens(pkv.cache_desc(kc), w.num_q_heads,
                                      w.context_lens[:nd].tolist())
    _, ws_bytes = pkv.decode_plan(pkv.cache_desc(kc), nd, w.num_q_heads, w.max_context_len,
                                  split)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)

    def run():
        pkv.paged_attn_mixed(q, kc, vc, qi, bt, kl, nd, max_q, w.max_context_len, w.scale,
                             split_tokens=split, out=out, workspace=ws)

    eager_us, us_med = _event_times(run, 10)
    us = _graph_us(run, 10) if args.graph else eager_us
    # the chunk part alone (the MFMA kernel) and the decode part alone
    qi_c, bt_c, kl_c = qi[nd:].contiguous(), bt[nd:].contiguous(), kl[nd:].contiguous()
    pf_us, _ = _event_times(lambda: pkv.paged_attn_prefill_chunk(
        q, kc, vc, qi_c, bt_c, kl_c, max_q, w.max_context_len, w.scale, out=out), 10)
    # the decode part alone: its two kernels, prepared and launched back to back
    q_d, bt_d, kl_d = q[:nd].contiguous(), bt[:nd].contiguous(), kl[:nd].contiguous()
    o_d = torch.empty_like(q_d)
    o_parts, l_parts, _ = pkv.paged_attn_decode_partials(
        q_d, kc, vc, bt_d, kl_d, w.max_context_len, w.scale, split_tokens=split, workspace=ws)
    c_part = pkv.binding.prepare_decode_partials(q_d, kc, vc, bt_d, kl_d, w.max_context_len,
                                                 w.scale, split, ws)
    c_merge = pkv.binding.prepare_merge_states(o_parts, l_parts, o_d)

    def dec():
        c_part()
        c_merge()

    dec_us = _back_to_back_us(dec, 20)
    # the decode rows read 321 MB, close to the 256 MB Infinity Cache: calls
    # back to back can find part of it there, so the cache-cold time is given too
    dec_cold_us = _cold_event_us(dec, 10)
    lens = w.context_lens.tolist()
    flops = A.prefill_flops(lens[nd:], chunk[nd:], w.num_q_heads, w.head_dim)
    dec_bytes = A.decode_kv_bytes(lens[:nd], w.num_kv_heads, w.head_dim, w.dtype)
    res = {"workload": "one chunked-prefill batch under page 1's 8192-token budget: 6 sequences "
                       "decoding at 8K..128K keys + two 4093-row prompt chunks (history 0 and "
                       "65536), 16 q / 2 kv heads, head_dim 128, f16, decode rows first",
           "query_tokens": int(sum(chunk)), "decode_split_tokens": split,
           "call_avg_us": round(us, 2),
           "eager_call_avg_us": round(eager_us, 2), "eager_call_median_us": round(us_med, 2),
           "query_tokens_per_s": round(sum(chunk) / (us * 1e-6), 1),
           "roofline": _mfma_roofline("prefill_kernel (the batch's chunks)", flops, pf_us, "f16"),
           "decode_rows": _hbm_roofline("decode_mfma_kernel + merge (the batch's decode rows)",
                                        dec_bytes, dec_us)}
    res["decode_rows"]["cold_cache"] = {"us": round(dec_cold_us, 2),
                                        "achieved_gbps": round(dec_bytes / (dec_cold_us * 1e-6) / 1e9, 1)}
    if sample:
        from oracle import pkvref
        hq = w.num_q_heads
        ind = w.q_indptr.tolist()
        toks = list(range(nd)) + [ind[b] + i for b in range(nd, w.batch) for i in (0, 2046, 4092)]
        rows = [t * hq + h for t in toks for h in (0, 15)]
        pkvref.kv_append(w.dtype, w.k_cache, w.v_cache, w.k_new, w.v_new, w.slots)
        run()
        torch.cuda.synchronize()
        ref, _ = pkvref.prefill(w.dtype, w.k_cache, w.v_cache, w.q, w.q_indptr, w.block_table,
                                w.context_lens, w.scale, rows=rows, n_threads=host_cores())
        got = out.float().cpu().double().numpy().reshape(-1, w.head_dim)[rows]
        res["parity"] = _parity(got, ref, w.dtype)
    return res


if __name__ == "__main__":
    main()
