"""Benchmark: paged decode tokens/s and achieved KV GB/s at 128K context.

One step is one pass of the decode hot path over one batch: kv_append of one
new token per sequence, the split-KV partial decode over every stored key
(the appended one included), and the log-sum-exp merge.  The default workload
is Llama-3-70B's per-GPU head share at 128K context: batch 8, 16 query / 2 KV
heads, head_dim 128, fp16 K/V in 16-token pages, 131072 keys per sequence.

Prints one JSON line.  `value` is decode tokens/s (batch / step time) with
every input resident in HBM before the timed region.  `roofline` reports the
partial-decode kernel: algorithmic KV bytes per launch over its mean launch
time measured with HIP events on the stream it runs on.  `cpu_baseline` is
the CPU oracle timed on this host's cores on a bounded sample of the same
workload.  `--prefill` adds the chunked-prefill kernel's MFMA figure.
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
    ap.add_argument("--prefill", action="store_true",
                    help="also time the chunked-prefill kernel (batch 4, 32768 history + 512 chunk)")
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
    call_append = (pkv.binding.prepare_kv_append(kc, vc, k_new, v_new, slots)
                   if has_append else None)
    call_partials = pkv.binding.prepare_decode_partials(*dargs, args.split_tokens, workspace)
    call_merge = pkv.binding.prepare_merge_states(o_parts, l_parts, out, lse)

    def step(ev=None):
        if call_append is not None:
            call_append()
        if ev is not None:
            ev[0].record()
        call_partials()
        if ev is not None:
            ev[1].record()
        call_merge()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t_begin.record()
    for i in range(args.steps):
        step(events[i])
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = t_begin.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    kern_us = [e0.elapsed_time(e1) * 1e3 for e0, e1 in events]
    kern_avg_us = float(np.mean(kern_us))

    kv_bytes = A.decode_kv_bytes(w.context_lens.tolist(), w.num_kv_heads, w.head_dim, w.dtype)
    achieved = kv_bytes / (kern_avg_us * 1e-6) / 1e9
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
        "roofline": {"bound": "hbm", "kernel": "decode_kernel (split-KV partials)",
                     "achieved": round(achieved, 1), "peak": A.HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / A.HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": kv_bytes,
                     "kernel_avg_us": round(kern_avg_us, 2)},
        "cpu_baseline": cpu,
        "parity": parity,
        "host_wall_s": round(wall, 4),
        "gen_s": round(gen_s, 1),
    }

    if args.prefill:
        line["prefill_chunk"] = bench_prefill(args, dev)

    print(json.dumps(line), flush=True)


def _kernel_sha() -> str:
    """Hash of the sources the partial-decode kernel is built from; a stored
    traffic figure is reported only while it matches."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_cache_04_amd", "csrc")
    for name in ("decode.hip", "pkv_device.h", "pkv_internal.h"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def bench_prefill(args, dev):
    import numpy as np
    import torch

    import paged_kv_cache_04_amd as pkv
    from paged_kv_cache_04_amd import accounting as A
    from paged_kv_cache_04_amd import workloads as W

    w = W.make("prefill")
    kc, vc = w.k_cache.to(dev), w.v_cache.to(dev)
    q, bt, kl = w.q.to(dev), w.block_table.to(dev), w.context_lens.to(dev)
    qi = w.q_indptr.to(dev)
    pkv.kv_append(kc, vc, w.k_new.to(dev), w.v_new.to(dev), w.slots.to(dev))
    out = torch.empty_like(q)
    chunk = w.meta["chunk_lens"]

    def run():
        pkv.paged_attn_prefill_chunk(q, kc, vc, qi, bt, kl, max(chunk), w.max_context_len,
                                     w.scale, out=out)

    for _ in range(3):
        run()
    torch.cuda.synchronize()
    ts = []
    for _ in range(10):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        run()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3)
    us = float(np.mean(ts))
    flops = A.prefill_flops(w.context_lens.tolist(), chunk, w.num_q_heads, w.head_dim)
    tf = flops / (us * 1e-6) / 1e12
    return {"workload": "batch 4, 32768-token paged history + 512-row causal chunk, 32 q / 8 kv "
                        "heads, head_dim 128, bf16",
            "kernel_avg_us": round(us, 2), "query_tokens_per_s": round(sum(chunk) / (us * 1e-6), 1),
            "roofline": {"bound": "mfma", "achieved": round(tf, 1),
                         "peak": A.MFMA_PEAK_TFLOPS["bf16"], "unit": "TFLOP/s",
                         "frac": round(tf / A.MFMA_PEAK_TFLOPS["bf16"], 4),
                         "algorithmic_flops_per_launch": flops}}


if __name__ == "__main__":
    main()
