#!/usr/bin/env python3
"""Benchmark of one mixed continuous-batching step of paged attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 3]

A step is the whole hot path over one synthetic batch: host scheduling and planning into pinned memory, one
host-to-device metadata copy, the KV append, split-KV decode, prefill tiles and the merge of split rows, for every
layer of the workload. Kernels run back to back on one compute stream; the host prepares step k+1 (into the other
of two pinned/device buffer pairs, copied on a stream of its own) while the device runs step k. Per-kernel durations
come from HIP events recorded on the compute stream around the decode, prefill and merge kernels of every
EVENTS_EVERY-th timed step. --concurrent instead runs the prefill-tile kernels on a second stream
beside the decode kernel (their event intervals then overlap). Inputs (caches with the history, the step's new
Q/K/V rows) are resident in HBM before timing starts.

Prints ONE JSON line on stdout; progress goes to stderr. The headline workload is the mixed chunked-prefill step
under max_batch_tokens 2048 (96 decodes, two continuing 512-token chunks and a 928-token new prompt; 32 query /
8 kv heads, head_dim 128, bf16, page 16).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "mixed-batch paged attention: query tokens/s + KV GB/s (% HBM / % MFMA peak)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")
EVENTS_EVERY = 4               # every EVENTS_EVERY-th timed step carries the per-kernel timing events
WARMUP_SECONDS = 0.3           # minimum duration of the untimed warm-up
DEVICE_SRC = os.path.join(ROOT, "paged_kv_attention_varlen_amd", "csrc", "cb_device.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_work(w, sched):
    """What the method must move or compute, per layer (no padding, no partial results).

    decode kernel bytes: every visible key of a decode row read once per kv head (K and V), plus its Q and O rows.
    append bytes: every new token's K and V rows read once and written once into the caches.
    prefill flops: 4*D per (query row, head, visible key) -- QK^T and PV, causal count.
    kv bytes: every visible key of every request read once per kv head (K and V).
    """
    e = 2 if w.dtype == "bf16" else 4
    qsl, seq = sched["query_start_loc"], sched["seq_lens"]
    out = []
    for lay in w.layers:
        wl = lay.window_left
        dec_bytes = pre_flops = kv_bytes = 0
        n_dec = 0
        for r in range(sched["num_reqs"]):
            q = int(qsl[r + 1] - qsl[r])
            ctx = int(seq[r]) - q
            pos = np.arange(ctx, ctx + q)
            lo = np.zeros_like(pos) if wl < 0 else np.maximum(0, pos - wl)
            n_vis = pos - lo + 1
            kv_bytes += int(ctx + q - lo[0]) * w.Hkv * 2 * w.D * e
            if q == 1:
                n_dec += 1
                dec_bytes += int(n_vis[0]) * w.Hkv * 2 * w.D * e + 2 * w.Hq * w.D * e
            else:
                pre_flops += int(n_vis.sum()) * 4 * w.D * w.Hq
        append_bytes = 4 * int(sched["num_tokens"]) * w.Hkv * w.D * e
        out.append({"decode_bytes": dec_bytes, "prefill_flops": pre_flops, "kv_bytes": kv_bytes, "decodes": n_dec,
                    "append_bytes": append_bytes})
    return out


def decode_source_sha() -> str:
    """SHA-256 of the decode launch's source: the shared device helpers and the KV append at the top of the device
    source (the append's work groups run inside the decode launch) and the split-KV decode section. Edits elsewhere
    (page copies, prefill, merge) leave the decode launch, and its measured traffic, unchanged."""
    src = open(DEVICE_SRC, encoding="utf-8").read()
    helpers = src[:src.index("// ============================================================================================ page copies")]
    start = src.index("// ===================================================================== split-KV decode")
    end = src.index("// ========================================================================= general per-token kernel")
    return hashlib.sha256((helpers + src[start:end]).encode()).hexdigest()


def stored_traffic(workload: int):
    """HBM bytes per decode launch from a rocprofv3 counter run, if taken on this workload and on the current decode
    kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    try:
        rec = json.load(open(TRAFFIC_FILE))
        if rec.get("decode_source_sha256") != decode_source_sha() or rec.get("workload") != workload:
            return None
        return rec.get("traffic_bytes_per_launch")
    except Exception:  # noqa: BLE001
        return None


def measure_swap(step, n_pages: int, reps: int = 5) -> dict:
    """Offloading round trip of n_pages distinct pages of the first layer (K and V): the gather kernel into a device
    staging buffer, the copy to pinned host memory, the copy back, and the scatter kernel into other pages. HIP events
    on the stream that runs them; bytes are the pages' bytes (the kernels read and write each once)."""
    import torch
    from paged_kv_attention_varlen_amd import copy_pages
    from paged_kv_attention_varlen_amd.swap import HostSwap
    L = step.layers[0]
    n_pages = min(n_pages, L.k_cache.shape[0] // 2)
    perm = torch.randperm(L.k_cache.shape[0], device="cuda").to(torch.int32)
    src, dst = perm[:n_pages].contiguous(), perm[n_pages:2 * n_pages].contiguous()
    pool = HostSwap(L.k_cache, L.v_cache, n_pages)
    page_bytes = (L.k_cache[0].numel() + L.v_cache[0].numel()) * L.k_cache.element_size()
    total = n_pages * page_bytes
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    t = {"gather": [], "to_host": [], "to_device": [], "scatter": []}
    for _ in range(reps + 1):
        ev[0].record()
        copy_pages(pool.stage_k, L.k_cache, None, src)
        copy_pages(pool.stage_v, L.v_cache, None, src)
        ev[1].record()
        pool.host_k.copy_(pool.stage_k, non_blocking=True)
        pool.host_v.copy_(pool.stage_v, non_blocking=True)
        ev[2].record()
        pool.stage_k.copy_(pool.host_k, non_blocking=True)
        pool.stage_v.copy_(pool.host_v, non_blocking=True)
        ev[3].record()
        copy_pages(L.k_cache, pool.stage_k, dst, None)
        copy_pages(L.v_cache, pool.stage_v, dst, None)
        ev[4].record()
        torch.cuda.synchronize()
        for k, (a, b) in zip(t, ((0, 1), (1, 2), (2, 3), (3, 4))):
            t[k].append(ev[a].elapsed_time(ev[b]))
    us = {k: float(np.median(v[1:])) * 1e3 for k, v in t.items()}
    return {"pages": n_pages, "bytes": total, "page_bytes": page_bytes,
            "us": {k: round(v, 1) for k, v in us.items()},
            "gb_per_s": {"gather (HBM read + write)": round(2 * total / (us["gather"] / 1e6) / 1e9, 1),
                         "device to pinned host": round(total / (us["to_host"] / 1e6) / 1e9, 1),
                         "pinned host to device": round(total / (us["to_device"] / 1e6) / 1e9, 1),
                         "scatter (HBM read + write)": round(2 * total / (us["scatter"] / 1e6) / 1e9, 1)}}


def cpu_baseline(w, sched, seconds: float):
    """Time the oracle (as it stands) on a bounded sample of the step's query rows: all decode rows first, then
    prefill rows in random order, until `seconds` of oracle time (repeating the step if it finishes sooner). Input
    generation is not timed."""
    from oracle import attention as A
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    qsl, seq, idx = sched["query_start_loc"], sched["seq_lens"], sched["req_index"]
    nd = sched["num_decodes"]
    order = [(r, 0) for r in range(nd)]
    pre = [(r, i) for r in range(nd, sched["num_reqs"]) for i in range(int(qsl[r + 1] - qsl[r]))]
    rng = np.random.default_rng(0)
    order += [pre[j] for j in rng.permutation(len(pre))]
    layer = 0
    wl = w.layers[layer].window_left
    done, spent = 0, 0.0
    # the whole step may take less than `seconds`: then its rows are timed again, pass after pass
    passes = max(1, int(seconds // 2) + 1)
    for r, i in (x for _ in range(passes) for x in order):
        if spent >= seconds:
            break
        q_len = int(qsl[r + 1] - qsl[r])
        ctx = int(seq[r]) - q_len
        pos = ctx + i
        lo = A.visible_range(pos, wl)[0]
        k = w.values("k", int(idx[r]), layer, lo, pos + 1)
        v = w.values("v", int(idx[r]), layer, lo, pos + 1)
        qr = w.values("q", int(idx[r]), layer, pos, pos + 1)
        t0 = time.perf_counter()
        A.attend_rows(qr, k, v, lo, [pos], w.scale, wl)
        spent += time.perf_counter() - t0
        done += 1
    return {"value": done / spent if spent > 0 else None, "unit": "query tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} query rows of layer '{w.layers[layer].name}' ({done / len(order):.2f} passes over "
                      f"the step's {len(order)} rows: {nd} decode rows first, then the prefill rows in random "
                      f"order), fp64 numpy, {spent:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=3, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--decode-split", type=int, default=0)
    ap.add_argument("--prefill-split", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--concurrent", action="store_true",
                    help="run the prefill kernels on a second stream concurrently with the decode kernel")
    ap.add_argument("--no-copy-stream", action="store_true",
                    help="copy each step's metadata on the compute stream instead of a stream of its own (which lets "
                         "the copy overlap the previous step's kernels)")
    ap.add_argument("--graphs", action="store_true",
                    help="replay each step's kernels as a captured HIP graph (steps that carry timing events run "
                         "eagerly)")
    ap.add_argument("--swap-pages", type=int, default=0,
                    help="also measure offloading N cache pages of the first layer to pinned host memory and back "
                         "(gather kernel, device-to-host copy, host-to-device copy, scatter kernel)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before the steps, run a plain device copy of this many MiB three times (untimed), the "
                         "known-size reference for scaling HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported (this build has no multi-GPU "
              "path: the step would shard by kv heads or by requests with no exchange inside attention)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from paged_kv_attention_varlen_amd import load_library
    from paged_kv_attention_varlen_amd.hip_events import HipEvent
    from paged_kv_attention_varlen_amd.step import Step, StepPipeline
    from synth import make_workload

    load_library()
    if not torch.cuda.is_available():
        log("no GPU visible")
        sys.exit(1)
    copy_ref = None
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(3):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 3
        copy_ref = {"bytes_read_plus_written": 2 * n * 4, "us": round(ms * 1e3, 1),
                    "gb_per_s": round(2 * n * 4 / (ms / 1e3) / 1e9, 1)}
        del src, dst
    w = make_workload(args.workload)
    log(f"[bench] workload {args.workload}: {w.name}")
    t = time.time()
    step = Step.from_workload(w, decode_split=args.decode_split, prefill_split=args.prefill_split, threads=16)
    pipe = StepPipeline(w, step, args.decode_split, args.prefill_split, concurrent=args.concurrent,
                        copy_stream=not args.no_copy_stream, graphs=args.graphs)
    sched = step.sched
    log(f"[bench] setup {time.time() - t:.1f}s; N={sched['num_reqs']} T={sched['num_tokens']} "
        f"decodes={sched['num_decodes']}; plans {[L.plan.counts() for L in step.layers]}")

    # untimed warm-up: at least W steps, and at least WARMUP_SECONDS of them so that the clocks have ramped up
    warm, t_warm = 0, time.perf_counter()
    while warm < args.warmup or time.perf_counter() - t_warm < WARMUP_SECONDS:
        pipe.run()
        warm += 1
        if warm % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    log(f"[bench] {warm} warm-up steps")
    L = len(w.layers)
    # Every EVENTS_EVERY-th timed step brackets its decode, prefill and merge kernels with events (6 per layer); the
    # kernel averages come from that sample of the timed steps. Each event is a packet in the stream and costs the
    # step a little time, so the other steps run without them. The timing events are recorded without the
    # system-scope fence (hipEventDisableSystemFence): they order nothing, and the cache write-back and invalidation
    # of that fence would otherwise be charged to the kernel that follows the event.
    timed = list(range(0, args.steps, EVENTS_EVERY))
    events = {k: [[HipEvent(timing=True, system_fence=False) for _ in range(6)] for _ in range(L)] for k in timed}
    cur = torch.cuda.current_stream()
    for per_step in events.values():
        for per_layer in per_step:
            for ev in per_layer:
                ev.record(cur)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        pipe.run(events.get(k))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    log(f"[bench] {args.steps} steps: {ms_per_step:.4f} ms/step")

    # per-kernel durations from the events (same stream as the launches)
    dec_ms = [[events[k][l][0].elapsed_time(events[k][l][1]) for k in timed] for l in range(L)]
    pre_ms = [[events[k][l][2].elapsed_time(events[k][l][3]) for k in timed] for l in range(L)]
    com_ms = [[events[k][l][4].elapsed_time(events[k][l][5]) for k in timed] for l in range(L)]
    work = algorithmic_work(w, sched)
    T = sched["num_tokens"]
    value = T / (ms_per_step / 1e3)
    kv_bytes = sum(x["kv_bytes"] for x in work)

    dec_t = sum(float(np.mean(dec_ms[l])) for l in range(L) if work[l]["decodes"])
    dec_b = sum(x["decode_bytes"] for x in work)
    # with the fused append, the decode launch also moves the step's new K/V rows into the caches
    fused = pipe.fused and all(x["decodes"] for x in work)
    app_b = sum(x["append_bytes"] for x in work) if fused else 0
    roofline = None
    if dec_t > 0:
        achieved = (dec_b + app_b) / (dec_t / 1e3) / 1e9
        label = "decode_kernel (split-KV decode, with the fused KV append)" if fused else \
            "decode_kernel (split-KV decode)"
        roofline = {"bound": "hbm", "kernel": label, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": stored_traffic(args.workload), "algorithmic_bytes_per_step": dec_b + app_b,
                    "of_which_append_bytes": app_b,
                    "launches_per_step": sum(1 for x in work if x["decodes"]),
                    "avg_launch_us": round(dec_t * 1e3 / max(1, sum(1 for x in work if x["decodes"])), 2),
                    "timed_steps_sampled": len(timed)}
    pre_t = sum(float(np.mean(pre_ms[l])) for l in range(L))
    pre_f = sum(x["prefill_flops"] for x in work)
    roofline_prefill = None
    if pre_f > 0 and pre_t > 0:
        tf = pre_f / (pre_t / 1e3) / 1e12
        # fp32 steps and shapes the MFMA tiles do not take run on the per-token VALU kernel instead
        fast = all(L_.plan.counts()["prefill"] > 0 and L_.plan.counts()["rowwise"] == 0 for L_ in step.layers)
        roofline_prefill = {"bound": "mfma", "kernel": "prefill_kernel (bf16 MFMA tiles)" if fast else
                            "prefill_kernel and rowwise_kernel (per-token VALU)", "achieved": round(tf, 1),
                            "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                            "algorithmic_flops_per_step": pre_f, "avg_launch_us": round(pre_t * 1e3 / L, 2),
                            "timed_steps_sampled": len(timed)}

    base = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample")
        base = cpu_baseline(w, sched, args.cpu_seconds)

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "query tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": warm, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic (seeded N(0,1) Q/K/V, shuffled page pools)",
        "config": {"workload": w.name, "requests": sched["num_reqs"], "query_tokens": T,
                   "decodes": sched["num_decodes"], "layers": [x.name for x in w.layers],
                   "kv_tokens_visible": int(kv_bytes // (w.Hkv * 2 * w.D * (2 if w.dtype == "bf16" else 4)))},
        "kv_gb_per_s": round(kv_bytes / (ms_per_step / 1e3) / 1e9, 1),
        "kernel_us": {"decode": round(dec_t * 1e3, 2), "prefill_and_rowwise": round(pre_t * 1e3, 2),
                      "combine": round(sum(float(np.mean(com_ms[l])) for l in range(L)) * 1e3, 2)},
        "roofline": roofline, "roofline_prefill": roofline_prefill, "cpu_baseline": base,
    }
    if copy_ref:
        line["device_copy_reference"] = copy_ref
    if args.swap_pages:
        line["kv_swap"] = measure_swap(step, args.swap_pages)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
