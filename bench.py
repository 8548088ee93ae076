#!/usr/bin/env python3
"""Benchmark of one mixed continuous-batching step of paged attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 5] [--configs 2,3,4]

A step is the whole hot path over one synthetic batch: host scheduling and planning into pinned memory, one
host-to-device metadata copy, the KV append, split-KV decode, prefill tiles and the merge of split rows, for every
layer of the workload. Kernels run back to back on one compute stream; the host prepares step k+1 (into the other
of two pinned/device buffer pairs, copied on a stream of its own) while the device runs step k. Inputs (caches with
the history, the step's new Q/K/V rows) are resident in HBM before timing starts.

The headline is the largest single-GPU workload: the hybrid full + sliding-window layer pair over one 8192-token
mixed step (128 decodes with context up to 32768, three 2048-token continuing chunks and a 1920-token new prompt;
32 query / 8 kv heads, head_dim 128, bf16, page 32, window 4096). Exactly W untimed warm-up steps, then K timed
steps between two device synchronisations: `value` is query tokens per second over those K steps (wall clock).
Per-kernel durations come from fence-free HIP events that the decode, prefill and merge launches of every
EVENTS_EVERY-th timed step record themselves as their kernels start and end (cb_attn_args.timing_start /
timing_stop), so that they time the kernels as a kernel trace does. A second pass of steps, each bracketed by step-boundary events,
gives the p10/p50/p90 step times; a third runs steps after a 1 GiB write (larger than the 256 MB last-level cache)
and reports the kernels' rooflines without a warm cache; a fourth times the same step with the prefill kernels on a
second stream beside the decode kernel (only its step time: the kernels then share the GPU). The mixed 2048-token
step, the decode-only step and the large decode batch are measured the same way and reported under `per_config`.

Prints ONE JSON line on stdout; progress goes to stderr.
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
FLUSH_BYTES = 1 << 30          # the write between flushed steps
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
    """HBM bytes per step of the decode launches (all layers) from rocprofv3 counter runs, if taken on this workload
    and on the current decode kernel source; None otherwise."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    try:
        recs = json.load(open(TRAFFIC_FILE)).get("records", [])
        sha = decode_source_sha()
        for rec in recs:
            if rec.get("workload") == workload and rec.get("decode_source_sha256") == sha:
                return rec.get("traffic_bytes_per_step")
    except Exception:  # noqa: BLE001
        return None
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
    """Time the oracle (as it stands) on a bounded sample of the step's query rows, every layer of the workload:
    the first decode rows one by one, then runs of up to 64 consecutive rows of the prefill chunks (random chunk,
    random start), each run in one call of the oracle's row attention per layer, as the oracle computes a request's
    rows. Stops after `seconds` of oracle time (or three times that of wall time, input generation included). Input
    generation is not timed. A token counts once all layers' rows of it are done."""
    from oracle import attention as A
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas = None
    qsl, seq, idx = sched["query_start_loc"], sched["seq_lens"], sched["req_index"]
    nd = sched["num_decodes"]
    rng = np.random.default_rng(0)
    units = [(r, 0, 1) for r in range(min(nd, 8))]
    chunks = list(range(nd, sched["num_reqs"]))
    for _ in range(512):
        if not chunks:
            break
        r = int(rng.choice(chunks))
        q = int(qsl[r + 1] - qsl[r])
        a = int(rng.integers(0, max(1, q - 63)))
        units.append((r, a, min(q, a + 64)))
    rows, spent, t_wall = 0, 0.0, time.perf_counter()
    n_dec = n_pre = 0
    for r, a, b in units:
        if spent >= seconds or time.perf_counter() - t_wall > 3 * seconds:
            break
        q_len = int(qsl[r + 1] - qsl[r])
        ctx = int(seq[r]) - q_len
        positions = list(range(ctx + a, ctx + b))
        for l, lay in enumerate(w.layers):
            lo = A.visible_range(positions[0], lay.window_left)[0]
            k = w.values("k", int(idx[r]), l, lo, positions[-1] + 1)
            v = w.values("v", int(idx[r]), l, lo, positions[-1] + 1)
            qr = w.values("q", int(idx[r]), l, positions[0], positions[-1] + 1)
            t0 = time.perf_counter()
            A.attend_rows(qr, k, v, lo, positions, w.scale, lay.window_left)
            spent += time.perf_counter() - t0
        rows += b - a
        if r < nd:
            n_dec += 1
        else:
            n_pre += b - a
    return {"value": rows / spent if spent > 0 else None, "unit": "query tokens/s",
            "cores": len(os.sched_getaffinity(0)), "blas_threads": blas, "kind": "oracle",
            "sample": f"{rows} query tokens of the headline step ({n_dec} decode rows, then {n_pre} prefill rows in "
                      f"runs of up to 64 consecutive rows of one chunk), every layer "
                      f"({', '.join(x.name for x in w.layers)}); fp64 numpy oracle, {spent:.1f} s of oracle time"}


def _pct(xs):
    a = np.asarray(xs, dtype=np.float64)
    return {"p10": round(float(np.percentile(a, 10)), 2), "p50": round(float(np.percentile(a, 50)), 2),
            "p90": round(float(np.percentile(a, 90)), 2), "n": int(a.size)}


def _rooflines(w, step, work, fused, dec_us, pre_us, n_sampled):
    """Decode roofline (HBM) and prefill roofline (MFMA) from per-layer mean kernel durations in microseconds."""
    L = len(w.layers)
    dec_t = sum(dec_us[l] for l in range(L) if work[l]["decodes"])
    dec_b = sum(x["decode_bytes"] for x in work)
    app_b = sum(x["append_bytes"] for x in work) if fused else 0
    n_dec_launch = sum(1 for x in work if x["decodes"])
    roofline = None
    if dec_t > 0:
        achieved = (dec_b + app_b) / (dec_t / 1e6) / 1e9
        roofline = {"bound": "hbm", "kernel": "decode_kernel (split-KV decode" +
                    (", with the fused KV append)" if fused else ")"),
                    "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                    "algorithmic_bytes_per_step": dec_b + app_b, "of_which_append_bytes": app_b,
                    "launches_per_step": n_dec_launch, "avg_launch_us": round(dec_t / max(1, n_dec_launch), 2),
                    "per_layer_us": [round(dec_us[l], 2) for l in range(L)], "timed_steps_sampled": n_sampled}
    pre_t = sum(pre_us[l] for l in range(L))
    pre_f = sum(x["prefill_flops"] for x in work)
    roofline_prefill = None
    if pre_f > 0 and pre_t > 0:
        tf = pre_f / (pre_t / 1e6) / 1e12
        fast = all(L_.plan.counts()["prefill"] > 0 and L_.plan.counts()["rowwise"] == 0 for L_ in step.layers)
        roofline_prefill = {"bound": "mfma", "kernel": "prefill_kernel (bf16 MFMA tiles)" if fast else
                            "prefill_kernel and rowwise_kernel (per-token VALU)", "achieved": round(tf, 1),
                            "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                            "algorithmic_flops_per_step": pre_f, "avg_launch_us": round(pre_t / L, 2),
                            "per_layer_us": [round(pre_us[l], 2) for l in range(L)],
                            "timed_steps_sampled": n_sampled}
    return roofline, roofline_prefill


def measure(index: int, steps: int, warmup: int, args, dist_steps: int, flush_steps: int = 0,
            concurrent_steps: int = 0):
    """Set up a workload and time it (see the module docstring). Returns (result dict, workload, step, schedule)."""
    import torch
    from harness import build_step, pipeline_for
    from paged_kv_attention_varlen_amd.hip_events import HipEvent
    from synth import make_workload

    w = make_workload(index)
    log(f"[bench] workload {index}: {w.name}")
    t = time.time()
    step = build_step(w, decode_split=args.decode_split, prefill_split=args.prefill_split, threads=16,
                      prefill_rows=args.prefill_rows)
    pipe = pipeline_for(w, step, decode_split=args.decode_split, prefill_split=args.prefill_split,
                        prefill_rows=args.prefill_rows,
                        concurrent=args.concurrent, copy_stream=not args.no_copy_stream, graphs=args.graphs)
    sched = step.sched
    log(f"[bench] setup {time.time() - t:.1f}s; N={sched['num_reqs']} T={sched['num_tokens']} "
        f"decodes={sched['num_decodes']}; plans {[L.plan.counts() for L in step.layers]}")
    for _ in range(warmup):
        pipe.run()
    torch.cuda.synchronize()
    L = len(w.layers)
    main = pipe.main
    # Every EVENTS_EVERY-th timed step brackets its decode, prefill and merge kernels with events (6 per layer), which
    # the kernels record as they start and end; the kernel averages come from that sample of the timed steps. The
    # events are created without the system-scope fence (hipEventDisableSystemFence): they order nothing.
    timed = list(range(0, steps, EVENTS_EVERY))
    events = {k: [[HipEvent(timing=True, system_fence=False) for _ in range(6)] for _ in range(L)] for k in timed}
    for per_step in events.values():
        for per_layer in per_step:
            for ev in per_layer:
                ev.record(main)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        pipe.run(events.get(k))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / steps
    log(f"[bench] workload {index}: {steps} steps {ms_per_step:.4f} ms/step")

    def mean_us(a, b, ran):
        # a call that launched nothing recorded its two events back to back on the stream: reported as 0
        return [float(np.mean([events[k][l][a].elapsed_time(events[k][l][b]) for k in timed])) * 1e3
                if ran(step.layers[l].plan.counts()) else 0.0 for l in range(L)]

    dec_us = mean_us(0, 1, lambda c: c["decode"] > 0)
    pre_us = mean_us(2, 3, lambda c: c["prefill"] + c["rowwise"] > 0 or (pipe.fused and c["decode"] == 0))
    com_us = mean_us(4, 5, lambda c: c["combine"] > 0)
    work = algorithmic_work(w, sched)
    fused = pipe.fused and all(x["decodes"] for x in work)
    roofline, roofline_prefill = _rooflines(w, step, work, fused, dec_us, pre_us, len(timed))
    if roofline is not None:
        roofline["traffic"] = stored_traffic(index)

    # step-time distribution: boundary events only, one per step
    bounds = [HipEvent(timing=True, system_fence=False) for _ in range(dist_steps + 1)]
    for k in range(dist_steps):
        bounds[k].record(main)
        pipe.run()
    bounds[-1].record(main)
    torch.cuda.synchronize()
    step_us = [bounds[k].elapsed_time(bounds[k + 1]) * 1e3 for k in range(dist_steps)]

    T = sched["num_tokens"]
    kv_bytes = sum(x["kv_bytes"] for x in work)
    res = {"workload": w.name, "index": index, "value": round(T / (ms_per_step / 1e3), 1),
           "unit": "query tokens/s", "steps": steps, "warmup": warmup, "ms_per_step": round(ms_per_step, 5),
           "step_us": _pct(step_us), "kv_gb_per_s": round(kv_bytes / (ms_per_step / 1e3) / 1e9, 1),
           "requests": sched["num_reqs"], "query_tokens": T, "decodes": sched["num_decodes"],
           "layers": [x.name for x in w.layers],
           "kv_tokens_visible": int(kv_bytes // (w.Hkv * 2 * w.D * (2 if w.dtype == "bf16" else 4))),
           "kernel_us": {"decode": round(sum(dec_us), 2), "prefill_and_rowwise": round(sum(pre_us), 2),
                         "combine": round(sum(com_us), 2)},
           "roofline": roofline, "roofline_prefill": roofline_prefill}

    if flush_steps:
        # each step after a 1 GiB write, steps synchronised one by one: the kernels start with a cold cache
        scrub = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
        fev = [[HipEvent(timing=True, system_fence=False) for _ in range(6)] for _ in range(L)]
        fd, fp = [], []
        for k in range(flush_steps):
            scrub.fill_(float(k))
            torch.cuda.synchronize()
            pipe.run(fev)
            torch.cuda.synchronize()
            fd.append([fev[l][0].elapsed_time(fev[l][1]) * 1e3 for l in range(L)])
            fp.append([fev[l][2].elapsed_time(fev[l][3]) * 1e3 for l in range(L)])
        del scrub
        fr, frp = _rooflines(w, step, work, fused, list(np.median(np.asarray(fd), axis=0)),
                             list(np.median(np.asarray(fp), axis=0)), flush_steps)
        res["flushed"] = {"steps": flush_steps, "write_bytes_before_each_step": FLUSH_BYTES,
                          "decode_frac": fr["frac"] if fr else None,
                          "decode_us": fr["avg_launch_us"] if fr else None,
                          "prefill_frac": frp["frac"] if frp else None,
                          "prefill_us": frp["avg_launch_us"] if frp else None}
    if args.graphs:
        res["graphs"] = {"captured": pipe.captures, "replayed": pipe.replays}
    if concurrent_steps and not args.concurrent:
        # the same step with the prefill-tile kernels on a second stream beside the decode kernel (the append then
        # runs as a launch of its own first, since the concurrent prefill kernels read the appended keys): the two
        # kernels share the GPU, so only the step time is reported
        cp = pipeline_for(w, step, decode_split=args.decode_split, prefill_split=args.prefill_split,
                          prefill_rows=args.prefill_rows,
                          concurrent=True, copy_stream=not args.no_copy_stream)
        for _ in range(warmup):
            cp.run()
        torch.cuda.synchronize()
        c0 = time.perf_counter()
        for _ in range(concurrent_steps):
            cp.run()
        torch.cuda.synchronize()
        cms = (time.perf_counter() - c0) * 1e3 / concurrent_steps
        res["concurrent_prefill_stream"] = {"steps": concurrent_steps, "warmup": warmup,
                                            "ms_per_step": round(cms, 5), "value": round(T / (cms / 1e3), 1),
                                            "unit": "query tokens/s"}
        log(f"[bench] workload {index}: concurrent prefill stream {cms:.4f} ms/step")
        del cp
    return res, w, step, pipe


def measure_loop(index: int, steps: int, warmup: int) -> dict:
    """A serving loop over the workload's requests: every step is scheduled from the request state the previous step
    left (each decode's context grows by one key, requests take fresh pages as they cross page boundaries, chunks
    advance), so consecutive steps differ in seq_lens, block tables and plans. The same loop, from the same start
    state, runs twice: with eager launches, and replaying HIP graphs captured per padded shape. Wall clock per step,
    the host's scheduling, planning, padding and request bookkeeping (the lifecycle in native code, in place)
    included, as in a serving loop; the new rows' values are not rewritten between steps (timing only: the
    serving-loop parity tests check the outputs)."""
    import torch
    from harness import build_step, pipeline_for
    from synth import make_workload

    w = make_workload(index)
    step = build_step(w, threads=16)
    res = {"workload": w.name, "index": index, "steps": steps, "warmup": warmup}
    for mode in ("eager", "graph replay by padded shape"):
        pipe = pipeline_for(w, step, graphs=mode != "eager")
        toks = 0
        for k in range(warmup + steps):
            if k == warmup:
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                captures0 = pipe.captures
            views = pipe.prepare()
            pipe.launch(views)
            if k >= warmup:
                toks += pipe.num_tokens
            pipe.advance()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        r = {"ms_per_step": round(ms, 5), "value": round(toks / (ms * steps / 1e3), 1), "unit": "query tokens/s"}
        if mode != "eager":
            r.update({"captures_in_timed_steps": pipe.captures - captures0, "captures": pipe.captures,
                      "replays": pipe.replays, "graphs_kept": len(pipe.graphs)})
        res[mode] = r
        log(f"[bench] serving loop, workload {index}, {mode}: {ms:.4f} ms/step")
        del pipe
        torch.cuda.synchronize()
    del step
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=5, choices=[1, 2, 3, 4, 5],
                    help="headline workload (default 5, the hybrid layer pair over one 8192-token step)")
    ap.add_argument("--configs", default="2,3,4",
                    help="comma-separated workloads also measured and reported under per_config ('' for none)")
    ap.add_argument("--config-steps", type=int, default=50, help="timed steps of each per_config workload")
    ap.add_argument("--config-warmup", type=int, default=10, help="warm-up steps of each per_config workload")
    ap.add_argument("--dist-steps", type=int, default=40, help="steps of the step-time distribution pass")
    ap.add_argument("--flush-steps", type=int, default=10,
                    help="steps of the headline run after a 1 GiB write each (0: skip)")
    ap.add_argument("--concurrent-steps", type=int, default=20,
                    help="steps of an extra headline pass with the prefill kernels on a second stream beside the "
                         "decode kernel (0: skip); only its step time is reported")
    ap.add_argument("--decode-split", type=int, default=0)
    ap.add_argument("--prefill-split", type=int, default=0)
    ap.add_argument("--prefill-rows", type=int, default=0, choices=(0, 128, 256),
                    help="query rows per prefill work group (0: the planner's choice)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--concurrent", action="store_true",
                    help="run the prefill kernels on a second stream concurrently with the decode kernel")
    ap.add_argument("--no-copy-stream", action="store_true",
                    help="copy each step's metadata on the compute stream instead of a stream of its own (which lets "
                         "the copy overlap the previous step's kernels)")
    ap.add_argument("--graphs", action="store_true",
                    help="replay each step's kernels as a HIP graph captured for its padded shape (steps that carry "
                         "timing events run the same padded launches eagerly)")
    ap.add_argument("--swap-pages", type=int, default=0,
                    help="also measure offloading N cache pages of the first layer to pinned host memory and back "
                         "(gather kernel, device-to-host copy, host-to-device copy, scatter kernel)")
    ap.add_argument("--loop-workload", type=int, default=2, choices=[2, 3, 4, 5],
                    help="workload of the serving-loop pass (eager launches against graph replay by padded shape)")
    ap.add_argument("--loop-steps", type=int, default=64, help="timed steps of the serving-loop pass (0: no pass)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before the steps, run a plain device copy of this many MiB three times (untimed), the "
                         "known-size reference for scaling HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported (the library has no multi-GPU "
              "path: the step would shard by kv heads or by requests with no exchange inside attention)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from paged_kv_attention_varlen_amd import load_library

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

    head, w, step, pipe = measure(args.workload, args.steps, args.warmup, args, args.dist_steps, args.flush_steps,
                                  args.concurrent_steps)
    sched = step.sched
    swap = measure_swap(step, args.swap_pages) if args.swap_pages else None
    del pipe, step
    torch.cuda.empty_cache()

    per_config = {}
    for c in [int(x) for x in args.configs.split(",") if x.strip()]:
        if c == args.workload:
            continue
        r, _, st, pp = measure(c, args.config_steps, args.config_warmup, args, args.dist_steps)
        per_config[str(c)] = r
        del st, pp
        torch.cuda.empty_cache()

    loop = None
    if args.loop_steps:
        try:
            loop = measure_loop(args.loop_workload, args.loop_steps, 16)
        except Exception as e:  # noqa: BLE001 - an extra pass must not cost the benchmark its line
            log(f"[bench] serving loop failed: {e!r}")
            loop = {"error": repr(e)}
            torch.cuda.synchronize()
            torch.cuda.empty_cache()

    base = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample")
        base = cpu_baseline(w, sched, args.cpu_seconds)

    line = {
        "metric": METRIC, "value": head["value"], "unit": "query tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic (seeded N(0,1) Q/K/V, shuffled page pools)",
        "config": {"workload": w.name, "index": args.workload, "requests": head["requests"],
                   "query_tokens": head["query_tokens"], "decodes": head["decodes"], "layers": head["layers"],
                   "kv_tokens_visible": head["kv_tokens_visible"]},
        "step_us": head["step_us"], "kv_gb_per_s": head["kv_gb_per_s"], "kernel_us": head["kernel_us"],
        "roofline": head["roofline"], "roofline_prefill": head["roofline_prefill"],
        "flushed": head.get("flushed"), "concurrent_prefill_stream": head.get("concurrent_prefill_stream"),
        "per_config": per_config, "serving_loop": loop, "cpu_baseline": base,
    }
    if "graphs" in head:
        line["graphs"] = head["graphs"]
    if copy_ref:
        line["device_copy_reference"] = copy_ref
    if swap:
        line["kv_swap"] = swap
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
