"""Build the device state of a synthetic workload's step and hand it to the package's pipeline.

History convention (setup, not part of the method): every cache page starts NaN; full layers then get positions
0 .. context-1 of every admitted request, sliding layers only the positions this step's queries can still see,
max(0, context - window_left) .. context-1, so older ring slots stay NaN. Positions are written through
cb_kv_append at the slots cb_slot_mapping gives for the request's pages.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np

import paged_kv_attention_varlen_amd as cb
from paged_kv_attention_varlen_amd.step import LayerState, Step, StepPipeline


def _torch():
    import torch
    return torch


def sched_pools(w):
    """The workload's layer pools as cb_build_metadata takes them, and the padding page id."""
    pools = [{"ring_len": lay.ring_len, "window_left": lay.window_left,
              "pool_pages": lay.num_pages - len(lay.padding_pages), "free_pages": lay.free_pages}
             for lay in w.layers]
    pad = w.layers[0].padding_pages[0] if w.layers[0].padding_pages else 0
    return pools, pad


def scheduler_for(w) -> cb.Scheduler:
    pools, pad = sched_pools(w)
    return cb.Scheduler(w.requests, pools, w.max_batch_tokens, w.max_requests, w.page_size, w.safety_margin, pad,
                        policy=w.policy)


def new_rows(w, sched, l: int, pool=None):
    """The step's new Q/K/V rows of layer l (float32 numpy, dtype-exact): q [T, Hq, D], k/v [T, Hkv, D]."""
    qsl, seq, idx = sched["query_start_loc"], sched["seq_lens"], sched["req_index"]
    N, T = sched["num_reqs"], sched["num_tokens"]
    q = np.empty((T, w.Hq, w.D), np.float32)
    k = np.empty((T, w.Hkv, w.D), np.float32)
    v = np.empty((T, w.Hkv, w.D), np.float32)

    def one(r):
        qs, qe = int(qsl[r]), int(qsl[r + 1])
        ctx = int(seq[r]) - (qe - qs)
        i = int(idx[r])
        return qs, qe, [w.values(n, i, l, ctx, ctx + qe - qs) for n in ("q", "k", "v")]

    for qs, qe, (a, b, c) in (pool.map(one, range(N)) if pool else map(one, range(N))):
        q[qs:qe], k[qs:qe], v[qs:qe] = a, b, c
    return q, k, v


def upload_new_rows(w, sched, step: Step, pool=None) -> None:
    """Write the step's new Q/K/V rows into `step`'s tensors (rows beyond the step's tokens become NaN), on the
    current stream."""
    torch = _torch()
    T = sched["num_tokens"]
    for l, L in enumerate(step.layers):
        q, k, v = new_rows(w, sched, l, pool)
        for dst, src in ((L.q, q), (L.k_new, k), (L.v_new, v)):
            dst[:T].copy_(torch.from_numpy(src).to(dst.dtype), non_blocking=False)
            dst[T:].fill_(float("nan"))


def fill_history(w, l: int, kc, vc, pool, device, dt, chunk_tokens: int = 1 << 18) -> None:
    """Write every admitted request's history into layer l's caches through cb_kv_append."""
    torch = _torch()
    lay = w.layers[l]
    P = w.page_size
    jobs = []
    for i, rq in enumerate(w.requests):
        if rq.num_computed == 0 or len(rq.pages[l]) == 0:
            continue
        lo = 0 if lay.window_left < 0 else max(0, rq.num_computed - lay.window_left)
        jobs.append((i, lo, rq.num_computed))

    def gen(job):
        i, lo, hi = job
        k = w.values("k", i, l, lo, hi)
        v = w.values("v", i, l, lo, hi)
        s = cb.slot_mapping(w.requests[i].pages[l], lay.ring_len, P, lo, hi)
        return torch.from_numpy(k).to(dt), torch.from_numpy(v).to(dt), torch.from_numpy(s)

    batch, n = [], 0

    def flush():
        nonlocal batch, n
        if not batch:
            return
        k = torch.cat([b[0] for b in batch]).to(device)
        v = torch.cat([b[1] for b in batch]).to(device)
        s = torch.cat([b[2] for b in batch]).to(device)
        cb.kv_append(kc, vc, k, v, s)
        batch, n = [], 0

    group = 16   # requests generated ahead of the copies, bounding host memory
    for g0 in range(0, len(jobs), group):
        for res in pool.map(gen, jobs[g0:g0 + group]):
            batch.append(res)
            n += res[0].shape[0]
            if n >= chunk_tokens:
                flush()
    flush()


def build_step(w, device: str = "cuda", decode_split: int = 0, prefill_split: int = 0, threads: int = 8,
               verbose: bool = False, rows: int = 0, workspace_bytes: int = 0, prefill_rows: int = 0) -> Step:
    """Schedule the workload's step (cb_build_metadata), plan every layer (cb_plan_attention), copy the metadata and
    plans to the device in one packed int32 buffer, and build the caches (NaN, then the history) and the step's
    new rows. rows: token capacity of the Q/K/V/output tensors (at least the step's tokens; extra rows are NaN);
    workspace_bytes: at least the plans' workspace."""
    torch = _torch()
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    P, Hq, Hkv, D = w.page_size, w.Hq, w.Hkv, w.D
    pools, pad = sched_pools(w)
    sched = cb.build_metadata(w.requests, pools, w.max_batch_tokens, w.max_requests, P, w.safety_margin, pad,
                              policy=w.policy)
    if sched["status"] != 0:
        raise RuntimeError(f"cb_build_metadata returned status {sched['status']}")
    N, T = sched["num_reqs"], sched["num_tokens"]
    qsl, seq = sched["query_start_loc"], sched["seq_lens"]
    rows = max(rows, T)

    # one packed int32 host buffer -> one H2D copy: per layer block table, slot mapping, plan
    plans, parts = [], []
    for l, lay in enumerate(w.layers):
        L = sched["layers"][l]
        ring = L["ring_len"] if lay.ring_len > 0 else None
        plan = cb.plan_attention(qsl, seq, ring, Hq, Hkv, D, P, dt, lay.window_left, decode_split, prefill_split,
                                 prefill_rows)
        plans.append(plan)
        parts += [L["block_table"].reshape(-1), L["slot_mapping"], plan.buffer]
    offs = np.cumsum([0] + [p.size for p in parts])
    packed = torch.from_numpy(np.concatenate(parts).astype(np.int32)).to(device)

    def view(k, shape=None):
        t = packed[offs[k]:offs[k + 1]]
        return t.view(*shape) if shape is not None else t

    layers = []
    pool = ThreadPoolExecutor(max(1, threads))
    for l, lay in enumerate(w.layers):
        L = sched["layers"][l]
        kc = torch.full((lay.num_pages, Hkv, P, D), float("nan"), dtype=dt, device=device)
        vc = torch.full((lay.num_pages, Hkv, D, P), float("nan"), dtype=dt, device=device)
        fill_history(w, l, kc, vc, pool, device, dt)
        q, k, v = new_rows(w, sched, l, pool)
        tens = []
        for src, H in ((q, Hq), (k, Hkv), (v, Hkv)):
            t = torch.full((rows, H, D), float("nan"), dtype=dt, device=device)
            t[:T] = torch.from_numpy(src).to(dt).to(device)
            tens.append(t)
        plan = plans[l]
        ws_bytes = max(cb.workspace_size(plan), int(workspace_bytes))
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=device) if ws_bytes else None
        out = torch.full((rows, Hq, D), float("nan"), dtype=dt, device=device)
        layers.append(LayerState(lay.name, lay.window_left, lay.ring_len > 0, kc, vc, plan,
                                 view(3 * l + 2), view(3 * l, (N, L["width"])), view(3 * l + 1),
                                 tens[0], tens[1], tens[2], out, ws))
        if verbose:
            print(f"[step] layer {lay.name}: plan {plan.counts()}", flush=True)
    pool.shutdown()
    torch.cuda.synchronize()
    return Step(sched, layers, w.scale, dt, Hq, Hkv, D, P)


def pipeline_for(w, step: Step, **kw) -> StepPipeline:
    """The package's step pipeline over the workload's requests and pools (keyword arguments go to StepPipeline)."""
    return StepPipeline(step, scheduler_for(w), **kw)
