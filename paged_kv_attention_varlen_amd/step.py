"""Device driver for one mixed step: metadata -> plans -> one host-to-device copy -> KV append -> attention.

`Step` strings the library's calls together for one or two layer types (a full layer, optionally a sliding layer)
that share the step's schedule. `Step.from_workload` builds the device state of a seeded synthetic workload: the
KV caches (every page first filled with NaN, so pages that must never be read poison any output that reads them),
the history of every admitted request written through cb_kv_append, and the step's new Q/K/V rows.

History convention (setup, not part of the method): full layers get positions 0 .. context-1; sliding layers get
only the positions this step's queries can still see, max(0, context - window_left) .. context-1, so older ring
slots stay NaN.
"""
from __future__ import annotations

import ctypes as C
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import List, Optional

import numpy as np

from .hip_events import HipEvent
from . import (CB_PHASE_COMBINE, CB_PHASE_DECODE, CB_PHASE_PREFILL, CB_PHASE_ROWWISE, AttnPlan, CbError, _abi,
               build_metadata, kv_append, paged_attention, plan_attention, workspace_size)


def _torch():
    import torch
    return torch


@dataclass
class LayerState:
    name: str
    window_left: int
    ring: bool
    k_cache: object            # torch [pages, Hkv, P, D]
    v_cache: object            # torch [pages, Hkv, D, P]
    plan: AttnPlan
    plan_dev: object           # torch int32 view into the packed device buffer
    block_table: object        # torch int32 [N, width]
    slot_mapping: object       # torch int32 [T]
    q: object                  # torch [T, Hq, D]
    k_new: object              # torch [T, Hkv, D]
    v_new: object
    out: object                # torch [T, Hq, D]
    workspace: Optional[object]


class Step:
    """One scheduled step on the device. Call `run()` (append + attention for every layer)."""

    def __init__(self, sched: dict, layers: List[LayerState], scale: float, dtype, Hq: int, Hkv: int, D: int, P: int):
        self.sched = sched
        self.layers = layers
        self.scale = scale
        self.dtype = dtype
        self.Hq, self.Hkv, self.D, self.P = Hq, Hkv, D, P

    # ---------------------------------------------------------------------------------------------- execution
    def append(self, l: int) -> None:
        L = self.layers[l]
        kv_append(L.k_cache, L.v_cache, L.k_new, L.v_new, L.slot_mapping)

    def attend(self, l: int, phases: int = 0, fused_append: bool = False) -> None:
        """Attention of layer l; fused_append=True also appends the step's new K/V in the same launches."""
        L = self.layers[l]
        extra = dict(k_new=L.k_new, v_new=L.v_new, slot_mapping=L.slot_mapping) if fused_append else {}
        paged_attention(L.out, L.q, L.k_cache, L.v_cache, L.block_table, L.plan, L.plan_dev, self.scale,
                        L.workspace, phases=phases, **extra)

    def run(self, fused_append: bool = False) -> None:
        for l in range(len(self.layers)):
            if fused_append:
                self.attend(l, fused_append=True)
            else:
                self.append(l)
                self.attend(l)

    PHASE_DECODE = CB_PHASE_DECODE
    PHASE_REST = CB_PHASE_ROWWISE | CB_PHASE_PREFILL | CB_PHASE_COMBINE

    # ------------------------------------------------------------------------------------------- construction
    @classmethod
    def from_workload(cls, w, device: str = "cuda", decode_split: int = 0, prefill_split: int = 0,
                      threads: int = 8, verbose: bool = False) -> "Step":
        torch = _torch()
        dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        P, Hq, Hkv, D = w.page_size, w.Hq, w.Hkv, w.D
        pools = [{"ring_len": lay.ring_len, "window_left": lay.window_left,
                  "pool_pages": lay.num_pages - len(lay.padding_pages), "free_pages": lay.free_pages}
                 for lay in w.layers]
        pad = w.layers[0].padding_pages[0] if w.layers[0].padding_pages else 0
        sched = build_metadata(w.requests, pools, w.max_batch_tokens, w.max_requests, P, w.safety_margin, pad,
                               policy=w.policy)
        if sched["status"] != 0:
            raise RuntimeError(f"cb_build_metadata returned status {sched['status']}")
        N, T = sched["num_reqs"], sched["num_tokens"]
        qsl, seq, idx = sched["query_start_loc"], sched["seq_lens"], sched["req_index"]

        # one packed int32 host buffer -> one H2D copy: per layer block table, slot mapping, plan
        plans, parts = [], []
        for l, lay in enumerate(w.layers):
            L = sched["layers"][l]
            ring = L["ring_len"] if lay.ring_len > 0 else None
            plan = plan_attention(qsl, seq, ring, Hq, Hkv, D, P, dt, lay.window_left, decode_split, prefill_split)
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
            _fill_history(w, l, kc, vc, pool, device, dt)
            q = torch.empty((T, Hq, D), dtype=dt)
            kn = torch.empty((T, Hkv, D), dtype=dt)
            vn = torch.empty((T, Hkv, D), dtype=dt)

            def new_rows(r):
                qs, qe = int(qsl[r]), int(qsl[r + 1])
                ctx = int(seq[r]) - (qe - qs)
                i = int(idx[r])
                return qs, qe, [w.values(n, i, l, ctx, ctx + qe - qs) for n in ("q", "k", "v")]

            for qs, qe, (a, b, c) in pool.map(new_rows, range(N)):
                q[qs:qe] = torch.from_numpy(a).to(dt)
                kn[qs:qe] = torch.from_numpy(b).to(dt)
                vn[qs:qe] = torch.from_numpy(c).to(dt)
            plan = plans[l]
            ws_bytes = workspace_size(plan)
            ws = torch.empty(ws_bytes, dtype=torch.uint8, device=device) if ws_bytes else None
            layers.append(LayerState(lay.name, lay.window_left, lay.ring_len > 0, kc, vc, plan,
                                     view(3 * l + 2), view(3 * l, (N, L["width"])), view(3 * l + 1),
                                     q.to(device), kn.to(device), vn.to(device),
                                     torch.empty((T, Hq, D), dtype=dt, device=device), ws))
            if verbose:
                print(f"[step] layer {lay.name}: plan {plan.counts()}", flush=True)
        pool.shutdown()
        torch.cuda.synchronize()
        return cls(sched, layers, w.scale, dt, Hq, Hkv, D, P)


def history_slots(pages: np.ndarray, lo: int, hi: int, P: int, ring_len: int) -> np.ndarray:
    """Cache slots (page * P + offset) of positions lo .. hi-1 of a request owning `pages` (logical order, or a
    ring of ring_len pages)."""
    pos = np.arange(lo, hi, dtype=np.int64)
    blk = pos // P
    if ring_len > 0:
        blk = blk % ring_len
    return (pages.astype(np.int64)[blk] * P + pos % P).astype(np.int32)


def _fill_history(w, l: int, kc, vc, pool, device, dt, chunk_tokens: int = 1 << 18) -> None:
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
        s = history_slots(np.asarray(w.requests[i].pages[l]), lo, hi, P, lay.ring_len)
        return torch.from_numpy(k).to(dt), torch.from_numpy(v).to(dt), torch.from_numpy(s)

    batch, n = [], 0

    def flush():
        nonlocal batch, n
        if not batch:
            return
        k = torch.cat([b[0] for b in batch]).to(device)
        v = torch.cat([b[1] for b in batch]).to(device)
        s = torch.cat([b[2] for b in batch]).to(device)
        kv_append(kc, vc, k, v, s)
        batch, n = [], 0

    group = 16   # requests generated ahead of the copies, bounding host memory
    for g0 in range(0, len(jobs), group):
        for res in pool.map(gen, jobs[g0:g0 + group]):
            batch.append(res)
            n += res[0].shape[0]
            if n >= chunk_tokens:
                flush()
    flush()


class StepPipeline:
    """Runs a step again and again the way a serving loop would, every stage included each time.

    Per step: the host schedules (cb_build_metadata) and plans every layer (cb_plan_attention) straight into a
    pinned int32 buffer, which one asynchronous copy moves to the device; two host/device buffer pairs alternate,
    so the host prepares step k+1 while the device still runs step k (the double-buffered async batching of the
    Transformers "continuous batching architecture" page). Then, in stream order: the KV append of every layer,
    the split-KV decode kernel, the prefill-tile and per-token kernels, and the merge of split rows.

    concurrent=True runs the prefill-tile and per-token kernels on a second compute stream beside the decode kernel
    (decode streams HBM while prefill keeps the matrix cores busy) and joins both before the merge. copy_stream=True
    moves the metadata copy to a stream of its own, so that it overlaps the previous step's kernels instead of
    sitting between steps. graphs=True replays the step's kernels as a captured HIP graph whenever the step's launch
    configuration (metadata buffer, plans, token count) was seen before. fused_append=True (the default, except with
    concurrent=True, whose prefill kernels would race the append) has cb_paged_attention write the new K/V itself:
    the append's work groups run after the decode work groups in the decode launch, in the decode kernel's tail,
    instead of in a launch of their own. All streams have the default priority.
    """

    def __init__(self, w, step: Step, decode_split: int = 0, prefill_split: int = 0, concurrent: bool = False,
                 copy_stream: bool = True, graphs: bool = False, fused_append: bool = True):
        from . import Scheduler
        torch = _torch()
        self.step = step
        self.w = w
        self.concurrent = concurrent
        self.fused = fused_append and not concurrent
        pools = [{"ring_len": lay.ring_len, "window_left": lay.window_left,
                  "pool_pages": lay.num_pages - len(lay.padding_pages), "free_pages": lay.free_pages}
                 for lay in w.layers]
        pad = w.layers[0].padding_pages[0] if w.layers[0].padding_pages else 0
        self.sched = Scheduler(w.requests, pools, w.max_batch_tokens, w.max_requests, w.page_size, w.safety_margin,
                               pad, policy=w.policy)
        dt = _abi.CB_DTYPE_BF16 if w.dtype == "bf16" else _abi.CB_DTYPE_F32
        self.shapes = [_abi.cb_attn_shape(w.Hq, w.Hkv, w.D, w.page_size, dt, lay.window_left, decode_split,
                                          prefill_split) for lay in w.layers]
        # capacity: the one-off Step already built this schedule and these plans
        meta = 8 * (step.sched["num_tokens"] + 4 * step.sched["num_reqs"] + 64) + sum(
            L["block_table"].size for L in step.sched["layers"])
        plan = sum(L.plan.buffer.size for L in step.layers)
        self.meta_cap = int(meta)
        self.cap = int(meta + 2 * plan + 1024)
        dev = step.layers[0].out.device
        self.host = [torch.empty(self.cap, dtype=torch.int32, pin_memory=True) for _ in range(2)]
        self.dev = [torch.empty(self.cap, dtype=torch.int32, device=dev) for _ in range(2)]
        self.main = torch.cuda.current_stream(dev)
        self.aux = torch.cuda.Stream(dev) if concurrent else None
        self.copier = torch.cuda.Stream(dev) if copy_stream else None
        # events are created once (torch creates the HIP event at its first record) and re-recorded every step
        self.copy_ev = [torch.cuda.Event(), torch.cuda.Event()]   # copy into buffer pair i finished
        # last kernels reading device buffer i finished: it only orders the next copy into that buffer after reads,
        # so it is recorded without the system-scope fence
        self.rel_ev = [HipEvent(system_fence=False), HipEvent(system_fence=False)]
        self.fork = torch.cuda.Event()
        self.join = torch.cuda.Event()
        for e in (*self.copy_ev, *self.rel_ev, self.fork, self.join):
            e.record(self.main)
        self.copied = [None, None]
        self.released = [None, None]
        self.k = 0
        # launch arguments marshalled once: only the per-step metadata pointers change between steps
        self.lib = _abi.load()
        self.h_main = C.c_void_p(self.main.cuda_stream)
        self.h_aux = C.c_void_p(self.aux.cuda_stream) if self.aux is not None else None
        self.args = []
        for l, L in enumerate(step.layers):
            a = _abi.cb_attn_args()
            a.out, a.q = L.out.data_ptr(), L.q.data_ptr()
            a.k_cache, a.v_cache = L.k_cache.data_ptr(), L.v_cache.data_ptr()
            a.shape = self.shapes[l]
            a.num_pages = L.k_cache.shape[0]
            a.scale = float(step.scale)
            a.workspace = L.workspace.data_ptr() if L.workspace is not None else None
            a.workspace_bytes = L.workspace.numel() if L.workspace is not None else 0
            self.args.append(a)
        self.append_args = [(L.k_cache.data_ptr(), L.v_cache.data_ptr(), L.k_new.data_ptr(), L.v_new.data_ptr(),
                             L.k_cache.shape[0], L.k_new.shape[0]) for L in step.layers]
        self.dtype = dt
        self.use_graphs = graphs
        self.graphs = {}

    def prepare(self):
        """Host half of a step: schedule + plan into the next pinned buffer and enqueue its copy to the device on
        the compute stream (stream order keeps it after the previous step's kernels that read that buffer).
        Returns the per-layer device views."""
        torch = _torch()
        from . import plan_into
        i = self.k % 2
        self.k += 1
        if self.copied[i] is not None:
            self.copied[i].synchronize()   # the pinned half of pair i is free again
        host = self.host[i].numpy()
        hs = self.sched.build_into(host[:self.meta_cap])
        N, T = hs.num_reqs, hs.num_tokens
        qsl = host[hs.off_query_start_loc:hs.off_query_start_loc + N + 1]
        seq = host[hs.off_seq_lens:hs.off_seq_lens + N]
        at = int(hs.used)
        plans = []
        for l, lay in enumerate(self.w.layers):
            ring = host[hs.off_ring_len[l]:hs.off_ring_len[l] + N] if lay.ring_len > 0 else None
            p = plan_into(qsl, seq, ring, self.shapes[l], host[at:])
            plans.append((p, at))
            at += int(p.info.used)
        dev = self.dev[i]
        ev = self.copy_ev[i]
        if self.copier is not None:
            # the copy waits only for the step that last read this device buffer, then runs beside the kernels of
            # the step in flight; the compute stream waits for it before this step's first kernel
            if self.released[i] is not None:
                self.released[i].wait(self.copier)
            with torch.cuda.stream(self.copier):
                dev[:at].copy_(self.host[i][:at], non_blocking=True)
            ev.record(self.copier)
            self.main.wait_event(ev)
        else:
            dev[:at].copy_(self.host[i][:at], non_blocking=True)
            ev.record(self.main)
        self.copied[i] = ev
        self.cur = i
        base = dev.data_ptr()
        views = []
        for l in range(len(self.w.layers)):
            p, off = plans[l]
            views.append((base + 4 * int(hs.off_block_table[l]), int(hs.table_width[l]),
                          base + 4 * int(hs.off_slot_mapping[l]), p.info, base + 4 * off))
        self.num_tokens = T
        return views

    def _check(self, status, what):
        if status != 0:
            raise CbError(status, what)

    def _launch(self, views, stream, handle, events=None):
        """Enqueue the step's kernels for the prepared metadata `views` on `stream` (C handle `handle`)."""
        lib = self.lib
        w = self.w
        T = self.num_tokens
        for l, (bt, width, sm, info, plan) in enumerate(views):
            kc, vc, kn, vn, n_pages, rows = self.append_args[l]
            if T > rows:
                raise ValueError("step has more new tokens than the pipeline's input rows")
            a = self.args[l]
            if self.fused:
                a.k_new, a.v_new, a.slot_mapping, a.num_new = kn, vn, sm, T
            else:
                a.k_new = a.v_new = a.slot_mapping = None
                a.num_new = 0
                self._check(lib.cb_kv_append(kc, vc, kn, vn, sm, T, n_pages, w.page_size, w.Hkv, w.D, self.dtype,
                                             handle), "cb_kv_append")

        def attend(l, phases, ev0=None, ev1=None, aux=False):
            bt, width, sm, info, plan = views[l]
            a = self.args[l]
            a.block_table, a.table_width, a.plan, a.plan_info, a.phases = bt, width, plan, info, phases
            s = self.aux if aux else stream
            if ev0 is not None:
                ev0.record(s)
            self._check(lib.cb_paged_attention(C.byref(a), self.h_aux if aux else handle), "cb_paged_attention")
            if ev1 is not None:
                ev1.record(s)

        n = len(views)
        E = (lambda l, k: events[l][k]) if events else (lambda l, k: None)
        pre = CB_PHASE_ROWWISE | CB_PHASE_PREFILL
        if self.concurrent:
            self.fork.record(stream)
            self.aux.wait_event(self.fork)
            for l in range(n):
                attend(l, pre, E(l, 2), E(l, 3), aux=True)
            for l in range(n):
                attend(l, CB_PHASE_DECODE, E(l, 0), E(l, 1))
            self.join.record(self.aux)
            stream.wait_event(self.join)
        else:
            for l in range(n):
                attend(l, CB_PHASE_DECODE, E(l, 0), E(l, 1))
                attend(l, pre, E(l, 2), E(l, 3))
        for l in range(n):
            attend(l, CB_PHASE_COMBINE, E(l, 4), E(l, 5))

    def _graph_for(self, views):
        """The step's kernels captured as a HIP graph, cached by everything their launches depend on: the metadata
        buffer (its device address), the plans (item counts, split sizes, section offsets), the block-table width
        and the token count. A step whose launch configuration was seen before replays its graph."""
        torch = _torch()
        key = (self.cur, self.num_tokens) + tuple(
            (bt, width, sm, plan, bytes(info)) for (bt, width, sm, info, plan) in views)
        g = self.graphs.get(key)
        if g is None:
            side = torch.cuda.Stream(self.main.device)
            side.wait_stream(self.main)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(side):
                g.capture_begin()
                self._launch(views, side, C.c_void_p(side.cuda_stream))
                g.capture_end()
            self.main.wait_stream(side)
            self.graphs[key] = g
        return g

    def run(self, events=None):
        """One full step. `events`, if given, holds per layer 6 timing events: decode start/end (compute stream),
        prefill start/end (the stream running the prefill-tile and per-token kernels), merge start/end. With
        graphs=True the step replays a captured graph, except when it carries events (then it runs eagerly)."""
        views = self.prepare()
        main = self.main
        if self.use_graphs and events is None and not self.concurrent:
            self._graph_for(views).replay()
        else:
            self._launch(views, main, self.h_main, events)
        if self.copier is not None:
            rel = self.rel_ev[self.cur]
            rel.record(main)
            self.released[self.cur] = rel
