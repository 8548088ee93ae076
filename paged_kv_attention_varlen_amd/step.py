"""Device driver for one mixed step: metadata -> plans -> one host-to-device copy -> KV append -> attention.

`Step` holds the device state of one scheduled step for one or two layer types (a full layer, optionally a sliding
layer) that share the step's schedule: per layer the caches, the step's new Q/K/V rows, the output, the plan and its
device copy, and the workspace. `StepPipeline` runs such a step again and again the way a serving loop does, every
host and device stage included each time. Neither knows where the tensors' contents came from.
"""
from __future__ import annotations

import ctypes as C
from collections import OrderedDict
from dataclasses import dataclass
from typing import List, Optional

import numpy as np

from .hip_events import HipEvent, memcpy_h2d_async
from . import (CB_LAYOUT_KD_VT, CB_PHASE_COMBINE, CB_PHASE_DECODE, CB_PHASE_PREFILL, CB_PHASE_ROWWISE, AttnPlan,
               CB_E_CAPACITY, CbError, Scheduler, _abi, check_dtypes, kv_append, paged_attention,
               schedule_arrays)


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


def _roundup(x: int, m: int) -> int:
    return -(-int(x) // m) * m if m > 1 else int(x)


class _Full(Exception):
    """The padded metadata of a step does not fit the pipeline's buffers (they are then doubled), or its padded plan
    needs more workspace than layer `layer` holds."""

    def __init__(self, layer=None, need=0):
        super().__init__()
        self.layer, self.need = layer, need


class StepPipeline:
    """Runs steps the way a serving loop does, every host and device stage included each time.

    Per step: the host schedules (cb_build_metadata, through `scheduler`, whose requests and free lists the caller
    may replace between steps with Scheduler.set_state) and plans every layer (cb_plan_attention) into a pinned int32
    buffer, which one asynchronous copy moves to the device; two host/device buffer pairs alternate, so the host
    prepares step k+1 while the device still runs step k (the double-buffered async batching of the Transformers
    "continuous batching architecture" page). Then, in stream order: the KV append of every layer, the split-KV
    decode kernel, the prefill-tile and per-token kernels, and the merge of split rows. The step's new Q/K/V rows are
    read from `step`'s tensors (row t = token t of the step), which the caller fills before `run`, in stream order on
    the compute stream; they must have a row per token.

    concurrent=True runs the prefill-tile and per-token kernels on a second compute stream beside the decode kernel
    and joins both before the merge. copy_stream=True moves the metadata copy to a stream of its own, so that it
    overlaps the previous step's kernels instead of sitting between steps. fused_append=True (the default, except
    with concurrent=True, whose prefill kernels would race the append) has cb_paged_attention write the new K/V
    itself: the append's work groups run after the decode work groups in the decode launch. All streams have the
    default priority.

    graphs=True replays the step's kernels as captured HIP graphs keyed by a padded shape (same page, section "CUDA
    图"): the token count is padded to a multiple of q_interval, every full layer's block-table width to a multiple of
    kv_interval tokens, the block-table rows to a multiple of 16, and each section of every plan (decode, prefill,
    per-token and merge items) and its count of split slots (which fixes the workspace layout) to a multiple of
    item_interval. The metadata is then written at addresses that depend
    only on the padded shape, the launches are sized for its capacities, and the kernels read the step's actual item
    counts from the device buffer (the `counts` argument of cb_paged_attention), so one graph serves every step that
    pads to the same shape. Padded tokens write their (unused) K/V rows into the reserved padding page, whose
    contents are never read as valid keys (same page, section "内存管理"). At most max_graphs graphs are kept, the
    least recently used evicted first.
    """

    def __init__(self, step: Step, scheduler: Scheduler, decode_split: int = 0, prefill_split: int = 0,
                 prefill_rows: int = 0, concurrent: bool = False, copy_stream: bool = True, graphs: bool = False, fused_append: bool = True,
                 q_interval: int = 64, kv_interval: int = 256, item_interval: int = 64, max_graphs: int = 8):
        torch = _torch()
        self.step = step
        self.sched = scheduler
        self.concurrent = concurrent
        self.fused = fused_append and not concurrent
        self.P = step.P
        self.n_layers = len(step.layers)
        if scheduler.L != self.n_layers or scheduler.page_size != step.P:
            raise ValueError("scheduler and step disagree on layers or page size")
        dt = _abi.CB_DTYPE_BF16 if str(step.dtype) == "torch.bfloat16" else _abi.CB_DTYPE_F32
        self.dtype = dt
        self.shapes = [_abi.cb_attn_shape(step.Hq, step.Hkv, step.D, step.P, dt, scheduler.windows[l], decode_split,
                                          prefill_split, prefill_rows) for l in range(self.n_layers)]
        self._shape_arr = (_abi.cb_attn_shape * max(self.n_layers, 1))(*self.shapes)
        for L in step.layers:
            check_dtypes(AttnPlan(None, self.shapes[0], None), q=L.q, out=L.out, k_cache=L.k_cache,
                         v_cache=L.v_cache, k_new=L.k_new, v_new=L.v_new)
        self.rows = min(L.q.shape[0] for L in step.layers)          # token capacity of the step's tensors
        self.use_graphs = graphs
        self.qi, self.kvi, self.ii = int(q_interval), int(kv_interval), int(item_interval)
        self.max_graphs = int(max_graphs)
        # buffer sizes start from the step the tensors were built for and double whenever a step needs more
        self.meta_cap = int(2 * (4 * step.sched["num_reqs"] + step.sched["num_tokens"] * self.n_layers + 64 + sum(
            Ls["block_table"].size + Ls["ring_len"].size for Ls in step.sched["layers"])) + 4096)
        self.plan_cap = int(2 * sum(L.plan.buffer.size for L in step.layers) + 4096)
        self.device = step.layers[0].out.device
        self.graphs = OrderedDict()
        self._alloc()
        dev = self.device
        self.main = torch.cuda.current_stream(dev)
        self.aux = torch.cuda.Stream(dev) if concurrent else None
        self.copier = torch.cuda.Stream(dev) if copy_stream else None
        # events are created once (torch creates the HIP event at its first record) and re-recorded every step
        # copy into buffer pair i finished: the kernels read what it copied, so it keeps the system-scope fence
        self.copy_ev = [HipEvent(), HipEvent()]
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
        self.h_copier = C.c_void_p(self.copier.cuda_stream) if self.copier is not None else None
        self.args = []
        for l, L in enumerate(step.layers):
            a = _abi.cb_attn_args()
            a.out, a.q = L.out.data_ptr(), L.q.data_ptr()
            a.k_cache, a.v_cache = L.k_cache.data_ptr(), L.v_cache.data_ptr()
            a.layout = CB_LAYOUT_KD_VT
            a.shape = self.shapes[l]
            a.num_pages = L.k_cache.shape[0]
            a.scale = float(step.scale)
            a.workspace = L.workspace.data_ptr() if L.workspace is not None else None
            a.workspace_bytes = L.workspace.numel() if L.workspace is not None else 0
            self.args.append(a)
        self.workspaces = [L.workspace for L in step.layers]
        self.ws_fits = [0] * self.n_layers     # split slots each layer's workspace is known to hold
        self.append_args = [(L.k_cache.data_ptr(), L.v_cache.data_ptr(), L.k_new.data_ptr(), L.v_new.data_ptr(),
                             L.k_cache.shape[0]) for L in step.layers]
        self.captures = 0          # graphs captured so far (evicted ones included)
        self.replays = 0
        self.key = None
        self.last_header = None    # cb_step header of the last prepared step
        self.last_plans = None     # its per-layer plan headers
        self._advanced = 0         # the step count (self.k) at the last advance(): at most one per prepared step
        self.keep_schedule = False  # True: prepare() also keeps the step's metadata as numpy arrays (last_schedule)
        self.last_schedule = None

    # ---------------------------------------------------------------------------------------------- host half
    def _alloc(self):
        """(Re)allocate the two pinned / device buffer pairs: [scheduler output | plans | padded metadata]."""
        torch = _torch()
        pad_cap = 2 * self.meta_cap + 2 * self.plan_cap + 64 * self.n_layers if self.use_graphs else 0
        self.cap = self.meta_cap + self.plan_cap + pad_cap
        self.host = [torch.empty(self.cap, dtype=torch.int32, pin_memory=True) for _ in range(2)]
        self.dev = [torch.empty(self.cap, dtype=torch.int32, device=self.device) for _ in range(2)]
        # per buffer pair, made once: host views and addresses, and the header and plan records cb_build_step fills
        # (a step's records stay valid until its buffer pair is scheduled into again, two steps later)
        L = self.n_layers
        self._host_np = [h.numpy() for h in self.host]
        self._host_addr = [h.data_ptr() for h in self.host]
        self._dev_addr = [d.data_ptr() for d in self.dev]
        self._hdr = [_abi.cb_step() for _ in range(2)]
        self._plan_infos = [(_abi.cb_plan * max(L, 1))() for _ in range(2)]
        self._plan_offs = [(C.c_int64 * max(L, 1))() for _ in range(2)]
        self.graphs.clear()    # captured launches point into the old buffers

    def _grow(self):
        torch = _torch()
        torch.cuda.synchronize(self.device)
        self.meta_cap *= 2
        self.plan_cap *= 2
        self._alloc()
        self.copied = [None, None]
        self.released = [None, None]

    def _grow_workspace(self, l, need):
        """Give layer l a workspace of at least `need` bytes (twice that, so that growth stays rare). The pipeline
        owns it from then on; captured graphs point at the old one and are dropped."""
        torch = _torch()
        torch.cuda.synchronize(self.device)
        ws = torch.empty(2 * need, dtype=torch.uint8, device=self.device)
        self.workspaces[l] = ws
        self.ws_fits[l] = 0
        self.args[l].workspace, self.args[l].workspace_bytes = ws.data_ptr(), ws.numel()
        self.graphs.clear()

    def _check_workspace(self, l, info):
        """Raise _Full(l, bytes) if layer l's workspace is too small for a plan with info's split slots."""
        if info.n_partials <= self.ws_fits[l]:
            return
        probe = _abi.cb_attn_args()
        probe.plan_info, probe.shape = info, self.shapes[l]
        need = int(self.lib.cb_paged_attention_workspace_size(C.byref(probe)))
        if need > self.args[l].workspace_bytes:
            raise _Full(l, need)
        self.ws_fits[l] = info.n_partials

    def _host_step(self, i):
        """Schedule and plan into pinned buffer i (one cb_build_step call); with graphs=True also lay the metadata out
        at its padded shape. Returns (header, plans, copy range lo, hi, launch views, graph key)."""
        host = self._host_np[i]
        hs, infos, offs = self._hdr[i], self._plan_infos[i], self._plan_offs[i]
        self.sched.build_step_into(self._host_addr[i], self.meta_cap, self.meta_cap + self.plan_cap, self._shape_arr,
                                   hs, infos, offs)
        T = hs.num_tokens
        if T > self.rows:
            raise ValueError(f"step has {T} tokens, the step's tensors hold {self.rows}")
        L = self.n_layers
        plans = [(AttnPlan(infos[l], self.shapes[l], None), self.meta_cap + int(offs[l])) for l in range(L)]
        if self.use_graphs:
            return (hs, plans) + self._pad(host, hs, plans, i)
        for l in range(L):
            self._check_workspace(l, infos[l])
        base = self._dev_addr[i]
        views = [(base + 4 * int(hs.off_block_table[l]), int(hs.table_width[l]),
                  base + 4 * int(hs.off_slot_mapping[l]), infos[l], base + 4 * off, None, T)
                 for l, (_, off) in enumerate(plans)]
        end = plans[-1][1] + int(infos[L - 1].used) if L else self.meta_cap
        return hs, plans, 0, end, views, None

    def _pad(self, host, hs, plans, i):
        """Write the step's metadata at the addresses of its padded shape (see the class docstring): per layer the
        block table, the slot mapping (padded tokens point into the padding page), the actual item counts, and the
        plan with every section at its capacity. Returns (copy range lo, hi, launch views, graph key)."""
        N, T = hs.num_reqs, hs.num_tokens
        P = self.P
        Tp = min(_roundup(max(T, 1), self.qi), self.rows)
        Np = _roundup(max(N, 1), 16)
        widths, caps = [], []
        for l, (p, _) in enumerate(plans):
            w = int(hs.table_width[l])
            wp = w if self.sched.rings[l] > 0 else _roundup(max(w, 1), max(1, self.kvi // P))
            widths.append(wp)
            info = p.info
            # n_partials sets where the workspace's second region (split maxima and sums) starts, so it is padded
            # and keyed like the item counts
            caps.append(tuple(_roundup(x, self.ii) for x in (info.n_decode, info.n_prefill, info.n_rowwise,
                                                             info.n_combine, info.n_partials)))
        at = lo = self.meta_cap + self.plan_cap
        need = at + sum(Np * wp + Tp + 8 + 8 * sum(c[:3]) + 4 * c[3] for wp, c in zip(widths, caps))

        if need > self.cap:
            raise _Full()
        base = self.dev[i].data_ptr()
        views = []
        for l, (p, poff) in enumerate(plans):
            w, wp = int(hs.table_width[l]), widths[l]
            bt = host[at:at + Np * wp].reshape(Np, wp)
            bt[:] = self.sched.pad_page
            if N and w:
                bt[:N, :w] = host[hs.off_block_table[l]:hs.off_block_table[l] + N * w].reshape(N, w)
            bt_at = at
            at += Np * wp
            sm = host[at:at + Tp]
            sm[:T] = host[hs.off_slot_mapping[l]:hs.off_slot_mapping[l] + T]
            sm[T:] = self.sched.pad_page * P + (np.arange(Tp - T) % P)
            sm_at = at
            at += Tp
            info = p.info
            cnt = host[at:at + 8]
            cnt[:] = 0
            cnt[:4] = (info.n_decode, info.n_prefill, info.n_rowwise, info.n_combine)
            cnt_at = at
            at += 8
            src = host[poff:poff + int(info.used)]
            padded = _abi.cb_plan()
            C.memmove(C.byref(padded), C.byref(info), C.sizeof(padded))
            pl_at = at
            offs = []
            for n, off, width, cap in ((info.n_decode, info.off_decode, 8, caps[l][0]),
                                       (info.n_prefill, info.off_prefill, 8, caps[l][1]),
                                       (info.n_rowwise, info.off_rowwise, 8, caps[l][2]),
                                       (info.n_combine, info.off_combine, 4, caps[l][3])):
                offs.append(at - pl_at)
                host[at:at + n * width] = src[off:off + n * width]
                at += cap * width
            padded.n_decode, padded.n_prefill, padded.n_rowwise, padded.n_combine, padded.n_partials = caps[l]
            padded.off_decode, padded.off_prefill, padded.off_rowwise, padded.off_combine = offs
            padded.used = at - pl_at
            padded.num_tokens = Tp
            self._check_workspace(l, padded)
            views.append((base + 4 * bt_at, wp, base + 4 * sm_at, padded, base + 4 * pl_at, base + 4 * cnt_at, Tp))
        # the prefill tile size picks the prefill kernel's work-group shape: part of the launch, so part of the key
        tiles = tuple(int(p.info.prefill_tokens) for p, _ in plans)
        return lo, at, views, (i, Tp, Np, tuple(widths), tuple(caps), tiles)

    def prepare(self):
        """Host half of a step: schedule + plan into the next pinned buffer and enqueue its copy to the device.
        Returns the per-layer launch views (block table, width, slot mapping, plan header, plan, counts, tokens)."""
        i = self.k % 2
        if self.copied[i] is not None:
            self.copied[i].synchronize()   # the pinned half of pair i is free again
        while True:
            try:
                hs, plans, lo, hi, views, key = self._host_step(i)
                break
            except CbError as e:
                if e.status != CB_E_CAPACITY:
                    raise
                self._grow()
            except _Full as e:
                if e.layer is None:
                    self._grow()
                else:
                    self._grow_workspace(e.layer, e.need)
        self.k += 1
        # copies: the records themselves belong to the buffer pair and are rewritten two steps later
        self.last_header = _abi.cb_step.from_buffer_copy(hs)
        self.last_plans = [_abi.cb_plan.from_buffer_copy(p.info) for p, _ in plans]
        if self.keep_schedule:
            self.last_schedule = schedule_arrays(self._host_np[i], hs, self.n_layers)
        self.num_tokens = hs.num_tokens
        ev = self.copy_ev[i]
        dst, src, nbytes = self._dev_addr[i] + 4 * lo, self._host_addr[i] + 4 * lo, 4 * (hi - lo)
        if self.copier is not None:
            # the copy waits only for the step that last read this device buffer, then runs beside the kernels of
            # the step in flight; the compute stream waits for it before this step's first kernel
            if self.released[i] is not None:
                self.released[i].wait_on(self.h_copier)
            memcpy_h2d_async(dst, src, nbytes, self.h_copier)
            ev.record_on(self.h_copier)
            ev.wait_on(self.h_main)
        else:
            memcpy_h2d_async(dst, src, nbytes, self.h_main)
            ev.record_on(self.h_main)
        self.copied[i] = ev
        self.cur = i
        self.key = key
        return views

    def _check(self, status, what):
        if status != 0:
            raise CbError(status, what)

    # -------------------------------------------------------------------------------------------- device half
    def _launch(self, views, stream, handle, events=None):
        """Enqueue the step's kernels for the prepared metadata `views` on `stream` (C handle `handle`)."""
        lib = self.lib
        st = self.step
        for l, (bt, width, sm, info, plan, counts, T) in enumerate(views):
            kc, vc, kn, vn, n_pages = self.append_args[l]
            a = self.args[l]
            a.counts = counts
            if self.fused:
                a.k_new, a.v_new, a.slot_mapping, a.num_new = kn, vn, sm, T
            else:
                a.k_new = a.v_new = a.slot_mapping = None
                a.num_new = 0
                self._check(lib.cb_kv_append(kc, vc, kn, vn, sm, T, n_pages, self.P, st.Hkv, st.D, self.dtype,
                                             CB_LAYOUT_KD_VT, handle), "cb_kv_append")

        def attend(l, phases, ev0=None, ev1=None, aux=False):
            bt, width, sm, info, plan, counts, T = views[l]
            a = self.args[l]
            a.block_table, a.table_width, a.plan, a.plan_info, a.phases = bt, width, plan, info, phases
            # the events are recorded by the call's first and last kernels as they start and end, so that the pair
            # times the kernels, not the dispatch after the previous work or the completion signal after them
            a.timing_start = ev0.handle if ev0 is not None else None
            a.timing_stop = ev1.handle if ev1 is not None else None
            self._check(lib.cb_paged_attention(C.byref(a), self.h_aux if aux else handle), "cb_paged_attention")
            a.timing_start = a.timing_stop = None

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
        elif not events:
            # no per-phase events: one call per layer launches its decode, per-token, prefill and merge kernels in
            # that order (the layers are independent, so each layer's merge may precede the next layer's kernels)
            for l in range(n):
                attend(l, 0)
            return
        else:
            for l in range(n):
                attend(l, CB_PHASE_DECODE, E(l, 0), E(l, 1))
                attend(l, pre, E(l, 2), E(l, 3))
        for l in range(n):
            attend(l, CB_PHASE_COMBINE, E(l, 4), E(l, 5))

    def _graph_for(self, views):
        """The step's kernels captured as a HIP graph for the step's padded shape (captured at its first use)."""
        torch = _torch()
        g = self.graphs.get(self.key)
        if g is not None:
            self.graphs.move_to_end(self.key)
            return g
        side = torch.cuda.Stream(self.main.device)
        side.wait_stream(self.main)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            g.capture_begin()
            self._launch(views, side, C.c_void_p(side.cuda_stream))
            g.capture_end()
        self.main.wait_stream(side)
        self.graphs[self.key] = g
        self.captures += 1
        while len(self.graphs) > self.max_graphs:
            self.graphs.popitem(last=False)
        return g

    def run(self, events=None):
        """One full step: prepare() then launch()."""
        self.launch(self.prepare(), events)

    def advance(self) -> None:
        """The request lifecycle after the last prepared step (Scheduler.advance_step, in native code, on the pinned
        metadata that step was scheduled into). A serving loop calls it once per step, after launch() and before
        the next prepare(); without it every step repeats the same schedule."""
        if self._advanced == self.k:
            raise RuntimeError("advance() was already called for this step; prepare() the next step first")
        self.sched.advance_step(self.last_header, self._host_np[self.cur])
        self._advanced = self.k

    def launch(self, views, events=None):
        """The device half of a prepared step. A caller that writes the step's new Q/K/V rows after seeing its
        schedule (keep_schedule) does so between prepare() and launch(), in stream order on the compute stream.
        `events`, if given, holds per layer 6 timing events: decode start/end (compute stream), prefill start/end
        (the stream running the prefill-tile and per-token kernels), merge start/end. With graphs=True the step
        replays the graph of its padded shape (captured at the shape's first step), except when it carries events:
        then the same padded launches run eagerly."""
        main = self.main
        if self.use_graphs and events is None and not self.concurrent:
            self._graph_for(views).replay()
            self.replays += 1
        else:
            self._launch(views, main, self.h_main, events)
        if self.copier is not None:
            rel = self.rel_ev[self.cur]
            rel.record_on(self.h_main)
            self.released[self.cur] = rel
