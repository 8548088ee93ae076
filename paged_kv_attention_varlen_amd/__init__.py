"""MI355X-native mixed-batch paged attention step of continuous batching.

Thin Python binding over the C ABI of libcb.so (include/cb.h); same call names. It only marshals arguments: the
scheduler, the planner and every kernel run inside the library. Device buffers are torch tensors (torch is used for
device memory and streams only). There is no fallback: if libcb.so is missing or the GPU is absent, calls raise.

    build_metadata   -> cb_build_metadata   (host)
    plan_attention   -> cb_plan_attention   (host)
    kv_append        -> cb_kv_append        (device, current torch stream)
    paged_attention  -> cb_paged_attention  (device, current torch stream)
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass

import numpy as np

from . import _abi
from ._abi import (CB_DECODING, CB_DTYPE_BF16, CB_DTYPE_F32, CB_E_CAPACITY, CB_E_NOSPACE, CB_OK,  # noqa: F401
                   CB_LAYOUT_KD_VT, CB_LAYOUT_PAGED_NHD, CB_PHASE_COMBINE, CB_PHASE_DECODE, CB_PHASE_PREFILL, CB_PHASE_ROWWISE, CB_POLICY_FIFO,
                   CB_POLICY_PREFILL_FIRST, CB_PREFILLING, CB_WAITING, CbError)

POLICIES = {"fifo": CB_POLICY_FIFO, "prefill_first": CB_POLICY_PREFILL_FIRST}

__all__ = ["build_metadata", "plan_attention", "kv_append", "paged_attention", "workspace_size", "AttnPlan",
           "Scheduler", "Request", "advance", "schedule_arrays", "plan_into", "slot_mapping", "validate_metadata", "check_dtypes", "load_library", "CbError"]


def load_library():
    return _abi.load()


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_abi.i32p) if a.size else C.cast(C.c_void_p(0), _abi.i32p)


# ------------------------------------------------------------------------------------------- cb_build_metadata

def _marshal_requests(requests, L, prompt_hashes, keep):
    n = len(requests)
    reqs = (_abi.cb_req * max(n, 1))()
    for i, rq in enumerate(requests):
        r = reqs[i]
        r.id, r.state, r.num_computed, r.num_pending = int(rq.id), int(rq.state), int(rq.num_computed), \
            int(rq.num_pending)
        for l in range(L):
            p = _i32(rq.pages[l])
            keep.append(p)
            r.n_pages[l] = p.size
            r.pages[l] = _ptr(p)
        h = None if prompt_hashes is None else prompt_hashes[i]
        if h is not None and len(h):
            h = np.ascontiguousarray(np.asarray(h, dtype=np.uint64))
            keep.append(h)
            r.prompt_hashes = h.ctypes.data_as(C.POINTER(C.c_uint64))
            r.n_prompt_blocks = h.size
    return reqs


def build_metadata(requests, layers, max_batch_tokens: int, max_requests: int, page_size: int,
                   safety_margin: float = 0.0, pad_page: int = 0, policy: str = "fifo", prefix_cache=None,
                   prompt_hashes=None) -> dict:
    """Schedule one step (cb_build_metadata). policy: "fifo" or "prefill_first".

    requests: sequence of objects with .id, .state (0 decoding / 1 prefilling / 2 waiting), .num_computed,
      .num_pending and .pages (one int array per layer), in arrival order.
    layers: sequence of dicts {ring_len, window_left, pool_pages, free_pages}.
    prefix_cache: a PrefixCache for prefix sharing at admission, with prompt_hashes[i] the chain hashes of request
      i's full prompt blocks (or None); the call then takes references in the cache.
    Returns a dict with "status" (int) and, unless the input was invalid, the metadata as numpy arrays.
    """
    lib = _abi.load()
    n = len(requests)
    L = len(layers)
    keep = []
    reqs = _marshal_requests(requests, L, prompt_hashes, keep)
    pools = (_abi.cb_layer_pool * max(L, 1))()
    for l, lay in enumerate(layers):
        f = _i32(lay["free_pages"])
        keep.append(f)
        pools[l].ring_len = int(lay["ring_len"])
        pools[l].window_left = int(lay["window_left"])
        pools[l].pool_pages = int(lay["pool_pages"])
        pools[l].n_free = f.size
        pools[l].free_pages = _ptr(f)
    params = _abi.cb_sched_params(int(max_batch_tokens), int(max_requests), int(page_size), int(pad_page), L,
                                  POLICIES[policy], float(safety_margin),
                                  prefix_cache._h if prefix_cache is not None else None)
    step = _abi.cb_step()
    cap = 4096
    while True:
        buf = np.zeros(cap, dtype=np.int32)
        st = lib.cb_build_metadata(reqs, n, C.byref(params), pools, _ptr(buf), cap, C.byref(step))
        if st != CB_E_CAPACITY:
            break
        cap = int(step.used)
    if st not in (CB_OK, CB_E_NOSPACE):
        return {"status": st}
    o = schedule_arrays(buf, step, L)
    o["status"] = st
    return o


def slot_mapping(pages, ring_len: int, page_size: int, lo: int, hi: int) -> np.ndarray:
    """cb_slot_mapping: cache slots of key positions lo .. hi-1 of a request owning `pages` (its block-table row,
    or its ring of ring_len pages)."""
    p = _i32(pages)
    out = np.zeros(max(hi - lo, 1), dtype=np.int32)
    st = _abi.load().cb_slot_mapping(_ptr(p), p.size, int(ring_len), int(page_size), int(lo), int(hi), _ptr(out))
    if st != CB_OK:
        raise CbError(st, "cb_slot_mapping")
    return out[:max(hi - lo, 0)]


def validate_metadata(query_start_loc, seq_lens, block_table, ring_len, slot_mapping, num_pages: int,
                      page_size: int, n_reserved: int):
    """cb_validate_metadata on host arrays. Returns None when the metadata is consistent, else (what, index) with
    what in {"query_start_loc", "seq_lens", "block_table", "slot_mapping", "arguments"}."""
    qsl, seq = _i32(query_start_loc), _i32(seq_lens)
    bt = _i32(block_table)
    width = bt.shape[1] if bt.ndim == 2 else 0
    rl = None if ring_len is None else _i32(ring_len)
    sm = None if slot_mapping is None else _i32(slot_mapping)
    what, idx = C.c_int32(), C.c_int32()
    st = _abi.load().cb_validate_metadata(_ptr(qsl), _ptr(seq), seq.size, _ptr(bt), width,
                                          None if rl is None else _ptr(rl), None if sm is None else _ptr(sm),
                                          int(qsl[-1]) if qsl.size else 0, int(num_pages), int(page_size),
                                          int(n_reserved), C.byref(what), C.byref(idx))
    if st == CB_OK:
        return None
    names = {0: "arguments", 1: "query_start_loc", 2: "seq_lens", 3: "block_table", 4: "slot_mapping"}
    return names.get(what.value, "arguments"), idx.value


@dataclass
class Request:
    """One request as the scheduler sees it (the fields of cb_req): state CB_DECODING / CB_PREFILLING / CB_WAITING,
    keys already computed, tokens to feed next, and per layer type the pages it owns (logical order, or its ring)."""
    id: int
    state: int
    num_computed: int
    num_pending: int
    pages: list


def _pack_schedule(schedule: dict):
    """The step metadata of `schedule` (as build_metadata returns it) as a packed int32 buffer and its cb_step
    header: the parts cb_advance reads (rows, seq_lens, req_index, block tables, used pages, prefix sharing)."""
    N = int(schedule["num_reqs"])
    parts = [_i32(schedule["query_start_loc"]), _i32(schedule["seq_lens"]), _i32(schedule["req_index"])]
    hdr = _abi.cb_step()
    hdr.num_reqs, hdr.num_tokens = N, int(schedule["num_tokens"])
    hdr.prefix_sharing = int(bool(schedule.get("prefix_sharing", False)))
    hdr.max_seq_len = int(schedule["seq_lens"].max()) if N else 0
    at = 0
    hdr.off_query_start_loc, at = at, at + N + 1
    hdr.off_seq_lens, at = at, at + N
    hdr.off_req_index, at = at, at + N
    for l, lay in enumerate(schedule["layers"]):
        bt = _i32(lay["block_table"]).reshape(-1)
        hdr.table_width[l] = int(lay["width"])
        hdr.used_pages[l] = int(lay["used_pages"])
        hdr.off_block_table[l], at = at, at + bt.size
        parts.append(bt)
    return np.ascontiguousarray(np.concatenate(parts).astype(np.int32)), hdr


def _store_stride(step, rings, page_size: int) -> int:
    """Pages per request and layer that cb_advance may write after the step `step` (its longest row, or a ring)."""
    return max([-(-int(step.max_seq_len) // page_size)] + [int(r) for r in rings] + [1])


def _unmarshal_requests(requests, reqs, L):
    """Request records from the marshalled cb_req array (page lists copied out of the library's view)."""
    out = []
    for i, rq in enumerate(requests):
        r = reqs[i]
        pages = [np.ctypeslib.as_array(r.pages[l], shape=(r.n_pages[l],)).copy() if r.n_pages[l] > 0
                 else np.zeros(0, np.int32) for l in range(L)]
        out.append(Request(int(rq.id), int(r.state), int(r.num_computed), int(r.num_pending), pages))
    return out


def advance(requests, schedule: dict, free_pages, ring_lens, page_size: int, prefix_cache=None,
            prompt_hashes=None):
    """Request lifecycle after a step has run (cb_advance; Transformers "continuous batching architecture" page,
    section "请求生命周期": a waiting request is admitted and prefilled in chunks, then decodes one token per step).

    schedule: the step's metadata as `build_metadata` returns it. Every scheduled request has now computed its keys
    up to its seq_len (its q_len tokens, plus any prompt tokens it reused from the prefix cache): a request whose
    prompt is done decodes next (one pending token: the one this step produced), otherwise it keeps prefilling; its
    pages are its block-table row (ceil(seq_len / page_size) pages, or its whole ring). Pages the step took leave the
    front of each free list, unless the step shared prefixes (the prefix cache allocated them); then every prompt
    block the step completed is registered in `prefix_cache` under its hash (prompt_hashes[i], chain hashes of
    request i's full prompt blocks), so that later requests can reuse it. Requests the step did not schedule are
    unchanged. Returns (requests, free_pages) as new lists (Request records in the input order)."""
    lib = _abi.load()
    L = len(schedule["layers"])
    n = len(requests)
    keep = []
    reqs = _marshal_requests(requests, L, prompt_hashes, keep)
    buf, hdr = _pack_schedule(schedule)
    pools = (_abi.cb_layer_pool * max(L, 1))()
    free = [_i32(f) for f in free_pages]
    for l in range(L):
        pools[l] = _abi.cb_layer_pool(int(ring_lens[l]), -1, 0, free[l].size, _ptr(free[l]))
    params = _abi.cb_sched_params(1, 1, int(page_size), 0, L, CB_POLICY_FIFO, 0.0,
                                  prefix_cache._h if prefix_cache is not None else None)
    stride = _store_stride(hdr, ring_lens, page_size)
    store = np.zeros(max(n, 1) * L * stride, dtype=np.int32)
    st = lib.cb_advance(reqs, n, C.byref(params), pools, _ptr(buf), C.byref(hdr), _ptr(store), stride)
    if st != CB_OK:
        raise CbError(st, "cb_advance")
    return _unmarshal_requests(requests, reqs, L), [f[f.size - pools[l].n_free:].copy() for l, f in enumerate(free)]


def schedule_arrays(buf: np.ndarray, step, n_layers: int) -> dict:
    """The metadata cb_build_metadata wrote into `buf` (header `step`, n_layers layer types) as a dict of numpy
    copies, in the form `build_metadata` returns."""
    N, T = step.num_reqs, step.num_tokens
    o = {"status": CB_OK, "num_reqs": N, "num_tokens": T, "num_decodes": step.num_decodes,
         "max_q_len": step.max_q_len, "max_seq_len": step.max_seq_len,
         "query_start_loc": buf[step.off_query_start_loc:step.off_query_start_loc + N + 1].copy(),
         "seq_lens": buf[step.off_seq_lens:step.off_seq_lens + N].copy(),
         "req_index": buf[step.off_req_index:step.off_req_index + N].copy(),
         "stalled": buf[step.off_stalled:step.off_stalled + step.n_stalled].copy(),
         "first_rejected": step.first_rejected, "held_by_margin": bool(step.held_by_margin), "layers": [],
         "prefix_sharing": bool(step.prefix_sharing),
         "matched_tokens": buf[step.off_matched:step.off_matched + N].copy()}
    for l in range(n_layers):
        w = step.table_width[l]
        bt = buf[step.off_block_table[l]:step.off_block_table[l] + N * w].reshape(N, w).copy()
        o["layers"].append({"block_table": bt,
                            "slot_mapping": buf[step.off_slot_mapping[l]:step.off_slot_mapping[l] + T].copy(),
                            "ring_len": buf[step.off_ring_len[l]:step.off_ring_len[l] + N].copy(),
                            "used_pages": step.used_pages[l], "width": w})
    return o


class Scheduler:
    """cb_build_metadata's arguments marshalled once, for repeated calls that write into caller buffers (e.g. pinned
    host memory that is then copied to the device in one transfer)."""

    def __init__(self, requests, layers, max_batch_tokens: int, max_requests: int, page_size: int,
                 safety_margin: float = 0.0, pad_page: int = 0, policy: str = "fifo", prefix_cache=None,
                 prompt_hashes=None):
        self._lib = _abi.load()
        self.prefix_cache = prefix_cache
        self.prompt_hashes = prompt_hashes
        self.L = len(layers)
        self.page_size = int(page_size)
        self.pad_page = int(pad_page)
        self.max_batch_tokens = int(max_batch_tokens)
        self.max_requests = int(max_requests)
        self.windows = [int(lay["window_left"]) for lay in layers]
        self.rings = [int(lay["ring_len"]) for lay in layers]
        self.params = _abi.cb_sched_params(int(max_batch_tokens), int(max_requests), int(page_size), int(pad_page),
                                           self.L, POLICIES[policy], float(safety_margin),
                                           prefix_cache._h if prefix_cache is not None else None)
        self.set_state(requests, [lay["free_pages"] for lay in layers], [int(lay["pool_pages"]) for lay in layers])

    def set_state(self, requests, free_pages, pool_pages=None) -> None:
        """Replace the request list (arrival order) and the free lists, e.g. after a step has been taken."""
        L = self.L
        keep = []
        n = len(requests)
        self.n = n
        self._requests = list(requests)
        self._free_pages = [np.asarray(f, dtype=np.int32) for f in free_pages]
        self._stale = False
        reqs = _marshal_requests(requests, L, self.prompt_hashes, keep)
        if pool_pages is None:
            pool_pages = [self.pools[l].pool_pages for l in range(L)]
        pools = (_abi.cb_layer_pool * max(L, 1))()
        for l in range(L):
            f = _i32(free_pages[l])
            keep.append(f)
            pools[l] = _abi.cb_layer_pool(self.rings[l], self.windows[l], int(pool_pages[l]), f.size, _ptr(f))
        self.reqs, self.pools, self._keep = reqs, pools, keep
        # page lists written by advance_step: [n][L][stride], grown (and the requests' pages moved) when a step needs
        # more pages per request than it holds
        self._store_stride = max([1] + [int(reqs[i].n_pages[l]) for i in range(n) for l in range(L)])
        self._store = np.zeros(max(n, 1) * L * self._store_stride, dtype=np.int32)

    @property
    def requests(self):
        """The request records (arrival order) as the scheduler's state holds them now."""
        self._sync()
        return self._requests

    @property
    def free_pages(self):
        """Each layer type's free list (allocation order) as the scheduler's state holds it now."""
        self._sync()
        return self._free_pages

    def _sync(self) -> None:
        if not self._stale:
            return
        self._requests = _unmarshal_requests(self._requests, self.reqs, self.L)
        self._free_pages = [np.ctypeslib.as_array(p.free_pages, shape=(p.n_free,)).copy() if p.n_free > 0
                            else np.zeros(0, np.int32) for p in self.pools[:self.L]]
        self._stale = False

    def _grow_store(self, stride: int) -> None:
        """A page store of `stride` pages per request and layer; requests whose pages live in the old one move."""
        L = self.L
        old = self._store
        new = np.zeros(max(self.n, 1) * L * stride, dtype=np.int32)
        base, end = old.ctypes.data, old.ctypes.data + old.nbytes
        for i in range(self.n):
            r = self.reqs[i]
            for l in range(L):
                addr = C.cast(r.pages[l], C.c_void_p).value or 0
                if base <= addr < end:
                    k = r.n_pages[l]
                    src = (addr - base) // 4
                    dst = (i * L + l) * stride
                    new[dst:dst + k] = old[src:src + k]
                    r.pages[l] = C.cast(C.c_void_p(new.ctypes.data + 4 * dst), _abi.i32p)
        self._keep.append(old)     # kept alive until the next set_state
        self._store, self._store_stride = new, stride

    def advance_step(self, step: _abi.cb_step, buf: np.ndarray) -> None:
        """After the step that build_into scheduled into `buf` (header `step`) has run: the request lifecycle
        (cb_advance) on the scheduler's marshalled requests and free lists, in place, with no per-request Python
        work; the `requests` / `free_pages` views catch up when read."""
        need = _store_stride(step, self.rings, self.page_size)
        if need > self._store_stride:
            self._grow_store(max(need, 2 * self._store_stride))
        st = self._lib.cb_advance(self.reqs, self.n, C.byref(self.params), self.pools, buf.ctypes.data_as(_abi.i32p),
                                  C.byref(step), _ptr(self._store), self._store_stride)
        if st != CB_OK:
            raise CbError(st, "cb_advance")
        self._stale = True

    def advance(self, schedule: dict) -> None:
        """After the step `schedule` (numpy form, e.g. schedule_arrays) has run: move every request along its
        lifecycle (`advance`) and drop the pages the step took from the free lists. advance_step does the same on
        the raw metadata buffer without leaving native code."""
        reqs, free = advance(self.requests, schedule, self.free_pages, self.rings, self.page_size, self.prefix_cache,
                             self.prompt_hashes)
        self.set_state(reqs, free)

    def build_step_into(self, out_addr: int, meta_capacity: int, out_capacity: int, shapes, step: _abi.cb_step,
                        plans, plan_offsets) -> None:
        """cb_build_step: schedule into the int32 buffer at address out_addr and plan every layer (shapes: a ctypes
        array of cb_attn_shape) into the same buffer after meta_capacity; fills `step`, `plans` (ctypes array of
        cb_plan) and `plan_offsets` (ctypes array of int64, from meta_capacity). Raises on any status but OK."""
        st = self._lib.cb_build_step(self.reqs, self.n, C.byref(self.params), self.pools, shapes, out_addr,
                                     meta_capacity, out_capacity, C.byref(step), plans, plan_offsets)
        if st != CB_OK:
            raise CbError(st, "cb_build_step")

    def build_into(self, out: np.ndarray) -> _abi.cb_step:
        """Schedule into `out` (a C-contiguous int32 array); returns the header. Raises on any status but OK."""
        step = _abi.cb_step()
        st = self._lib.cb_build_metadata(self.reqs, self.n, C.byref(self.params), self.pools,
                                         out.ctypes.data_as(_abi.i32p), out.size, C.byref(step))
        if st != CB_OK:
            raise CbError(st, "cb_build_metadata")
        return step


def plan_into(query_start_loc: np.ndarray, seq_lens: np.ndarray, ring_len, shape: _abi.cb_attn_shape,
              out: np.ndarray) -> AttnPlan:
    """cb_plan_attention writing into `out` (C-contiguous int32 array); returns the plan with `buffer` = its view."""
    info = _abi.cb_plan()
    n = seq_lens.size
    st = _abi.load().cb_plan_attention(_ptr(query_start_loc), _ptr(seq_lens), None if ring_len is None else
                                       _ptr(ring_len), n, C.byref(shape), out.ctypes.data_as(_abi.i32p), out.size,
                                       C.byref(info))
    if st != CB_OK:
        raise CbError(st, "cb_plan_attention")
    return AttnPlan(info, shape, out[:int(info.used)])


# ------------------------------------------------------------------------------------------- cb_plan_attention

@dataclass
class AttnPlan:
    info: _abi.cb_plan
    shape: _abi.cb_attn_shape
    buffer: np.ndarray          # host int32 plan

    def counts(self) -> dict:
        i = self.info
        return {"decode": i.n_decode, "prefill": i.n_prefill, "rowwise": i.n_rowwise, "combine": i.n_combine,
                "partials": i.n_partials, "decode_split": i.decode_split, "prefill_split": i.prefill_split,
                "prefill_tokens": i.prefill_tokens}

    def items(self, kind: str) -> np.ndarray:
        i = self.info
        n, off, w = {"decode": (i.n_decode, i.off_decode, 8), "prefill": (i.n_prefill, i.off_prefill, 8),
                     "rowwise": (i.n_rowwise, i.off_rowwise, 8), "combine": (i.n_combine, i.off_combine, 4)}[kind]
        return self.buffer[off:off + n * w].reshape(n, w)


def _dtype_code(dtype) -> int:
    import torch
    if dtype in (torch.float32, "f32", "float32"):
        return CB_DTYPE_F32
    if dtype in (torch.bfloat16, "bf16", "bfloat16"):
        return CB_DTYPE_BF16
    raise ValueError(f"unsupported dtype {dtype}")


def plan_attention(query_start_loc, seq_lens, ring_len, num_q_heads: int, num_kv_heads: int, head_dim: int,
                   page_size: int, dtype, window_left: int = -1, decode_split: int = 0,
                   prefill_split: int = 0, prefill_rows: int = 0) -> AttnPlan:
    """Split a step into kernel work items (cb_plan_attention). ring_len: per-row ring lengths or None.
    prefill_rows: query rows per prefill work group, 128 or 256, or 0 for the planner's choice."""
    lib = _abi.load()
    qsl = _i32(query_start_loc)
    seq = _i32(seq_lens)
    n = seq.size
    rl = None if ring_len is None else _i32(ring_len)
    shape = _abi.cb_attn_shape(int(num_q_heads), int(num_kv_heads), int(head_dim), int(page_size),
                               _dtype_code(dtype), int(window_left), int(decode_split), int(prefill_split),
                               int(prefill_rows))
    info = _abi.cb_plan()
    cap = 1024
    while True:
        buf = np.zeros(cap, dtype=np.int32)
        st = lib.cb_plan_attention(_ptr(qsl), _ptr(seq), None if rl is None else _ptr(rl), n, C.byref(shape),
                                   _ptr(buf), cap, C.byref(info))
        if st != CB_E_CAPACITY:
            break
        cap = int(info.used)
    if st != CB_OK:
        raise CbError(st, "cb_plan_attention")
    return AttnPlan(info, shape, buf[:int(info.used)].copy())


# ------------------------------------------------------------------------------------------------ device calls

def _stream(stream):
    import torch
    if stream is None:
        return C.c_void_p(torch.cuda.current_stream().cuda_stream)
    return C.c_void_p(getattr(stream, "cuda_stream", stream))


def _check_dev(t, name):
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")


def kv_append(k_cache, v_cache, k_new, v_new, slot_mapping, stream=None) -> None:
    """cb_kv_append: k_cache [pages, Hkv, P, D], v_cache [pages, Hkv, D, P], k_new/v_new [T, Hkv, D], slot_mapping
    [T] int32 (device tensors)."""
    lib = _abi.load()
    for t, nm in ((k_cache, "k_cache"), (v_cache, "v_cache"), (k_new, "k_new"), (v_new, "v_new"),
                  (slot_mapping, "slot_mapping")):
        _check_dev(t, nm)
    n_pages, Hkv, P, D = k_cache.shape
    if tuple(v_cache.shape) != (n_pages, Hkv, D, P) or k_new.shape[1:] != (Hkv, D) or v_new.shape != k_new.shape:
        raise ValueError("cache / new-row shapes do not match")
    if slot_mapping.numel() != k_new.shape[0] or str(slot_mapping.dtype) != "torch.int32":
        raise ValueError("slot_mapping must be int32 [T]")
    if not (k_cache.dtype == v_cache.dtype == k_new.dtype == v_new.dtype):
        raise ValueError("dtype mismatch")
    st = lib.cb_kv_append(k_cache.data_ptr(), v_cache.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
                          slot_mapping.data_ptr(), k_new.shape[0], n_pages, P, Hkv, D, _dtype_code(k_cache.dtype),
                          CB_LAYOUT_KD_VT, _stream(stream))
    if st != CB_OK:
        raise CbError(st, "cb_kv_append")


def copy_pages(dst, src, dst_pages=None, src_pages=None, stream=None) -> None:
    """cb_kv_copy_pages: page i of the copy goes from src[src_pages[i]] to dst[dst_pages[i]] (None: page i).
    dst, src: contiguous device tensors whose first dimension counts pages (a cache tensor, or a swap buffer of
    the same page shape); dst_pages / src_pages: int32 device tensors of equal length, or None."""
    lib = _abi.load()
    for t, nm in ((dst, "dst"), (src, "src")):
        _check_dev(t, nm)
    if tuple(dst.shape[1:]) != tuple(src.shape[1:]) or dst.dtype != src.dtype:
        raise ValueError("dst and src must hold pages of the same shape and dtype")
    lists = [x for x in (dst_pages, src_pages) if x is not None]
    for x in lists:
        _check_dev(x, "page list")
        if str(x.dtype) != "torch.int32":
            raise ValueError("page lists must be int32")
    if len({x.numel() for x in lists}) > 1:
        raise ValueError("page lists differ in length")
    n = lists[0].numel() if lists else min(dst.shape[0], src.shape[0])
    page_bytes = (dst[0].numel() if dst.shape[0] else src[0].numel()) * dst.element_size()
    st = lib.cb_kv_copy_pages(dst.data_ptr(), dst_pages.data_ptr() if dst_pages is not None else None, dst.shape[0],
                              src.data_ptr(), src_pages.data_ptr() if src_pages is not None else None, src.shape[0],
                              n, page_bytes, _stream(stream))
    if st != CB_OK:
        raise CbError(st, "cb_kv_copy_pages")


# ------------------------------------------------------------------------------------------------ prefix cache

def block_hashes(tokens, page_size: int) -> np.ndarray:
    """cb_block_hashes: chain hashes (uint64) of the full blocks of a token sequence."""
    t = _i32(tokens)
    out = np.zeros(max(t.size // page_size, 1), dtype=np.uint64)
    st = _abi.load().cb_block_hashes(_ptr(t), t.size, int(page_size), out.ctypes.data_as(C.POINTER(C.c_uint64)))
    if st != CB_OK:
        raise CbError(st, "cb_block_hashes")
    return out[:t.size // page_size]


class PrefixCache:
    """The library's prefix cache (cb_pcache_*): page sharing by block hash with reference counts and lazy
    demotion of freed blocks. Page lists in and out are int32 numpy arrays."""

    def __init__(self, num_pages: int, free_pages):
        self._lib = _abi.load()
        f = _i32(free_pages)
        h = C.c_void_p()
        st = self._lib.cb_pcache_create(int(num_pages), _ptr(f), f.size, C.byref(h))
        if st != CB_OK:
            raise CbError(st, "cb_pcache_create")
        self._h = h

    def __del__(self):
        if getattr(self, "_h", None) and self._h.value:
            self._lib.cb_pcache_destroy(self._h)
            self._h = None

    def _call(self, st, what):
        if st != CB_OK:
            raise CbError(st, what)

    def match(self, hashes) -> np.ndarray:
        hs = np.ascontiguousarray(np.asarray(hashes, dtype=np.uint64))
        out = np.zeros(max(hs.size, 1), dtype=np.int32)
        n = C.c_int32()
        self._call(self._lib.cb_pcache_match(self._h, hs.ctypes.data_as(C.POINTER(C.c_uint64)), hs.size, _ptr(out),
                                             C.byref(n)), "cb_pcache_match")
        return out[:n.value].copy()

    def lookup(self, hashes):
        """Pages of the leading registered blocks (no references taken) and how many of them are free."""
        hs = np.ascontiguousarray(np.asarray(hashes, dtype=np.uint64))
        out = np.zeros(max(hs.size, 1), dtype=np.int32)
        n, nf = C.c_int32(), C.c_int32()
        self._call(self._lib.cb_pcache_lookup(self._h, hs.ctypes.data_as(C.POINTER(C.c_uint64)), hs.size, _ptr(out),
                                              C.byref(n), C.byref(nf)), "cb_pcache_lookup")
        return out[:n.value].copy(), nf.value

    def allocate(self, n: int) -> np.ndarray:
        out = np.zeros(max(n, 1), dtype=np.int32)
        self._call(self._lib.cb_pcache_allocate(self._h, int(n), _ptr(out)), "cb_pcache_allocate")
        return out[:n].copy()

    def commit(self, page: int, h) -> None:
        self._call(self._lib.cb_pcache_commit(self._h, int(page), int(h)), "cb_pcache_commit")

    def release(self, pages) -> None:
        p = _i32(pages)
        self._call(self._lib.cb_pcache_release(self._h, _ptr(p), p.size), "cb_pcache_release")

    def stats(self):
        a, b, c = C.c_int32(), C.c_int32(), C.c_int32()
        self._call(self._lib.cb_pcache_stats(self._h, C.byref(a), C.byref(b), C.byref(c)), "cb_pcache_stats")
        return a.value, b.value, c.value

    def page_info(self, page: int):
        r, reg, h = C.c_int32(), C.c_int32(), C.c_uint64()
        self._call(self._lib.cb_pcache_page_info(self._h, int(page), C.byref(r), C.byref(reg), C.byref(h)),
                   "cb_pcache_page_info")
        return r.value, bool(reg.value), h.value


def _args(out, q, k_cache, v_cache, block_table, plan: AttnPlan, plan_dev, scale, workspace, phases=0):
    a = _abi.cb_attn_args()
    a.out, a.q = out.data_ptr(), q.data_ptr()
    a.k_cache, a.v_cache = k_cache.data_ptr(), v_cache.data_ptr()
    a.layout = CB_LAYOUT_KD_VT
    a.block_table = block_table.data_ptr()
    a.plan = plan_dev.data_ptr()
    a.plan_info = plan.info
    a.shape = plan.shape
    a.num_pages = k_cache.shape[0]
    a.table_width = block_table.shape[1] if block_table.dim() == 2 else 0
    a.scale = float(scale)
    a.workspace = workspace.data_ptr() if workspace is not None else None
    a.workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    a.phases = int(phases)
    return a


def check_dtypes(plan: AttnPlan, **tensors) -> None:
    """Raise ValueError unless every given tensor has the element type the plan was made for. The C ABI sees only
    pointers, so this is the one place a bf16 plan paired with fp32 tensors (or the reverse) is caught before a
    kernel would index them with the wrong element size."""
    want = plan.shape.dtype
    for name, t in tensors.items():
        if t is None:
            continue
        if _dtype_code(t.dtype) != want:
            raise ValueError(f"{name} has dtype {t.dtype}, the plan's dtype code is {want}")


def workspace_size(plan: AttnPlan) -> int:
    a = _abi.cb_attn_args()
    a.plan_info = plan.info
    a.shape = plan.shape
    return int(_abi.load().cb_paged_attention_workspace_size(C.byref(a)))


def paged_attention(out, q, k_cache, v_cache, block_table, plan: AttnPlan, plan_dev, scale: float,
                    workspace=None, stream=None, phases: int = 0, k_new=None, v_new=None, slot_mapping=None) -> None:
    """cb_paged_attention: out/q [T, Hq, D]; caches as in kv_append; block_table [N, width] int32; plan_dev = the
    plan's int32 buffer on the device; workspace: a device byte tensor of at least workspace_size(plan) bytes;
    phases: 0 for the whole step, or a mask of CB_PHASE_* to launch only some of its kernels.
    k_new, v_new [T, Hkv, D] and slot_mapping [T] int32 (all or none): the fused append, which writes the step's new
    K/V into the caches in the same launches (the caller then skips kv_append for the step)."""
    lib = _abi.load()
    for t, nm in ((out, "out"), (q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"),
                  (block_table, "block_table"), (plan_dev, "plan")):
        _check_dev(t, nm)
    sh = plan.shape
    if tuple(q.shape) != (plan.info.num_tokens, sh.num_q_heads, sh.head_dim) or out.shape != q.shape:
        raise ValueError("q/out shape does not match the plan")
    if tuple(k_cache.shape[1:]) != (sh.num_kv_heads, sh.page_size, sh.head_dim):
        raise ValueError("k_cache shape does not match the plan")
    if tuple(v_cache.shape) != (k_cache.shape[0], sh.num_kv_heads, sh.head_dim, sh.page_size):
        raise ValueError("v_cache shape does not match the plan")
    if plan_dev.numel() < plan.buffer.size or str(plan_dev.dtype) != "torch.int32":
        raise ValueError("plan_dev must hold the plan's int32 buffer")
    check_dtypes(plan, q=q, out=out, k_cache=k_cache, v_cache=v_cache)
    if str(block_table.dtype) != "torch.int32":
        raise ValueError("block_table must be int32")
    a = _args(out, q, k_cache, v_cache, block_table, plan, plan_dev, scale, workspace, phases)
    if k_new is not None:
        for t, nm in ((k_new, "k_new"), (v_new, "v_new"), (slot_mapping, "slot_mapping")):
            _check_dev(t, nm)
        if tuple(k_new.shape) != (plan.info.num_tokens, sh.num_kv_heads, sh.head_dim) or v_new.shape != k_new.shape:
            raise ValueError("k_new / v_new shape does not match the plan")
        if slot_mapping.numel() != k_new.shape[0] or str(slot_mapping.dtype) != "torch.int32":
            raise ValueError("slot_mapping must be int32 [T]")
        check_dtypes(plan, k_new=k_new, v_new=v_new)
        a.k_new, a.v_new, a.slot_mapping = k_new.data_ptr(), v_new.data_ptr(), slot_mapping.data_ptr()
        a.num_new = k_new.shape[0]
    elif v_new is not None or slot_mapping is not None:
        raise ValueError("k_new, v_new and slot_mapping go together")
    st = lib.cb_paged_attention(C.byref(a), _stream(stream))
    if st != CB_OK:
        raise CbError(st, "cb_paged_attention")
