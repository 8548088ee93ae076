"""Workload-level oracle: the expected metadata, attention rows and cache pages of one synthetic step.

Test infrastructure only. Inputs come from the seeded generator in `synth`; nothing here reads a value produced by
the HIP path.

Harness convention shared with the GPU side (input setup, not part of the method): before the step, every cache page
holds NaN; then each admitted request's history is written -- full layers: positions 0 .. context-1; sliding layers:
only the positions a query of this step can still see, max(0, context - window_left) .. context-1. The step's own new
tokens are then appended through the scheduler's slot_mapping.
"""
from __future__ import annotations

import numpy as np

from . import attention as A
from . import scheduler as S


def schedule(w):
    """Run the reference scheduler over a synthetic workload."""
    layers = [{"ring_len": l.ring_len, "window_left": l.window_left,
               "pool_pages": l.num_pages - len(l.padding_pages), "free_pages": l.free_pages} for l in w.layers]
    pad = w.layers[0].padding_pages[0] if w.layers[0].padding_pages else 0
    return S.build_metadata(w.requests, layers, w.max_batch_tokens, w.max_requests, w.page_size,
                            w.safety_margin, pad, policy=w.policy)


def history_range(w, layer: int, ctx: int):
    """Positions of one request's history that the harness writes before the step (see module docstring)."""
    wl = w.layers[layer].window_left
    return (0 if wl < 0 else max(0, ctx - wl)), ctx


def rows_reference(w, layer: int, sched, tokens=None):
    """fp64 expected output rows of `layer` for the scheduled step.

    tokens: iterable of global token indices (rows of the ragged batch) to compute, or None for all.
    Returns {token: array [Hq, D]}. Keys come straight from the request's logical (contiguous) sequence: history
    positions then this step's new tokens -- the definition, with no paging involved.
    """
    qsl = sched["query_start_loc"]
    seq = sched["seq_lens"]
    idx = sched["req_index"]
    wl = w.layers[layer].window_left
    want = None if tokens is None else sorted(set(int(t) for t in tokens))
    out = {}
    for r in range(sched["num_reqs"]):
        qs, qe = int(qsl[r]), int(qsl[r + 1])
        if want is None:
            local = list(range(qe - qs))
        else:
            local = [t - qs for t in want if qs <= t < qe]
        if not local:
            continue
        q_len = qe - qs
        ctx = int(seq[r]) - q_len
        i = int(idx[r])
        positions = [ctx + j for j in local]
        lo = A.visible_range(positions[0], wl)[0]
        top = positions[-1]
        k = w.values("k", i, layer, lo, top + 1)
        v = w.values("v", i, layer, lo, top + 1)
        q = np.concatenate([w.values("q", i, layer, p, p + 1) for p in positions]) if len(local) < q_len else \
            w.values("q", i, layer, ctx, ctx + q_len)
        res = A.attend_rows(q, k, v, lo, positions, w.scale, wl)
        for n, j in enumerate(local):
            out[qs + j] = res[n]
    return out


def step_inputs(w, layer: int, sched):
    """Ragged new-token tensors of the step: q [T, Hq, D], k/v [T, Hkv, D] (float32, dtype-exact)."""
    qsl = sched["query_start_loc"]
    seq = sched["seq_lens"]
    idx = sched["req_index"]
    T = sched["num_tokens"]
    q = np.zeros((T, w.Hq, w.D), np.float32)
    k = np.zeros((T, w.Hkv, w.D), np.float32)
    v = np.zeros((T, w.Hkv, w.D), np.float32)
    for r in range(sched["num_reqs"]):
        qs, qe = int(qsl[r]), int(qsl[r + 1])
        ctx = int(seq[r]) - (qe - qs)
        i = int(idx[r])
        q[qs:qe] = w.values("q", i, layer, ctx, ctx + qe - qs)
        k[qs:qe] = w.values("k", i, layer, ctx, ctx + qe - qs)
        v[qs:qe] = w.values("v", i, layer, ctx, ctx + qe - qs)
    return q, k, v


def pages_reference(w, layer: int, sched, pages=None):
    """Expected cache contents after history fill + the step's append, as logical [page, offset, Hkv, D] float32.

    pages: iterable of physical page ids to build (None: the whole pool). Returns (page_ids, k, v) with NaN wherever
    nothing was written. Uses the oracle's own slot rule for the history and the oracle scheduler's slot_mapping
    for the new tokens.
    """
    lay = w.layers[layer]
    P = w.page_size
    ids = np.arange(lay.num_pages) if pages is None else np.array(sorted(set(int(p) for p in pages)))
    where = {int(p): n for n, p in enumerate(ids)}
    k = np.full((len(ids), P, w.Hkv, w.D), np.nan, np.float32)
    v = np.full((len(ids), P, w.Hkv, w.D), np.nan, np.float32)

    def put(slot, kr, vr):
        page, off = slot // P, slot % P
        n = where.get(page)
        if n is not None:
            k[n, off] = kr
            v[n, off] = vr

    # history of every admitted request (scheduled or not): walk its logical blocks, keep those whose physical page
    # was asked for, and write their positions in order
    for i, rq in enumerate(w.requests):
        if len(rq.pages[layer]) == 0 or rq.num_computed == 0:
            continue
        a, b = history_range(w, layer, rq.num_computed)
        for blk in range(a // P, (b - 1) // P + 1 if b > a else a // P):
            if A.physical_page(rq.pages[layer], blk, lay.ring_len) not in where:
                continue
            s, e = max(a, blk * P), min(b, (blk + 1) * P)
            kh = w.values("k", i, layer, s, e)
            vh = w.values("v", i, layer, s, e)
            for n, pos in enumerate(range(s, e)):
                put(A.slot_of(rq.pages[layer], pos, P, lay.ring_len), kh[n], vh[n])
    # the step's append
    _, kn, vn = step_inputs(w, layer, sched)
    for t, slot in enumerate(sched["layers"][layer]["slot_mapping"]):
        if slot >= 0:
            put(int(slot), kn[t], vn[t])
    return ids, k, v
