"""Plain Python reference of the step's host metadata (FIFO fill, page allocation, ragged metadata).

Test infrastructure only: the product never imports it; it shares no code with the C++ scheduler it checks.

Rules followed (Transformers "continuous batching architecture" page, sections "调度器"/"FIFO"/"准入"/"内存管理";
"Continuous Batching" blog, languisher.top, sections "扩展：vLLM v1 中的实现" and "扩展：与 Chunked Prefill 结合"):

* A forward pass takes at most `max_batch_tokens` query tokens and `max_requests` requests.
* FIFO order: first the active decodes (one token each), then the active prefills (continuing chunks), then the
  waiting requests in arrival order. A prompt longer than the budget left is cut; the rest waits for the next step.
* Admission of a waiting request is all-or-nothing across the layer types: if any allocator lacks the pages, nothing
  is allocated and the request is rejected. Reading: admission stops at the first rejection (no skipping ahead).
* While the free fraction of any pool is below `safety_margin`, new prefills are held (decodes continue).
* Reading for active requests that need pages no pool can give: they are reported stalled and left out of the step.
* Pages come from the front of each layer's free list. Full layers add pages as the sequence grows; a sliding layer
  gives each request a fixed ring of `ring_len` pages at admission.
* Metadata: query_start_loc [N+1] (exclusive prefix sum of the query lengths plus the total), seq_lens [N]
  (context + this step's tokens), block_table [N, width] padded with the padding page, slot_mapping [T].
* After a step (`advance`, same page, section "请求生命周期"): each scheduled request's context is its seq_len, a
  finished prompt turns to decoding, its pages are its block-table row, the free lists lose the step's pages.
"""
from __future__ import annotations

import numpy as np

DECODING, PREFILLING, WAITING = 0, 1, 2
OK, E_INVAL, E_NOSPACE = "ok", "inval", "nospace"


def _cdiv(a, b):
    return -(-a // b)


def ring_is_large_enough(ring_len, window_left, max_chunk, page_size):
    """A ring must hold every key still visible to this step's queries plus the keys the step appends.

    Queries at ctx..ctx+q-1 see back to ctx-window_left, so window_left+q consecutive positions must map to distinct
    ring slots; with arbitrary alignment they span at most (window_left+q+page_size-2)//page_size + 1 pages.
    """
    return ring_len >= (window_left + max_chunk + page_size - 2) // page_size + 1


FIFO, PREFILL_FIRST = "fifo", "prefill_first"


def build_metadata(requests, layers, max_batch_tokens, max_requests, page_size, safety_margin=0.0, pad_page=0,
                   policy=FIFO, prefix_cache=None, prompt_hashes=None):
    """Schedule one step.

    requests: sequence with .state, .num_computed, .num_pending, .pages (list per layer), in arrival order.
    layers: sequence of dicts {ring_len, window_left, pool_pages, free_pages}.
    policy: FIFO fills the budget with active decodes, then active prefills, then waiting requests (Transformers
    "continuous batching architecture" page, section "FIFO"); PREFILL_FIRST finishes prefill work before decodes
    resume (section "PrefillFirst"). Reading taken: active prefills, then waiting requests, then decodes with what
    is left of the budget; pages are taken from the free lists in that order. Either way the rows are laid out
    decodes first, then continuing prefills, then admitted requests, each group in scheduling order.
    Returns a dict (see module docstring); "status" is "ok", "inval" or "nospace".

    prefix_cache (an oracle.prefix_cache.PrefixCache over the pool's pages) turns on prefix sharing at admission
    (same page, sections "前缀缓存" and "准入"). Sharing is on only when every layer can share, i.e. every layer is a
    full-attention layer (the page: sliding-window and hybrid models disable it); with a ring layer the cache is
    ignored. Readings taken, with sharing on:
      * one layer type (the cache manages one pool); every page the step takes comes from the cache's allocator
        (its empty pages, then demoted initialized ones), not from the layer's free list;
      * a waiting request whose prompt has not started (num_computed 0, no pages) first looks up the leading blocks of its
        prompt, prompt_hashes[i] (chain hashes of its full prompt blocks); at most (num_pending - 1) // page_size
        of them count, so that the step still computes at least one prompt token (the one whose output starts the
        generation); their pages become its first pages and its context starts at matched * page_size;
      * admission stays all-or-nothing: the match is taken only if the fresh pages for the rest of the chunk can be
        allocated too, counting matched pages that sat free in the cache as leaving the free pool;
      * the safety margin and every availability check use the cache's free pages.
    The returned dict then also holds "matched_tokens" [N] (context reused from the cache per row).
    """
    if policy not in (FIFO, PREFILL_FIRST):
        return {"status": E_INVAL}
    P = page_size
    L = len(layers)
    if P < 1 or max_batch_tokens < 1 or max_requests < 1 or L < 1:
        return {"status": E_INVAL}
    for lay in layers:
        if lay["ring_len"] > 0:
            if lay["window_left"] < 0 or not ring_is_large_enough(lay["ring_len"], lay["window_left"],
                                                                   max_batch_tokens, P):
                return {"status": E_INVAL}
    for rq in requests:
        if rq.num_computed < 0 or rq.num_pending < 1 or rq.state not in (DECODING, PREFILLING, WAITING):
            return {"status": E_INVAL}
        if rq.state == DECODING and rq.num_pending != 1:
            return {"status": E_INVAL}
        for l, lay in enumerate(layers):
            owned = len(rq.pages[l])
            if lay["ring_len"] > 0:
                if rq.state != WAITING and owned != lay["ring_len"]:
                    return {"status": E_INVAL}
            elif owned < _cdiv(rq.num_computed, P):
                return {"status": E_INVAL}

    free = [np.asarray(lay["free_pages"], dtype=np.int32) for lay in layers]
    taken = [0] * L
    sharing = prefix_cache is not None and L == 1 and all(lay["ring_len"] == 0 for lay in layers)
    pc = prefix_cache if sharing else None

    def needs(rq, q):
        out = []
        for l, lay in enumerate(layers):
            have = len(rq.pages[l])
            if lay["ring_len"] > 0:
                out.append(max(0, lay["ring_len"] - have))
            else:
                out.append(max(0, _cdiv(rq.num_computed + q, P) - have))
        return out

    def n_free(l):
        return pc.n_free() if pc is not None else len(free[l]) - taken[l]

    def fits(nd):
        return all(nd[l] <= n_free(l) for l in range(L))

    def take(nd):
        got = []
        for l in range(L):
            if pc is not None:
                got.append(np.array(pc.allocate(nd[l]), dtype=np.int32))
            else:
                got.append(free[l][taken[l]:taken[l] + nd[l]].copy())
            taken[l] += nd[l]
        return got

    rows = {DECODING: [], PREFILLING: [], WAITING: []}   # (request index, q_len, new pages per layer, matched)
    stalled = []
    first_rejected = -1
    held = False
    budget = max_batch_tokens

    def n_rows():
        return sum(len(v) for v in rows.values())

    def decodes():
        """active decodes, one token each"""
        nonlocal budget
        for i, rq in enumerate(requests):
            if rq.state != DECODING:
                continue
            if n_rows() >= max_requests or budget < 1:
                break
            nd = needs(rq, 1)
            if not fits(nd):
                stalled.append(i)
                continue
            rows[DECODING].append((i, 1, take(nd), 0))
            budget -= 1

    def prefills():
        """active prefills, continuing where they stopped"""
        nonlocal budget
        for i, rq in enumerate(requests):
            if rq.state != PREFILLING:
                continue
            if n_rows() >= max_requests or budget < 1:
                break
            q = min(rq.num_pending, budget)
            nd = needs(rq, q)
            if not fits(nd):
                stalled.append(i)
                continue
            rows[PREFILLING].append((i, q, take(nd), 0))
            budget -= q

    def admit():
        """waiting requests in arrival order (admission)"""
        nonlocal budget, held, first_rejected
        for i, rq in enumerate(requests):
            if rq.state != WAITING:
                continue
            if n_rows() >= max_requests or budget < 1:
                break
            if any(lay["pool_pages"] > 0 and n_free(l) < safety_margin * lay["pool_pages"]
                   for l, lay in enumerate(layers)):
                held = True
                break
            hit = []
            if pc is not None and rq.num_computed == 0 and len(rq.pages[0]) == 0 and prompt_hashes is not None:
                cap = (rq.num_pending - 1) // P
                hit = pc.lookup(list(prompt_hashes[i])[:cap])
            m = len(hit) * P
            q = min(rq.num_pending - m, budget)
            if hit:
                # the matched pages are the request's first pages; matched pages that sit free in the cache leave
                # its free pool when matched
                nd = [max(0, _cdiv(m + q, P) - len(hit))]
                leaving = sum(1 for p_ in hit if pc.ref[p_] == 0)
                ok = nd[0] <= n_free(0) - leaving
            else:
                nd = needs(rq, q)
                ok = fits(nd)
            if not ok:
                first_rejected = i
                break
            if hit:
                got = np.array(pc.match(list(prompt_hashes[i])[:len(hit)]), dtype=np.int32)
                rows[WAITING].append((i, q, [np.concatenate([got, take(nd)[0]])], m))
            else:
                rows[WAITING].append((i, q, take(nd), 0))
            budget -= q

    for stage in ((decodes, prefills, admit) if policy == FIFO else (prefills, admit, decodes)):
        stage()
    stalled.sort()
    num_decodes = len(rows[DECODING])
    rows = rows[DECODING] + rows[PREFILLING] + rows[WAITING]

    N = len(rows)
    q_lens = np.array([q for _, q, _, _ in rows], dtype=np.int64)
    qsl = np.zeros(N + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(q_lens)
    T = int(qsl[-1])
    seq_lens = np.array([requests[i].num_computed + m + q for i, q, _, m in rows], dtype=np.int32)
    req_index = np.array([i for i, _, _, _ in rows], dtype=np.int32)

    out = {"status": OK, "query_start_loc": qsl, "seq_lens": seq_lens, "req_index": req_index,
           "num_reqs": N, "num_tokens": T, "num_decodes": num_decodes, "stalled": np.array(stalled, np.int32),
           "first_rejected": first_rejected, "held_by_margin": held, "layers": [],
           "prefix_sharing": sharing, "matched_tokens": np.array([m for _, _, _, m in rows], dtype=np.int32)}
    if N == 0 and (stalled or first_rejected >= 0):
        out["status"] = E_NOSPACE

    for l, lay in enumerate(layers):
        R = lay["ring_len"]
        if R > 0:
            width = R
        else:
            width = max((_cdiv(int(s), P) for s in seq_lens), default=0)
        table = np.full((N, width), pad_page, dtype=np.int32)
        slots = np.zeros(T, dtype=np.int32)
        for r, (i, q, new, m) in enumerate(rows):
            rq = requests[i]
            pages = np.concatenate([np.asarray(rq.pages[l], dtype=np.int32), new[l]]).astype(np.int32)
            if R > 0:
                table[r, :] = pages[:R]
            else:
                n = _cdiv(int(seq_lens[r]), P)
                table[r, :n] = pages[:n]
            for j in range(q):
                pos = rq.num_computed + m + j
                blk, off = pos // P, pos % P
                phys = table[r, blk % R] if R > 0 else table[r, blk]
                slots[qsl[r] + j] = phys * P + off
        out["layers"].append({"block_table": table, "slot_mapping": slots,
                              "ring_len": np.full(N, R, dtype=np.int32), "used_pages": taken[l], "width": width})
    return out


def advance(requests, schedule, free_pages, page_size, prefix_cache=None, prompt_hashes=None):
    """The request lifecycle after a step has run (Transformers "continuous batching architecture" page, section
    "请求生命周期"): a waiting request is admitted and prefilled chunk by chunk; once its whole prompt is in the
    cache it decodes, one token per step.

    Readings: after the step, request i = req_index[r] holds every key up to seq_lens[r], so its context becomes
    seq_lens[r] and its pending prompt shrinks by the keys gained (this step's tokens plus any prompt blocks it
    reused from the prefix cache); with nothing left it turns to decoding, with one pending token (the one just
    produced). Its pages are what its block-table row addresses: ceil(seq_len / page_size) pages, or its whole ring.
    The step's pages came off the front of each free list, unless the step shared prefixes: then they came from the
    prefix cache, which registers (commit) each prompt block the step filled completely. Unscheduled requests keep
    their state. Returns (requests, free_pages) as new lists; the input is not modified."""
    import copy
    P = page_size
    out = [copy.copy(rq) for rq in requests]
    for rq in out:
        rq.pages = [np.asarray(p, dtype=np.int32).copy() for p in rq.pages]
    shared = bool(schedule.get("prefix_sharing", False))
    qsl, seqs = schedule["query_start_loc"], schedule["seq_lens"]
    for r, i in enumerate(schedule["req_index"]):
        rq = out[int(i)]
        seq = int(seqs[r])
        context = seq - int(qsl[r + 1] - qsl[r])
        if shared and prefix_cache is not None and prompt_hashes is not None and prompt_hashes[int(i)] is not None:
            hashes = prompt_hashes[int(i)]
            row = schedule["layers"][0]["block_table"][r]
            for blk in range(context // P, min(seq // P, len(hashes))):   # blocks this step completed
                prefix_cache.commit(int(row[blk]), int(hashes[blk]))
        gained = seq - rq.num_computed
        rq.num_computed = seq
        rq.num_pending = rq.num_pending - gained
        if rq.num_pending > 0:
            rq.state = PREFILLING
        else:
            rq.state, rq.num_pending = DECODING, 1
        for l, lay in enumerate(schedule["layers"]):
            ring = int(lay["ring_len"][r])
            keep = ring if ring > 0 else _cdiv(seq, P)
            rq.pages[l] = np.array(lay["block_table"][r][:keep], dtype=np.int32)
    free = []
    for l, lay in enumerate(schedule["layers"]):
        taken = 0 if shared else int(lay["used_pages"])
        free.append(np.asarray(free_pages[l], dtype=np.int32)[taken:].copy())
    return out, free
