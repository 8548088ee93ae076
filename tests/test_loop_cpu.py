"""The request lifecycle across steps (advance): hand-worked cases, and a multi-step run whose every step's
metadata equals the oracle scheduler's on the same request state."""
import dataclasses

import numpy as np

import paged_kv_attention_varlen_amd as cb
from harness import sched_pools
from oracle import scheduler as OS
from synth import DECODING, PREFILLING, WAITING, make_workload


def _schedule(reqs, pools, budget, P, pad=0):
    return cb.build_metadata(reqs, pools, budget, 64, P, 0.0, pad)


def test_prompt_chunks_then_decodes():
    """A 10-token prompt under a 4-token budget: chunks of 4, 4, 2, then one token per step."""
    P = 4
    pools = [{"ring_len": 0, "window_left": -1, "pool_pages": 20, "free_pages": np.arange(2, 22, dtype=np.int32)}]
    reqs = [cb.Request(7, WAITING, 0, 10, [np.zeros(0, np.int32)])]
    free = [pools[0]["free_pages"]]
    seen = []
    for _ in range(5):
        pools[0]["free_pages"] = free[0]
        s = _schedule(reqs, pools, 4, P)
        seen.append((int(s["query_start_loc"][-1]), int(s["seq_lens"][0])))
        reqs, free = cb.advance(reqs, s, free, [0], P)
    assert seen == [(4, 4), (4, 8), (2, 10), (1, 11), (1, 12)]
    r = reqs[0]
    assert (r.state, r.num_computed, r.num_pending) == (DECODING, 12, 1)
    # pages: ceil(12 / 4) = 3 pages taken from the front of the free list, in order; the next step needs a fourth
    assert r.pages[0].tolist() == [2, 3, 4]
    assert free[0][0] == 5


def test_unscheduled_requests_are_unchanged():
    P = 16
    pools = [{"ring_len": 0, "window_left": -1, "pool_pages": 10, "free_pages": np.arange(2, 12, dtype=np.int32)}]
    reqs = [cb.Request(0, DECODING, 20, 1, [np.array([12, 13], np.int32)]),
            cb.Request(1, WAITING, 0, 100, [np.zeros(0, np.int32)])]
    s = _schedule(reqs, pools, 1, P)                 # budget 1: only the decode runs
    out, free = cb.advance(reqs, s, [pools[0]["free_pages"]], [0], P)
    assert (out[0].num_computed, out[0].state) == (21, DECODING)
    assert (out[1].num_computed, out[1].num_pending, out[1].state) == (0, 100, WAITING)
    assert free[0].tolist() == pools[0]["free_pages"].tolist()


def _as_workload(w, reqs, free):
    layers = [dataclasses.replace(lay, free_pages=f) for lay, f in zip(w.layers, free)]
    return dataclasses.replace(w, requests=reqs, layers=layers)


def test_multi_step_metadata_equals_the_oracle_scheduler():
    """Reduced mixed step and hybrid pair, eight steps each: the library's schedule of every step (after advance)
    equals the oracle scheduler's on the same state, bit for bit."""
    for idx in (3, 5):
        w = make_workload(idx, mini=True)
        rings = [lay.ring_len for lay in w.layers]
        reqs = list(w.requests)
        free = [lay.free_pages for lay in w.layers]
        states = set()
        for k in range(8):
            wk = _as_workload(w, reqs, free)
            pools, pad = sched_pools(wk)
            got = cb.build_metadata(wk.requests, pools, w.max_batch_tokens, w.max_requests, w.page_size,
                                    w.safety_margin, pad, policy=w.policy)
            want = OS.build_metadata(wk.requests, pools, w.max_batch_tokens, w.max_requests, w.page_size,
                                     w.safety_margin, pad, policy=w.policy)
            for key in ("query_start_loc", "seq_lens", "req_index"):
                assert np.array_equal(got[key], want[key]), (idx, k, key)
            for l in range(len(w.layers)):
                for key in ("block_table", "slot_mapping"):
                    assert np.array_equal(got["layers"][l][key], want["layers"][l][key]), (idx, k, l, key)
            states |= {r.state for r in wk.requests}
            reqs, free = cb.advance(wk.requests, got, free, rings, w.page_size)
        assert {DECODING, PREFILLING, WAITING} <= states
        assert all(r.state == DECODING for r in reqs)


def _random_loop(seed, steps=24):
    """A random serving loop: one full layer type, or a full and a sliding one (ring); FIFO or PrefillFirst; requests
    arrive over time with random prompt lengths. Yields the layer pool dicts, budget, page size and policy, and per
    step the new arrivals."""
    rng = np.random.default_rng(seed)
    P = int(rng.choice([2, 4, 8, 16]))
    budget = int(rng.integers(P, 8 * P))
    hybrid = bool(rng.integers(0, 2))
    policy = "prefill_first" if rng.integers(0, 3) == 0 else "fifo"
    layers = []
    for l in range(2 if hybrid else 1):
        n_pages = int(rng.integers(60, 400))
        free = (rng.permutation(np.arange(2, n_pages)) if rng.integers(0, 2) else np.arange(2, n_pages))
        if l == 1:
            window = int(rng.integers(1, 6 * P))
            ring = (window + budget + P - 2) // P + 1 + int(rng.integers(0, 3))
            layers.append({"ring_len": ring, "window_left": window, "pool_pages": n_pages - 2,
                           "free_pages": free.astype(np.int32)})
        else:
            layers.append({"ring_len": 0, "window_left": -1, "pool_pages": n_pages - 2,
                           "free_pages": free.astype(np.int32)})
    arrivals = [[int(rng.integers(1, 5 * P)) for _ in range(int(rng.integers(0, 3)))] for _ in range(steps)]
    return layers, budget, P, policy, arrivals


def _same_requests(a, b):
    assert len(a) == len(b)
    for x, y in zip(a, b):
        assert (x.id, x.state, x.num_computed, x.num_pending) == (y.id, y.state, y.num_computed, y.num_pending)
        assert len(x.pages) == len(y.pages)
        for p, q in zip(x.pages, y.pages):
            assert np.array_equal(np.asarray(p), np.asarray(q))


import pytest  # noqa: E402


@pytest.mark.parametrize("seed", range(16))
def test_native_lifecycle_equals_the_oracle_on_random_loops(seed):
    """cb_advance (through the functional advance, and in place through Scheduler.advance_step on the raw metadata
    buffer) equals the oracle's lifecycle step by step: request states, contexts, pending tokens, pages and free
    lists, over random serving loops with arrivals, chunked prompts, decodes, rings and both policies."""
    layers, budget, P, policy, arrivals = _random_loop(seed)
    L = len(layers)
    reqs_o, free_o = [], [lay["free_pages"].copy() for lay in layers]
    reqs_f, free_f = [], [lay["free_pages"].copy() for lay in layers]
    sched = cb.Scheduler([], layers, budget, 16, P, 0.0, 0, policy=policy)
    buf = np.zeros(1 << 16, dtype=np.int32)
    next_id = 0
    ran = 0
    for k, new in enumerate(arrivals):
        for n in new:
            for lst in (reqs_o, reqs_f):
                lst.append(cb.Request(next_id, WAITING, 0, n, [np.zeros(0, np.int32) for _ in range(L)]))
            next_id += 1
        if new:
            sched.set_state(sched.requests + [cb.Request(r.id, r.state, r.num_computed, r.num_pending,
                                                         [p.copy() for p in r.pages]) for r in reqs_f[-len(new):]],
                            sched.free_pages)
        pools_o = [dict(lay, free_pages=f) for lay, f in zip(layers, free_o)]
        want = OS.build_metadata(reqs_o, pools_o, budget, 16, P, 0.0, 0, policy=policy)
        if want["status"] != "ok":
            break
        got = cb.build_metadata(reqs_f, [dict(lay, free_pages=f) for lay, f in zip(layers, free_f)], budget, 16, P,
                                0.0, 0, policy=policy)
        hdr = sched.build_into(buf)
        assert np.array_equal(got["seq_lens"], want["seq_lens"]) and hdr.num_reqs == want["num_reqs"]
        reqs_o, free_o = OS.advance(reqs_o, want, free_o, P)
        reqs_f, free_f = cb.advance(reqs_f, got, free_f, [lay["ring_len"] for lay in layers], P)
        sched.advance_step(hdr, buf)
        ran += 1
        _same_requests(reqs_f, reqs_o)
        _same_requests(sched.requests, reqs_o)
        for l in range(L):
            assert np.array_equal(free_f[l], free_o[l]) and np.array_equal(sched.free_pages[l], free_o[l]), (k, l)
    assert ran >= 4


def test_advance_step_grows_its_page_store():
    """A decode loop long enough that the requests' page lists outgrow the scheduler's page store: the store grows,
    the pages move with it, and every step still equals the oracle's lifecycle."""
    P = 2
    layers = [{"ring_len": 0, "window_left": -1, "pool_pages": 300, "free_pages": np.arange(2, 302, dtype=np.int32)}]
    reqs = [cb.Request(i, DECODING, 3, 1, [np.array([2 * i + 2, 2 * i + 3], np.int32)]) for i in range(3)]
    free = [np.arange(8, 302, dtype=np.int32)]
    sched = cb.Scheduler(reqs, [dict(layers[0], free_pages=free[0])], 64, 8, P)
    stride0 = sched._store_stride
    buf = np.zeros(4096, dtype=np.int32)
    for k in range(40):
        want = OS.build_metadata(reqs, [dict(layers[0], free_pages=free[0])], 64, 8, P)
        hdr = sched.build_into(buf)
        sched.advance_step(hdr, buf)
        reqs, free = OS.advance(reqs, want, free, P)
        _same_requests(sched.requests, reqs)
        assert np.array_equal(sched.free_pages[0], free[0])
    assert sched._store_stride > stride0


def test_cb_advance_checks_before_changing_anything():
    """A store too small for the step's rows (CB_E_CAPACITY), or a row index out of range (CB_E_INVAL): the call
    fails and leaves the requests and free lists as they were."""
    import ctypes as C
    from paged_kv_attention_varlen_amd import _abi
    P = 4
    layers = [{"ring_len": 0, "window_left": -1, "pool_pages": 20, "free_pages": np.arange(2, 22, dtype=np.int32)}]
    sched = cb.Scheduler([cb.Request(0, WAITING, 0, 10, [np.zeros(0, np.int32)])], layers, 16, 4, P)
    buf = np.zeros(1024, dtype=np.int32)
    hdr = sched.build_into(buf)
    lib = _abi.load()
    store = np.zeros(2, dtype=np.int32)
    st = lib.cb_advance(sched.reqs, 1, C.byref(sched.params), sched.pools, buf.ctypes.data_as(_abi.i32p),
                        C.byref(hdr), store.ctypes.data_as(_abi.i32p), 2)     # the row needs 3 pages
    assert st == cb.CB_E_CAPACITY
    assert sched.reqs[0].num_computed == 0 and sched.reqs[0].state == WAITING and sched.pools[0].n_free == 20
    bad = buf.copy()
    bad[hdr.off_req_index] = 5
    store = np.zeros(16, dtype=np.int32)
    st = lib.cb_advance(sched.reqs, 1, C.byref(sched.params), sched.pools, bad.ctypes.data_as(_abi.i32p),
                        C.byref(hdr), store.ctypes.data_as(_abi.i32p), 4)
    assert st == 1   # CB_E_INVAL
    assert sched.reqs[0].num_computed == 0 and sched.pools[0].n_free == 20
    # the failed calls changed nothing, so the real call applies the step once: the whole 10-token prompt ran
    # (budget 16), the request decodes next and owns ceil(10 / 4) = 3 pages, the first three of the free list
    assert hdr.num_tokens == 10 and hdr.used_pages[0] == 3
    sched.advance_step(hdr, buf)
    r = sched.requests[0]
    assert (r.state, r.num_computed, r.num_pending) == (DECODING, 10, 1)
    assert r.pages[0].tolist() == [2, 3, 4] and sched.free_pages[0].tolist() == list(range(5, 22))
