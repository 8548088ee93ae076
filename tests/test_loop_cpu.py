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
