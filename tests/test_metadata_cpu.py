"""cb_build_metadata (C++) against the oracle's scheduler reference (Python), bit for bit, on the five workloads,
their reduced variants, seeded random request mixes and the error paths."""
import numpy as np
import pytest

import oracle.scheduler as S
import paged_kv_attention_varlen_amd as cb
from oracle.reference import schedule as oracle_schedule
from synth import DECODING, PREFILLING, WAITING, Request, make_workload

_STATUS = {S.OK: cb.CB_OK, S.E_INVAL: 1, S.E_NOSPACE: cb.CB_E_NOSPACE}


def _pools(w):
    return [{"ring_len": l.ring_len, "window_left": l.window_left, "pool_pages": l.num_pages - len(l.padding_pages),
             "free_pages": l.free_pages} for l in w.layers]


def _compare(ref, got):
    assert _STATUS[ref["status"]] == got["status"]
    if ref["status"] == S.E_INVAL:
        return
    for k in ("num_reqs", "num_tokens", "num_decodes", "first_rejected", "held_by_margin"):
        assert ref[k] == got[k], k
    for k in ("query_start_loc", "seq_lens", "req_index", "stalled"):
        assert np.array_equal(np.asarray(ref[k], np.int64), np.asarray(got[k], np.int64)), k
    assert len(ref["layers"]) == len(got["layers"])
    for a, b in zip(ref["layers"], got["layers"]):
        assert a["used_pages"] == b["used_pages"]
        assert a["block_table"].shape == b["block_table"].shape
        assert np.array_equal(a["block_table"], b["block_table"])
        assert np.array_equal(a["slot_mapping"], b["slot_mapping"])
        assert np.array_equal(a["ring_len"], b["ring_len"])


@pytest.mark.parametrize("mini", [True, False], ids=["reduced", "full"])
@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_workload_metadata_bit_exact(idx, mini):
    w = make_workload(idx, mini=mini)
    ref = oracle_schedule(w)
    pad = w.layers[0].padding_pages[0] if w.layers[0].padding_pages else 0
    got = cb.build_metadata(w.requests, _pools(w), w.max_batch_tokens, w.max_requests, w.page_size,
                            w.safety_margin, pad)
    _compare(ref, got)


def _random_case(rng, two_layers):
    P = int(rng.choice([1, 2, 4, 16]))
    budget = int(rng.integers(1, 64))
    window = int(rng.integers(0, 20))
    ring = (window + budget + P - 2) // P + 1 + int(rng.integers(0, 2))
    L = 2 if two_layers else 1
    n_pages = 400
    perm = [rng.permutation(np.arange(2, n_pages)).astype(np.int32) for _ in range(L)]
    pos = [0] * L
    reqs = []
    for i in range(int(rng.integers(0, 12))):
        st = int(rng.choice([DECODING, PREFILLING, WAITING]))
        comp = int(rng.integers(0, 40)) if st != WAITING else int(rng.choice([0, 0, rng.integers(0, 10)]))
        pend = 1 if st == DECODING else int(rng.integers(1, 50))
        pages = []
        for l in range(L):
            need = (comp + P - 1) // P if l == 0 else (ring if st != WAITING else 0)
            extra = int(rng.integers(0, 2)) if l == 0 else 0
            pages.append(perm[l][pos[l]:pos[l] + need + extra].copy())
            pos[l] += need + extra
        reqs.append(Request(i, st, comp, pend, pages))
    layers = []
    for l in range(L):
        nfree = int(rng.integers(0, 30))
        layers.append({"ring_len": 0 if l == 0 else ring, "window_left": -1 if l == 0 else window,
                       "pool_pages": n_pages - 2, "free_pages": perm[l][pos[l]:pos[l] + nfree]})
    margin = float(rng.choice([0.0, 0.0, 0.25, 0.5, 0.9375]))
    cap = int(rng.integers(1, 10))
    return reqs, layers, budget, cap, P, margin


@pytest.mark.parametrize("policy", [S.FIFO, S.PREFILL_FIRST])
@pytest.mark.parametrize("seed", range(60))
def test_random_mixes_bit_exact(seed, policy):
    rng = np.random.default_rng(seed)
    reqs, layers, budget, cap, P, margin = _random_case(rng, two_layers=bool(seed % 2))
    ref = S.build_metadata(reqs, layers, budget, cap, P, margin, 0, policy=policy)
    got = cb.build_metadata(reqs, layers, budget, cap, P, margin, 0, policy=policy)
    _compare(ref, got)


@pytest.mark.parametrize("idx", [3, 5])
def test_workload_prefill_first_bit_exact(idx):
    w = make_workload(idx)
    pad = w.layers[0].padding_pages[0] if w.layers[0].padding_pages else 0
    ref = S.build_metadata(w.requests, _pools(w), w.max_batch_tokens, w.max_requests, w.page_size, 0.0, pad,
                           policy=S.PREFILL_FIRST)
    got = cb.build_metadata(w.requests, _pools(w), w.max_batch_tokens, w.max_requests, w.page_size, 0.0, pad,
                            policy="prefill_first")
    _compare(ref, got)
    # the chunks get the budget first: every prompt token that fits is scheduled before any decode
    pre = int(np.diff(ref["query_start_loc"])[ref["num_decodes"]:].sum())
    assert pre == min(w.max_batch_tokens, sum(rq.num_pending for rq in w.requests if rq.state != DECODING))


def test_unknown_policy_is_rejected():
    lay = [{"ring_len": 0, "window_left": -1, "pool_pages": 10, "free_pages": np.arange(2, 12)}]
    ok = [Request(0, WAITING, 0, 3, [np.zeros(0, np.int32)])]
    assert S.build_metadata(ok, lay, 16, 8, 4, policy="lifo")["status"] == S.E_INVAL
    lib = cb._abi.load()
    params = cb._abi.cb_sched_params(16, 8, 4, 0, 1, 7, 0.0)
    pools = (cb._abi.cb_layer_pool * 1)(cb._abi.cb_layer_pool(0, -1, 10, 0, None))
    step = cb._abi.cb_step()
    buf = np.zeros(64, np.int32)
    reqs = (cb._abi.cb_req * 1)()
    st = lib.cb_build_metadata(reqs, 0, cb.C.byref(params), pools, buf.ctypes.data_as(cb._abi.i32p), 64,
                               cb.C.byref(step))
    assert st == cb._abi.CB_E_INVAL


def test_error_paths_match():
    lay = [{"ring_len": 0, "window_left": -1, "pool_pages": 10, "free_pages": np.arange(2, 12)}]
    bad = [
        [Request(0, DECODING, 4, 2, [np.array([3], np.int32)])],               # decode with 2 tokens
        [Request(0, DECODING, 9, 1, [np.array([3], np.int32)])],               # too few owned pages
        [Request(0, 7, 0, 1, [np.zeros(0, np.int32)])],                         # unknown state
        [Request(0, WAITING, -1, 1, [np.zeros(0, np.int32)])],                  # negative context
        [Request(0, PREFILLING, 0, 0, [np.zeros(0, np.int32)])],                # nothing pending
    ]
    for reqs in bad:
        assert S.build_metadata(reqs, lay, 16, 8, 4)["status"] == S.E_INVAL
        assert cb.build_metadata(reqs, lay, 16, 8, 4)["status"] == cb._abi.CB_E_INVAL
    ok = [Request(0, WAITING, 0, 3, [np.zeros(0, np.int32)])]
    assert cb.build_metadata(ok, lay, 0, 8, 4)["status"] == cb._abi.CB_E_INVAL     # zero budget
    ring_small = [{"ring_len": 2, "window_left": 8, "pool_pages": 10, "free_pages": np.arange(2, 12)}]
    assert cb.build_metadata(ok, ring_small, 16, 8, 4)["status"] == cb._abi.CB_E_INVAL


def test_nospace_leaves_free_list_untouched():
    a = Request(0, DECODING, 8, 1, [np.array([5, 6], np.int32)])
    w = Request(1, WAITING, 0, 9, [np.zeros(0, np.int32)])
    free = np.array([40], np.int32)
    got = cb.build_metadata([a, w], [{"ring_len": 0, "window_left": -1, "pool_pages": 10, "free_pages": free}],
                            16, 8, 4)
    # the decode takes the only page; the waiting request needs 3 and is refused without taking any
    assert got["status"] == cb.CB_OK and got["num_reqs"] == 1 and got["first_rejected"] == 1
    assert got["layers"][0]["used_pages"] == 1
    got = cb.build_metadata([w], [{"ring_len": 0, "window_left": -1, "pool_pages": 10, "free_pages": free}],
                            16, 8, 4)
    assert got["status"] == cb.CB_E_NOSPACE and got["layers"][0]["used_pages"] == 0 and got["num_reqs"] == 0
