"""Pins of the CPU oracle against things other than itself.

Each check raises AssertionError on failure. tests/test_oracle_pins.py runs them; tests/test_oracle_mutants.py plants
one mistake at a time into the oracle and asserts that at least one check fails.

What pins what:
  worked example (printed values of the "Continuous Batching" blog)  -> scheduler prefix sums, seq_lens, paging rule
  explicit (T,T) block-diagonal mask (same blog)                     -> ragged causal bound of paged_attention
  closed forms (single key, equal scores, a hand-solved 2-key case)  -> softmax, scale, weighted sum of V
  torch SDPA (CPU float64, explicit mask)                            -> attend with context and sliding window
  paged == contiguous, chunked == one-shot, decode == last prefill row, batch invariance -> gather, append, ring
  FIFO fill numbers of the workloads, all-or-nothing admission, 4-slot timeline of the nxmr.cn blog -> scheduler
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import oracle.attention as A
import oracle.reference as R
import oracle.scheduler as S
from synth import DECODING, PREFILLING, WAITING, Request, make_workload

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


def _layer(ring_len=0, window_left=-1, pool_pages=1000, free_pages=()):
    return {"ring_len": ring_len, "window_left": window_left, "pool_pages": pool_pages,
            "free_pages": np.asarray(free_pages, dtype=np.int32)}


def run_oracle_step(w, layer=0):
    """Whole step through the oracle's paged path: schedule, fill history + append into a logical NaN cache,
    paged attention. Returns (sched, out[T, Hq, D], q)."""
    sched = R.schedule(w)
    ids, kc, vc = R.pages_reference(w, layer, sched)
    q, _, _ = R.step_inputs(w, layer, sched)
    lay = sched["layers"][layer]
    rl = lay["ring_len"] if w.layers[layer].ring_len > 0 else None
    out = A.paged_attention(q, kc.astype(np.float64), vc.astype(np.float64), sched["query_start_loc"],
                            sched["seq_lens"], lay["block_table"], w.page_size, w.scale, w.layers[layer].window_left,
                            rl)
    return sched, out, q


# --------------------------------------------------------------------------------------------- worked example


def check_worked_example_metadata():
    g = golden("worked_example.json")
    w = make_workload(1)
    sched = R.schedule(w)
    assert sched["status"] == S.OK
    qsl = sched["query_start_loc"].tolist()
    assert qsl[:-1] == g["printed"]["seq_start_loc"], qsl
    assert qsl == g["derived_by_hand"]["query_start_loc"], qsl
    assert sched["seq_lens"].tolist() == g["printed"]["seq_len"]
    for r, name in enumerate("ABC"):
        assert list(range(qsl[r], qsl[r + 1])) == g["printed"]["global_index"][name]
    lay = sched["layers"][0]
    assert lay["block_table"][2].tolist() == g["printed"]["block_table_C"]
    assert lay["slot_mapping"][6:9].tolist() == g["derived_by_hand"]["slot_mapping_C"]


def check_worked_example_address():
    g = golden("worked_example.json")
    ex = g["printed"]["address_example"]
    P = g["printed"]["BLOCK_SIZE"]
    table = g["printed"]["block_table_C"]
    assert A.page_of(ex["kv_pos"], P) == (ex["logical_block"], ex["block_offset"])
    assert A.physical_page(table, ex["logical_block"]) == ex["physical_block"]
    k2 = g["derived_by_hand"]["kv_pos_2_C"]
    assert A.page_of(2, P) == (k2["logical_block"], k2["block_offset"])
    # markers: cache[page, off] = 100*page + off; C's keys c0, c1, c2 live at (7,0), (7,1), (18,0)
    cache = np.zeros((32, P, 1, 1))
    for p in range(32):
        for o in range(P):
            cache[p, o] = 100 * p + o
    got = A.gather(cache, table, [0, 1, 2], P)[:, 0, 0].tolist()
    assert got == [700.0, 701.0, 1800.0], got


def check_explicit_mask():
    g = golden("worked_example.json")
    qsl = g["derived_by_hand"]["query_start_loc"]
    mask = A.block_diagonal_causal_mask(qsl)
    assert int(mask.sum()) == g["derived_by_hand"]["mask_ones"]
    gi = g["printed"]["global_index"]
    for name, idx in gi.items():
        for a in idx:
            for b in range(9):
                assert mask[a, b] == (b in idx and b <= a)
    # the paged, offset-bounded oracle equals dense attention under the explicit mask
    w = make_workload(1)
    sched, out, q = run_oracle_step(w)
    _, k, v = R.step_inputs(w, 0, sched)
    ref = A.masked_attention(q, k, v, mask, w.scale)
    assert np.max(np.abs(out - ref)) < 1e-12


# ------------------------------------------------------------------------------------------------ closed forms


def check_single_key_returns_value():
    rng = _rng(1)
    q = rng.standard_normal((1, 4, 16))
    k = rng.standard_normal((1, 2, 16))
    v = rng.standard_normal((1, 2, 16))
    out = A.attend(q, k, v, 0, 0.25)
    for h in range(4):
        assert np.array_equal(out[0, h], v[0, h // 2])


def check_equal_scores_give_mean():
    rng = _rng(2)
    q = rng.standard_normal((6, 2, 8))
    k = np.zeros((6, 1, 8))
    v = rng.standard_normal((6, 1, 8))
    out = A.attend(q, k, v, 0, 0.3)
    for i in range(6):
        for h in range(2):
            assert np.allclose(out[i, h], v[:i + 1, 0].mean(axis=0), rtol=0, atol=1e-14)


def check_hand_solved_two_keys():
    # s = scale * <q, k_j> = [0, ln 3]  ->  p = [1/4, 3/4]; v0 = e0, v1 = e1  ->  out = [1/4, 3/4]
    scale = 0.5
    q = np.array([[[1.0, 0.0]]])
    k = np.array([[[0.0, 0.0]], [[math.log(3.0) / scale, 0.0]]])
    v = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])
    out = A.attend(q, k, v, 1, scale)
    assert np.allclose(out[0, 0], [0.25, 0.75], rtol=0, atol=1e-15), out
    # and the first key alone (position 0 with q_len 2): only itself is visible
    q2 = np.array([[[1.0, 0.0]], [[1.0, 0.0]]])
    out2 = A.attend(q2, k, v, 0, scale)
    assert np.allclose(out2[0, 0], [1.0, 0.0]) and np.allclose(out2[1, 0], [0.25, 0.75])


def check_gqa_equals_repeated_mha():
    rng = _rng(3)
    q = rng.standard_normal((5, 8, 16))
    k = rng.standard_normal((9, 2, 16))
    v = rng.standard_normal((9, 2, 16))
    a = A.attend(q, k, v, 4, 0.2)
    b = A.attend(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), 4, 0.2)
    assert np.allclose(a, b, rtol=0, atol=1e-14)


def check_against_torch_sdpa():
    import torch
    rng = _rng(4)
    for ctx, q_len, wl in ((0, 7, -1), (13, 5, -1), (21, 6, 5), (3, 9, 0)):
        Hq, Hkv, D = 6, 3, 16
        q = rng.standard_normal((q_len, Hq, D))
        k = rng.standard_normal((ctx + q_len, Hkv, D))
        v = rng.standard_normal((ctx + q_len, Hkv, D))
        scale = 1.0 / math.sqrt(D)
        ours = A.attend(q, k, v, ctx, scale, wl)
        pos_q = np.arange(ctx, ctx + q_len)[:, None]
        pos_k = np.arange(ctx + q_len)[None, :]
        allowed = pos_k <= pos_q
        if wl >= 0:
            allowed &= pos_k >= pos_q - wl
        G = Hq // Hkv
        tq = torch.from_numpy(q).permute(1, 0, 2)                       # [Hq, q_len, D]
        tk = torch.from_numpy(np.repeat(k, G, axis=1)).permute(1, 0, 2)
        tv = torch.from_numpy(np.repeat(v, G, axis=1)).permute(1, 0, 2)
        ref = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, attn_mask=torch.from_numpy(allowed), scale=scale).permute(1, 0, 2).numpy()
        assert np.max(np.abs(ours - ref)) < 1e-12, (ctx, q_len, wl)


# --------------------------------------------------------------------------------------- paging and chunking


def _fill_logical(rng, n_pages, P, Hkv, D, table, ctx_total, ring_len=0, lo=0):
    kc = np.full((n_pages, P, Hkv, D), np.nan)
    vc = np.full((n_pages, P, Hkv, D), np.nan)
    k = rng.standard_normal((ctx_total, Hkv, D))
    v = rng.standard_normal((ctx_total, Hkv, D))
    for pos in range(lo, ctx_total):
        s = A.slot_of(table, pos, P, ring_len)
        kc[s // P, s % P] = k[pos]
        vc[s // P, s % P] = v[pos]
    return kc, vc, k, v


def check_paged_equals_contiguous():
    rng = _rng(5)
    P, Hq, Hkv, D = 4, 4, 2, 8
    ctx, q_len = 37, 5
    n = -(-(ctx + q_len) // P)
    table = rng.permutation(64)[:n]
    kc, vc, k, v = _fill_logical(rng, 64, P, Hkv, D, table, ctx + q_len)
    q = rng.standard_normal((q_len, Hq, D))
    paged = A.paged_attention(q, kc, vc, [0, q_len], [ctx + q_len], table[None, :], P, 0.3)
    contiguous = A.attend(q, k, v, ctx, 0.3)
    assert np.array_equal(paged, contiguous)
    # ring: window 9, ring of ceil((9 + 5 + 2)/4) + 1 = 5 pages, only the live positions written
    wl, ring = 9, 5
    rtable = rng.permutation(64)[:ring]
    lo = max(0, ctx - wl)
    kc, vc, k, v = _fill_logical(rng, 64, P, Hkv, D, rtable, ctx + q_len, ring, lo)
    paged = A.paged_attention(q, kc, vc, [0, q_len], [ctx + q_len], rtable[None, :], P, 0.3, wl, [ring])
    contiguous = A.attend(q, k, v, ctx, 0.3, wl)
    assert np.array_equal(paged, contiguous)
    assert not np.isnan(paged).any()


def _simulate(prompt_len, budget, P=4, Hq=4, Hkv=2, D=8, seed=6, wl=-1, ring=0):
    """Feed one prompt through oracle steps of at most `budget` tokens; return {position: row}."""
    rng = _rng(seed)
    allq = rng.standard_normal((prompt_len, Hq, D))
    allk = rng.standard_normal((prompt_len, Hkv, D))
    allv = rng.standard_normal((prompt_len, Hkv, D))
    n_pages = 64
    free = rng.permutation(np.arange(2, n_pages)).astype(np.int32)
    kc = np.full((n_pages, P, Hkv, D), np.nan)
    vc = np.full((n_pages, P, Hkv, D), np.nan)
    rq = Request(0, WAITING, 0, prompt_len, [np.zeros(0, np.int32)])
    rows = {}
    while rq.num_pending > 0:
        lay = _layer(ring, wl, n_pages - 2, free)
        sched = S.build_metadata([rq], [lay], budget, 8, P)
        assert sched["status"] == S.OK
        L = sched["layers"][0]
        q_len = int(sched["query_start_loc"][1])
        c = rq.num_computed
        A.kv_append(kc, vc, allk[c:c + q_len], allv[c:c + q_len], L["slot_mapping"], P)
        out = A.paged_attention(allq[c:c + q_len], kc, vc, sched["query_start_loc"], sched["seq_lens"],
                                L["block_table"], P, 0.35, wl, L["ring_len"] if ring else None)
        for i in range(q_len):
            rows[c + i] = out[i]
        used = L["used_pages"]
        new = free[:used]
        free = free[used:]
        rq = Request(0, PREFILLING if rq.num_pending > q_len else DECODING, c + q_len, rq.num_pending - q_len,
                     [np.concatenate([rq.pages[0], new]).astype(np.int32)])
    return rows, (allq, allk, allv)


def check_chunked_equals_oneshot():
    # full attention: the prompt fed in chunks of 7 equals the prompt fed at once, and the definition
    chunked, (q, k, v) = _simulate(23, 7)
    oneshot, _ = _simulate(23, 64)
    direct = A.attend(q, k, v, 0, 0.35)
    for pos in range(23):
        assert np.array_equal(chunked[pos], direct[pos]), pos
        assert np.array_equal(oneshot[pos], direct[pos]), pos
    # sliding window 6 over a ring sized for chunks of up to 7: chunks of 7 and of 3 both equal the definition
    ring = (6 + 7 + 4 - 2) // 4 + 1
    c7, _ = _simulate(23, 7, wl=6, ring=ring)
    c3, _ = _simulate(23, 3, wl=6, ring=ring)
    direct = A.attend(q, k, v, 0, 0.35, 6)
    for pos in range(23):
        assert np.array_equal(c7[pos], direct[pos]), pos
        assert np.array_equal(c3[pos], direct[pos]), pos


def check_decode_equals_last_prefill_row():
    rng = _rng(7)
    q = rng.standard_normal((12, 4, 8))
    k = rng.standard_normal((12, 2, 8))
    v = rng.standard_normal((12, 2, 8))
    full = A.attend(q, k, v, 0, 0.4)
    dec = A.attend(q[11:12], k, v, 11, 0.4)
    assert np.array_equal(full[11], dec[0])


def check_sliding_window():
    rng = _rng(8)
    q = rng.standard_normal((6, 2, 8))
    k = rng.standard_normal((20, 1, 8))
    v = rng.standard_normal((20, 1, 8))
    # window at least as long as every position: same as full attention
    assert np.array_equal(A.attend(q, k, v, 14, 0.3, 19), A.attend(q, k, v, 14, 0.3))
    # brute force: explicit mask pos-4 <= kv_pos <= pos
    pos_q = np.arange(14, 20)[:, None]
    pos_k = np.arange(20)[None, :]
    mask = (pos_k <= pos_q) & (pos_k >= pos_q - 4)
    assert np.max(np.abs(A.attend(q, k, v, 14, 0.3, 4) - A.masked_attention(q, k, v, mask, 0.3))) < 1e-14
    # each row sees exactly window_left + 1 keys
    assert mask.sum(axis=1).tolist() == [5] * 6


def check_batch_invariance():
    w = make_workload(3, mini=True)
    sched, out, _ = run_oracle_step(w)
    alone = {}
    qsl = sched["query_start_loc"]
    for r in range(sched["num_reqs"]):
        i = int(sched["req_index"][r])
        rq = w.requests[i]
        q_len = int(qsl[r + 1] - qsl[r])
        ctx = rq.num_computed
        q = w.values("q", i, 0, ctx, ctx + q_len)
        k = w.values("k", i, 0, 0, ctx + q_len)
        v = w.values("v", i, 0, 0, ctx + q_len)
        alone = A.attend(q, k, v, ctx, w.scale)
        assert np.array_equal(out[qsl[r]:qsl[r + 1]], alone), r


def check_workload_paged_equals_definition():
    for idx in (2, 5):
        w = make_workload(idx, mini=True)
        for layer in range(len(w.layers)):
            sched, out, _ = run_oracle_step(w, layer)
            ref = R.rows_reference(w, layer, sched)
            for t, row in ref.items():
                assert np.array_equal(out[t], row), (idx, layer, t)
            assert not np.isnan(out).any()


# --------------------------------------------------------------------------------------------------- scheduler


def check_fifo_fill_of_workloads():
    w = make_workload(3)
    s = R.schedule(w)
    ql = np.diff(s["query_start_loc"]).tolist()
    assert s["num_decodes"] == 96 and ql == [1] * 96 + [512, 512, 928] and s["num_tokens"] == 2048
    assert s["seq_lens"][96:].tolist() == [1536, 3584, 928]
    w = make_workload(5)
    s = R.schedule(w)
    ql = np.diff(s["query_start_loc"]).tolist()
    assert ql == [1] * 128 + [2048, 2048, 2048, 1920] and s["num_tokens"] == 8192
    for idx in (2, 4):
        w = make_workload(idx)
        s = R.schedule(w)
        n = len(w.requests)
        assert s["num_reqs"] == n and s["num_decodes"] == n and s["num_tokens"] == n
        # a decode needs a new page exactly when its context fills its last page
        boundary = sum(1 for rq in w.requests if rq.num_computed % w.page_size == 0)
        assert s["layers"][0]["used_pages"] == boundary


def check_padding_pages_never_allocated():
    for idx in (2, 3, 4, 5):
        w = make_workload(idx, mini=True)
        s = R.schedule(w)
        for l, lay in enumerate(w.layers):
            L = s["layers"][l]
            for r in range(s["num_reqs"]):
                n = L["width"] if lay.ring_len > 0 else -(-int(s["seq_lens"][r]) // w.page_size)
                assert not set(L["block_table"][r, :n].tolist()) & set(lay.padding_pages)
                assert set(L["block_table"][r, n:].tolist()) <= {0}


def check_admission_all_or_nothing():
    P = 4
    dec = Request(0, DECODING, 9, 1, [np.arange(10, 13, dtype=np.int32), np.arange(20, 26, dtype=np.int32)])
    new = Request(1, WAITING, 0, 10, [np.zeros(0, np.int32), np.zeros(0, np.int32)])
    ring = (3 + 16 + P - 2) // P + 1
    full_free = np.arange(40, 50, dtype=np.int32)
    # sliding pool has fewer pages than one ring: the new request is rejected and takes no full page either
    s = S.build_metadata([dec, new], [_layer(0, -1, 50, full_free), _layer(ring, 3, 50, np.arange(60, 63))], 16, 8, P)
    assert s["status"] == S.OK and s["num_reqs"] == 1 and s["first_rejected"] == 1
    assert s["layers"][0]["used_pages"] == 0 and s["layers"][1]["used_pages"] == 0
    # with room in both, it is admitted: ceil(10/4) = 3 full pages and one whole ring
    s = S.build_metadata([dec, new], [_layer(0, -1, 50, full_free), _layer(ring, 3, 50, np.arange(60, 60 + ring))],
                         16, 8, P)
    assert s["num_reqs"] == 2 and s["layers"][0]["used_pages"] == 3 and s["layers"][1]["used_pages"] == ring
    assert s["layers"][0]["block_table"][1, :3].tolist() == [40, 41, 42]
    # head-of-line: a second waiting request behind a rejected one is not admitted
    small = Request(2, WAITING, 0, 1, [np.zeros(0, np.int32), np.zeros(0, np.int32)])
    s = S.build_metadata([dec, new, small], [_layer(0, -1, 50, full_free), _layer(ring, 3, 50, np.arange(60, 63))],
                         16, 8, P)
    assert s["num_reqs"] == 1 and s["first_rejected"] == 1


def check_stall_nospace_margin_cap():
    P = 4
    a = Request(0, DECODING, 8, 1, [np.array([5, 6], np.int32)])        # needs a third page
    b = Request(1, DECODING, 6, 1, [np.array([7, 8], np.int32)])        # fits in its second page
    s = S.build_metadata([a, b], [_layer(0, -1, 10, [])], 16, 8, P)
    assert s["status"] == S.OK and s["stalled"].tolist() == [0] and s["req_index"].tolist() == [1]
    assert s["layers"][0]["slot_mapping"].tolist() == [8 * 4 + 2]
    s = S.build_metadata([a], [_layer(0, -1, 10, [])], 16, 8, P)
    assert s["status"] == S.E_NOSPACE and s["num_reqs"] == 0
    # safety margin: 3 free of 10 pages is below 0.5 -> the waiting prompt is held, the decode runs
    w = Request(2, WAITING, 0, 3, [np.zeros(0, np.int32)])
    s = S.build_metadata([b, w], [_layer(0, -1, 10, [30, 31, 32])], 16, 8, P, safety_margin=0.5)
    assert s["held_by_margin"] and s["num_reqs"] == 1
    s = S.build_metadata([b, w], [_layer(0, -1, 10, [30, 31, 32])], 16, 8, P, safety_margin=0.2)
    assert not s["held_by_margin"] and s["num_reqs"] == 2
    # request cap and token budget
    many = [Request(i, DECODING, 2, 1, [np.array([40 + i], np.int32)]) for i in range(6)]
    s = S.build_metadata(many, [_layer(0, -1, 100, [])], 16, 4, P)
    assert s["num_reqs"] == 4 and s["req_index"].tolist() == [0, 1, 2, 3]
    s = S.build_metadata(many, [_layer(0, -1, 100, [])], 3, 8, P)
    assert s["num_reqs"] == 3
    # FIFO: decodes, then active prefills, then waiting -- whatever the list order
    pf = Request(7, PREFILLING, 4, 5, [np.array([50], np.int32)])
    wt = Request(8, WAITING, 0, 2, [np.zeros(0, np.int32)])
    s = S.build_metadata([wt, pf, many[0]], [_layer(0, -1, 100, np.arange(60, 70))], 16, 8, P)
    assert s["req_index"].tolist() == [2, 1, 0] and np.diff(s["query_start_loc"]).tolist() == [1, 5, 2]
    # invalid inputs
    assert S.build_metadata([Request(0, DECODING, 3, 2, [np.array([1], np.int32)])],
                            [_layer()], 16, 8, P)["status"] == S.E_INVAL
    assert S.build_metadata([Request(0, DECODING, 9, 1, [np.array([1], np.int32)])],
                            [_layer()], 16, 8, P)["status"] == S.E_INVAL
    assert S.build_metadata([wt], [_layer(2, 4, 10, [])], 16, 8, P)["status"] == S.E_INVAL


def check_prefill_first_order():
    """PrefillFirst finishes prefill work before decodes resume (Transformers "continuous batching architecture"
    page, section "PrefillFirst"): with a budget of 8, a decode, a continuing prefill with 6 prompt tokens left and
    a waiting prompt of 5, FIFO runs the decode, the 6 tokens and 1 token of the new prompt; PrefillFirst runs the 6
    tokens and 2 of the new prompt, and the decode waits for budget. Rows are laid out decodes first either way;
    pages come from the free list in scheduling order."""
    P = 4
    d = Request(0, DECODING, 8, 1, [np.array([5, 6], np.int32)])          # needs a third page (a new block)
    pf = Request(1, PREFILLING, 4, 6, [np.array([7], np.int32)])         # 4 + 6 = 10 keys -> 2 more pages
    wt = Request(2, WAITING, 0, 5, [np.zeros(0, np.int32)])
    free = np.arange(20, 30, dtype=np.int32)
    s = S.build_metadata([d, pf, wt], [_layer(0, -1, 50, free)], 8, 8, P)
    assert s["req_index"].tolist() == [0, 1, 2] and np.diff(s["query_start_loc"]).tolist() == [1, 6, 1]
    assert s["layers"][0]["block_table"][0, :3].tolist() == [5, 6, 20]            # the decode took page 20 first
    s = S.build_metadata([d, pf, wt], [_layer(0, -1, 50, free)], 8, 8, P, policy=S.PREFILL_FIRST)
    assert s["req_index"].tolist() == [1, 2] and np.diff(s["query_start_loc"]).tolist() == [6, 2]
    assert s["num_decodes"] == 0 and s["stalled"].tolist() == []
    assert s["layers"][0]["block_table"][0, :3].tolist() == [7, 20, 21]           # the prefill took 20, 21
    # with budget to spare the decode runs after the prefill work, laid out first, taking the next free page
    s = S.build_metadata([d, pf, wt], [_layer(0, -1, 50, free)], 16, 8, P, policy=S.PREFILL_FIRST)
    assert s["req_index"].tolist() == [0, 1, 2] and np.diff(s["query_start_loc"]).tolist() == [1, 6, 5]
    assert s["layers"][0]["block_table"][0, :3].tolist() == [5, 6, 24]
    # the safety margin holds new prompts, never the work already running (page: FIFO default 0.15)
    s = S.build_metadata([d, pf, wt], [_layer(0, -1, 50, free[:3])], 16, 8, P, safety_margin=0.15,
                         policy=S.PREFILL_FIRST)
    assert s["held_by_margin"] and s["req_index"].tolist() == [0, 1]
    s = S.build_metadata([d, pf, wt], [_layer(0, -1, 50, free[:2])], 16, 8, P, safety_margin=0.15,
                         policy=S.PREFILL_FIRST)
    assert s["held_by_margin"] and s["req_index"].tolist() == [1]
    assert s["stalled"].tolist() == [0]         # the last free pages went to the prefill: the decode stalls
    s = S.build_metadata([d, pf, wt], [_layer(0, -1, 50, free[:2])], 16, 8, P, safety_margin=0.15)
    assert s["held_by_margin"] and s["req_index"].tolist() == [0] and s["stalled"].tolist() == [1]


def check_swap_roundtrip_preserves_attention():
    """Offloading moves a request's pages to a swap buffer and back into other free pages; with the block table
    pointing at the new pages, every output row is unchanged (attention depends on the pages' contents only through
    the block table)."""
    rng = np.random.default_rng(11)
    P, Hq, Hkv, D, n_pages = 4, 4, 2, 8, 24
    qsl = np.array([0, 1, 4], np.int32)
    seq = np.array([11, 9], np.int32)
    table = np.array([[5, 9, 2], [7, 3, 14]], np.int32)
    kc = rng.standard_normal((n_pages, P, Hkv, D))
    vc = rng.standard_normal((n_pages, P, Hkv, D))
    q = rng.standard_normal((4, Hq, D))
    before = A.paged_attention(q, kc, vc, qsl, seq, table, P, 0.3)
    swap_k = np.zeros((3, P, Hkv, D))
    swap_v = np.zeros((3, P, Hkv, D))
    A.copy_pages(swap_k, None, kc, table[1])
    A.copy_pages(swap_v, None, vc, table[1])
    kc[table[1]] = np.nan                        # the freed pages are reused by someone else
    vc[table[1]] = np.nan
    new = np.array([20, 16, 18], np.int32)
    A.copy_pages(kc, new, swap_k, None)
    A.copy_pages(vc, new, swap_v, None)
    table2 = table.copy()
    table2[1] = new
    after = A.paged_attention(q, kc, vc, qsl, seq, table2, P, 0.3)
    assert np.array_equal(before, after)
    # out-of-range pairs are skipped, the rest copied
    dst = np.zeros((2, 3))
    A.copy_pages(dst, np.array([1, 5]), np.arange(9.0).reshape(3, 3), np.array([2, 0]))
    assert dst.tolist() == [[0, 0, 0], [6, 7, 8]]


def check_four_slot_timeline():
    g = golden("four_slot_example.json")
    steps = g["decode_steps"]
    names = list(steps)
    reqs = {n: Request(i, DECODING if n != "E" else WAITING, 1, 1, [np.array([i], np.int32)])
            for i, n in enumerate(names)}
    reqs["E"] = Request(4, WAITING, 0, 1, [np.zeros(0, np.int32)])
    left = dict(steps)
    finish, enter = {}, None
    free = np.arange(100, 2000, dtype=np.int32)
    step = 0
    while left:
        step += 1
        active = [reqs[n] for n in names if n in left]
        s = S.build_metadata(active, [_layer(0, -1, 10000, free)], 1024, g["slots"], 4096)
        assert s["status"] == S.OK
        ran = [active[i] for i in s["req_index"].tolist()]
        free = free[s["layers"][0]["used_pages"]:]
        for rq in ran:
            n = names[rq.id]
            if n == "E" and enter is None:
                enter = step - 1
            left[n] -= 1
            if left[n] == 0:
                finish[n] = step
                del left[n]
            else:
                reqs[n] = Request(rq.id, DECODING, rq.num_computed + 1, 1,
                                  [rq.pages[0] if len(rq.pages[0]) else np.array([999 + rq.id], np.int32)])
    c = g["continuous"]
    assert enter == c["E_enters_at_step"], enter
    assert finish == c["finish_step"], finish
    ms = g["ms_per_step"] / 1000.0
    assert max(finish.values()) * ms == c["makespan_s"]
    lat = {n: finish[n] * ms for n in names}
    assert lat == c["latency_s"]
    assert round(sum(lat.values()) / len(lat), 6) == c["mean_latency_s"]
    # static batching (context only): the first four run to the longest, then E alone
    first = max(steps[n] for n in names[:4])
    st = {n: steps[n] for n in names[:4]}
    st["E"] = first + steps["E"]
    assert st == g["static"]["finish_step"] and st["E"] * ms == g["static"]["makespan_s"]
    assert round(g["static"]["latency_s"]["E"] / lat["E"], 1) == g["E_speedup"]
    assert sum(steps.values()) == g["total_tokens"]


def check_request_lifecycle():
    """The lifecycle after each step (Transformers page, section "请求生命周期"), hand-worked from its rules.
    A 10-token prompt under a 4-token budget with 4-key pages prefills in chunks of 4, 4 and 2, then decodes one
    token per step: (tokens, seq_len) per step (4, 4), (4, 8), (2, 10), (1, 11), (1, 12). After the fifth step it
    decodes with context 12 and one pending token and owns ceil(12 / 4) = 3 pages, the first three of the free list
    (2, 3, 4), whose front is then page 5. A sliding layer's request owns its whole ring from admission on. With
    prefix sharing, a step registers exactly the prompt blocks it completed: a 10-token prompt with 4-key pages has
    two full blocks, filled by the first two chunks of 4."""
    P = 4
    free = [np.arange(2, 22, dtype=np.int32)]
    reqs = [Request(7, WAITING, 0, 10, [np.zeros(0, np.int32)])]
    seen = []
    for _ in range(5):
        s = S.build_metadata(reqs, [_layer(0, -1, 20, free[0])], 4, 8, P)
        seen.append((int(s["num_tokens"]), int(s["seq_lens"][0])))
        reqs, free = S.advance(reqs, s, free, P)
    assert seen == [(4, 4), (4, 8), (2, 10), (1, 11), (1, 12)], seen
    r = reqs[0]
    assert (r.state, r.num_computed, r.num_pending) == (DECODING, 12, 1)
    assert r.pages[0].tolist() == [2, 3, 4] and int(free[0][0]) == 5
    # a request the step leaves out keeps everything
    idle = Request(8, WAITING, 0, 50, [np.zeros(0, np.int32)])
    s = S.build_metadata([r, idle], [_layer(0, -1, 20, free[0])], 1, 8, P)
    out, free2 = S.advance([r, idle], s, free, P)
    assert (out[1].state, out[1].num_computed, out[1].num_pending) == (WAITING, 0, 50)
    assert (out[0].num_computed, out[0].state, out[0].pages[0].tolist()) == (13, DECODING, [2, 3, 4, 5])
    assert free2[0].tolist() == free[0][1:].tolist()
    # ring layer: window 3, ring of 4 pages taken at admission; the pages stay the ring as the request grows
    ring_free = [np.arange(30, 40, dtype=np.int32)]
    q = [Request(1, WAITING, 0, 6, [np.zeros(0, np.int32)])]
    for k in range(3):
        s = S.build_metadata(q, [_layer(4, 3, 10, ring_free[0])], 4, 8, P)
        q, ring_free = S.advance(q, s, ring_free, P)
        assert q[0].pages[0].tolist() == [30, 31, 32, 33]
    assert (q[0].num_computed, q[0].state) == (7, DECODING) and ring_free[0].tolist() == list(range(34, 40))
    # prefix sharing: blocks 0 and 1 of the prompt are registered by the steps that complete them, block 2 never
    from oracle.prefix_cache import PrefixCache, block_hashes
    prompt = np.arange(100, 110, dtype=np.int32)
    hashes = [block_hashes(prompt, P)]
    cache = PrefixCache(20, list(range(2, 20)))
    q = [Request(3, WAITING, 0, 10, [np.zeros(0, np.int32)])]
    registered = []
    for k in range(3):
        s = S.build_metadata(q, [_layer(0, -1, 18, np.zeros(0, np.int32))], 4, 8, P, prefix_cache=cache,
                             prompt_hashes=hashes)
        q, _ = S.advance(q, s, [np.zeros(0, np.int32)], P, cache, hashes)
        registered.append(sorted(cache.index.values()))
    pages = q[0].pages[0].tolist()
    assert registered == [[pages[0]], [pages[0], pages[1]], [pages[0], pages[1]]], (registered, pages)


ALL_CHECKS = [
    check_worked_example_metadata, check_worked_example_address, check_explicit_mask,
    check_single_key_returns_value, check_equal_scores_give_mean, check_hand_solved_two_keys,
    check_gqa_equals_repeated_mha, check_against_torch_sdpa, check_paged_equals_contiguous,
    check_chunked_equals_oneshot, check_decode_equals_last_prefill_row, check_sliding_window,
    check_batch_invariance, check_workload_paged_equals_definition, check_fifo_fill_of_workloads,
    check_padding_pages_never_allocated, check_admission_all_or_nothing, check_stall_nospace_margin_cap,
    check_prefill_first_order, check_swap_roundtrip_preserves_attention, check_four_slot_timeline,
    check_request_lifecycle,
]
