"""Prefix sharing at admission (Transformers "continuous batching architecture" page, sections "前缀缓存" and "准入"):
the oracle scheduler's reading pinned on hand-worked cases. A request whose prompt starts with blocks another
request has completed reuses their pages and starts its chunk at the matched context; at least one prompt token is
always computed; admission stays all-or-nothing; a ring (sliding) layer turns sharing off."""
from types import SimpleNamespace as NS

import numpy as np

import oracle.prefix_cache as O
from oracle import scheduler as S

P = 4
DEC, PRE, WAIT = S.DECODING, S.PREFILLING, S.WAITING
PROMPT_A = np.arange(10, dtype=np.int32)                                       # blocks 0, 1 full; block 2 partial
PROMPT_B = np.concatenate([np.arange(8), np.arange(100, 106)]).astype(np.int32)  # shares A's blocks 0 and 1


def req(rid, state, computed, pending, pages=()):
    return NS(id=rid, state=state, num_computed=computed, num_pending=pending, pages=[np.array(pages, np.int32)])


def full_pool(free):
    return [{"ring_len": 0, "window_left": -1, "pool_pages": len(free), "free_pages": np.array(free, np.int32)}]


def a_after_first_step(cache):
    """A alone: admitted with 10 tokens on fresh pages 2, 3, 4; its two completed blocks are then registered."""
    s = S.build_metadata([req(0, WAIT, 0, 10)], full_pool([]), 64, 8, P, prefix_cache=cache,
                         prompt_hashes=[O.block_hashes(PROMPT_A, P)])
    assert s["status"] == "ok" and s["layers"][0]["block_table"].tolist() == [[2, 3, 4]]
    assert s["matched_tokens"].tolist() == [0]
    ha = O.block_hashes(PROMPT_A, P)
    assert cache.commit(2, ha[0]) and cache.commit(3, ha[1])
    return req(0, DEC, 10, 1, [2, 3, 4])


def test_second_request_reuses_the_shared_prefix_pages():
    cache = O.PrefixCache(22, range(2, 22))
    a = a_after_first_step(cache)
    b = req(1, WAIT, 0, len(PROMPT_B))
    hashes = [O.block_hashes(PROMPT_A, P), O.block_hashes(PROMPT_B, P)]
    s = S.build_metadata([a, b], full_pool([]), 64, 8, P, prefix_cache=cache, prompt_hashes=hashes)
    assert s["status"] == "ok" and s["prefix_sharing"]
    # A decodes position 10 (page 4, offset 2); B skips 8 tokens and prefills positions 8..13 on fresh pages 5, 6
    assert s["query_start_loc"].tolist() == [0, 1, 7]
    assert s["seq_lens"].tolist() == [11, 14]
    assert s["matched_tokens"].tolist() == [0, 8]
    L = s["layers"][0]
    assert L["block_table"].tolist() == [[2, 3, 4, 0], [2, 3, 5, 6]]
    assert L["slot_mapping"].tolist() == [18, 20, 21, 22, 23, 24, 25]
    assert L["used_pages"] == 2
    assert [cache.ref[p] for p in (2, 3, 4, 5, 6)] == [2, 2, 1, 1, 1]


def test_at_least_one_prompt_token_is_computed():
    """A prompt made only of cached blocks still computes its last block's tokens: 8 tokens match at most 1 block."""
    cache = O.PrefixCache(22, range(2, 22))
    a = a_after_first_step(cache)
    b = req(1, WAIT, 0, 8)
    s = S.build_metadata([a, b], full_pool([]), 64, 8, P, prefix_cache=cache,
                         prompt_hashes=[O.block_hashes(PROMPT_A, P), O.block_hashes(PROMPT_A[:8], P)])
    assert s["matched_tokens"].tolist() == [0, 4]
    assert s["seq_lens"].tolist() == [11, 8]
    assert s["layers"][0]["block_table"].tolist()[1] == [2, 5, 0]


def test_admission_is_all_or_nothing_with_a_match():
    """Pool of four pages: after A only page 5 is free; B matches two blocks but needs two fresh pages -> refused,
    and the cache is untouched (no references taken)."""
    cache = O.PrefixCache(6, [2, 3, 4, 5])
    a = a_after_first_step(cache)
    b = req(1, WAIT, 0, len(PROMPT_B))
    s = S.build_metadata([a, b], full_pool([]), 64, 8, P, prefix_cache=cache,
                         prompt_hashes=[O.block_hashes(PROMPT_A, P), O.block_hashes(PROMPT_B, P)])
    assert s["first_rejected"] == 1 and s["num_reqs"] == 1
    assert [cache.ref[p] for p in (2, 3, 4, 5)] == [1, 1, 1, 0] and cache.empty == [5]


def test_match_of_freed_blocks_counts_them_out_of_the_free_pool():
    """A has finished and released its pages: 2 and 3 stay initialized (their blocks registered), 4 is empty.
    B matches 2 and 3 -- which leave the free pool -- and takes its fresh pages from the empty ones first."""
    cache = O.PrefixCache(8, [2, 3, 4, 5, 6])
    a_after_first_step(cache)
    assert cache.release([2, 3, 4]) and cache.stats() == (3, 2, 2)
    b = req(1, WAIT, 0, len(PROMPT_B))
    s = S.build_metadata([b], full_pool([]), 64, 8, P, prefix_cache=cache,
                         prompt_hashes=[O.block_hashes(PROMPT_B, P)])
    assert s["layers"][0]["block_table"].tolist() == [[2, 3, 5, 6]]
    assert cache.stats() == (1, 0, 2) and cache.empty == [4]
    # with only one fresh page obtainable besides the matched ones the same admission is refused
    cache2 = O.PrefixCache(6, [2, 3, 4, 5])
    a_after_first_step(cache2)
    assert cache2.release([2, 3, 4])
    assert cache2.allocate(1) == [5] and cache2.n_free() == 3          # free: 4 (empty), 2 and 3 (initialized)
    s = S.build_metadata([req(1, WAIT, 0, len(PROMPT_B))], full_pool([]), 64, 8, P, prefix_cache=cache2,
                         prompt_hashes=[O.block_hashes(PROMPT_B, P)])
    assert s["first_rejected"] == 0 and cache2.stats() == (1, 2, 2)


def test_a_ring_layer_turns_sharing_off():
    """Full + sliding layer types: the cache is ignored; pages come from the layers' free lists as usual."""
    cache = O.PrefixCache(22, range(2, 22))
    a_after_first_step(cache)
    before = (list(cache.ref), cache.stats())
    layers = [{"ring_len": 0, "window_left": -1, "pool_pages": 10, "free_pages": np.arange(30, 40, dtype=np.int32)},
              {"ring_len": 8, "window_left": 8, "pool_pages": 16, "free_pages": np.arange(50, 66, dtype=np.int32)}]
    b = NS(id=1, state=WAIT, num_computed=0, num_pending=len(PROMPT_B), pages=[np.zeros(0, np.int32)] * 2)
    s = S.build_metadata([b], layers, 16, 8, P, prefix_cache=cache, prompt_hashes=[O.block_hashes(PROMPT_B, P)])
    assert not s["prefix_sharing"] and s["matched_tokens"].tolist() == [0]
    assert s["layers"][0]["block_table"].tolist() == [[30, 31, 32, 33]]
    assert (list(cache.ref), cache.stats()) == before


def _cache_state(c, n_pages, lib_side):
    if lib_side:
        info = [c.page_info(p) for p in range(n_pages)]
        return c.stats(), [(r, bool(reg), h if reg else 0) for r, reg, h in info]
    return c.stats(), [(c.ref[p], c.hash[p] is not None, c.hash[p] or 0) for p in range(n_pages)]


import pytest  # noqa: E402


@pytest.mark.parametrize("seed", range(12))
def test_library_matches_oracle_on_random_shared_prefix_loops(seed):
    """Random serving loops with shared prompt prefixes: requests arrive, share prefixes of a few base prompts,
    prefill in chunks, decode and finish (releasing their pages). Every step the library's schedule equals the
    oracle's (metadata, matched context, pages) and both caches hold the same state; the same lifecycle then moves
    both request lists on, registering the prompt blocks each step completed."""
    import paged_kv_attention_varlen_amd as cb
    rng = np.random.default_rng(seed)
    P = int(rng.choice([4, 8, 16]))
    n_pages = int(rng.integers(40, 120))
    free0 = rng.permutation(np.arange(2, n_pages)).astype(np.int32)
    cc, co = cb.PrefixCache(n_pages, free0), O.PrefixCache(n_pages, free0.tolist())
    bases = [rng.integers(0, 1000, 6 * P).astype(np.int32) for _ in range(3)]
    prompts, reqs_c, reqs_o = {}, [], []
    next_id = 0
    budget = int(rng.integers(P, 6 * P))
    pools = [{"ring_len": 0, "window_left": -1, "pool_pages": n_pages - 2, "free_pages": np.zeros(0, np.int32)}]
    matched_any = False
    for step in range(14):
        for _ in range(int(rng.integers(0, 3))):            # arrivals
            b = bases[int(rng.integers(0, 3))]
            head = b[:int(rng.integers(0, len(b) + 1))]
            prompt = np.concatenate([head, rng.integers(0, 1000, int(rng.integers(1, 3 * P)))]).astype(np.int32)
            prompts[next_id] = prompt
            for lst in (reqs_c, reqs_o):
                lst.append(cb.Request(next_id, WAIT, 0, len(prompt), [np.zeros(0, np.int32)]))
            next_id += 1
        hashes = [O.block_hashes(prompts[r.id], P) for r in reqs_c]
        sc = cb.build_metadata(reqs_c, pools, budget, 8, P, 0.1, 0, prefix_cache=cc, prompt_hashes=hashes)
        so = S.build_metadata(reqs_o, pools, budget, 8, P, 0.1, 0, prefix_cache=co, prompt_hashes=hashes)
        assert (sc["status"] == 0) == (so["status"] == "ok") or (sc["status"] == 2 and so["status"] == "nospace")
        if so["status"] == "inval":
            break
        for key in ("query_start_loc", "seq_lens", "req_index", "matched_tokens", "stalled"):
            assert np.array_equal(sc[key], so[key]), (seed, step, key)
        assert sc["first_rejected"] == so["first_rejected"] and sc["held_by_margin"] == so["held_by_margin"]
        for key in ("block_table", "slot_mapping"):
            assert np.array_equal(sc["layers"][0][key], so["layers"][0][key]), (seed, step, key)
        assert sc["layers"][0]["used_pages"] == so["layers"][0]["used_pages"]
        matched_any |= bool(np.any(so["matched_tokens"] > 0))
        reqs_c, _ = cb.advance(reqs_c, sc, [np.zeros(0, np.int32)], [0], P, cc, hashes)
        reqs_o, _ = S.advance(reqs_o, so, [np.zeros(0, np.int32)], P, co, hashes)
        assert _cache_state(cc, n_pages, True) == _cache_state(co, n_pages, False), (seed, step)
        # a decoding request finishes now and then: its pages go back (shared ones stay with their other holders)
        done = [k for k, r in enumerate(reqs_c) if r.state == DEC and rng.random() < 0.3]
        for k in sorted(done, reverse=True):
            pages = reqs_c[k].pages[0]
            cc.release(pages)
            assert co.release([int(p) for p in pages])
            del reqs_c[k], reqs_o[k]
        assert _cache_state(cc, n_pages, True) == _cache_state(co, n_pages, False), (seed, step, "release")
    assert next_id > 0
    assert matched_any, "the random loop never shared a prefix"
