"""The prefix cache (page sharing by block hash): the oracle's rules pinned on hand-made cases and the FNV-1a
published test vectors, then the C++ implementation against the oracle on random operation sequences, bit for bit."""
import numpy as np
import pytest

import oracle.prefix_cache as O
import paged_kv_attention_varlen_amd as cb

# FNV-1a 64-bit test vectors published with the algorithm (Fowler/Noll/Vo)
FNV_VECTORS = [(b"", 0xcbf29ce484222325), (b"a", 0xaf63dc4c8601ec8c), (b"foobar", 0x85944171f73967e8)]


@pytest.mark.parametrize("data,want", FNV_VECTORS)
def test_fnv1a_published_vectors(data, want):
    assert O.fnv1a64(data) == want
    lib = cb._abi.load()
    buf = cb.C.create_string_buffer(data, len(data)) if data else None
    assert lib.cb_fnv1a64(buf, len(data)) == want


def test_block_hashes_chain():
    rng = np.random.default_rng(1)
    P = 4
    a = rng.integers(0, 50000, 23).astype(np.int32)
    b = a.copy()
    b[13] += 1                                          # differs inside block 3
    ha, hb = O.block_hashes(a, P), O.block_hashes(b, P)
    assert len(ha) == 5 and ha[:3] == hb[:3] and all(x != y for x, y in zip(ha[3:], hb[3:]))
    # a block's hash depends on what precedes it: the same tokens after a different prefix hash differently
    c = np.concatenate([a[4:8], a[4:8]])
    hc = O.block_hashes(c, P)
    assert hc[0] != hc[1]
    for t in (a, b, c, a[:3], np.zeros(0, np.int32)):
        assert cb.block_hashes(t, P).tolist() == O.block_hashes(t, P)


def test_rules_on_hand_made_cases():
    c = O.PrefixCache(10, [2, 3, 4, 5, 6])
    a = c.allocate(3)
    assert a == [2, 3, 4] and c.stats() == (2, 0, 0)
    for p, h in zip(a[:2], (101, 102)):                 # two full blocks of request A
        assert c.commit(p, h)
    # request B with the same two leading blocks shares A's pages and takes references
    assert c.match([101, 102, 999]) == [2, 3] and c.ref[2] == 2 and c.ref[3] == 2
    # A finishes: the shared pages stay with B; A's private page 4 goes back empty
    assert c.release([2, 3, 4]) and c.ref[2] == 1 and c.stats() == (3, 0, 2)
    # B finishes: its pages are freed but keep their blocks (initialized), most recent last
    assert c.release([3, 2]) and c.stats() == (3, 2, 2) and c.initialized == [3, 2]
    # a later request C matches them again and pulls them out of the free pool
    assert c.match([101]) == [2] and c.initialized == [3]
    assert c.release([2]) and c.initialized == [3, 2]
    # fresh pages: the empty ones first, in order, then the most recently freed initialized page is demoted
    assert c.allocate(4) == [5, 6, 4, 2] and 101 not in c.index and 102 in c.index
    assert c.allocate(2) is None and c.stats() == (0, 1, 1)   # all or nothing
    # a block already registered elsewhere leaves the committing page private
    assert c.commit(5, 102) and c.hash[5] is None
    # releasing more references than held is refused, and changes nothing
    assert not c.release([5, 5]) and c.ref[5] == 1


@pytest.mark.parametrize("seed", range(40))
def test_library_matches_oracle_on_random_operations(seed):
    rng = np.random.default_rng(seed)
    n_pages = int(rng.integers(4, 40))
    free = rng.permutation(n_pages)[:int(rng.integers(1, n_pages + 1))].astype(np.int32)
    ref = O.PrefixCache(n_pages, free)
    lib = cb.PrefixCache(n_pages, free)
    held = []                                            # pages with references, one entry per reference
    hashes = [int(h) for h in rng.integers(1, 2 ** 63, 12, dtype=np.int64)]
    for _ in range(200):
        op = int(rng.integers(0, 4))
        if op == 0:
            n = int(rng.integers(0, 6))
            want = ref.allocate(n)
            if want is None:
                with pytest.raises(cb.CbError):
                    lib.allocate(n)
            else:
                assert lib.allocate(n).tolist() == want
                held += want
        elif op == 1 and held:
            p = int(rng.choice(held))
            h = hashes[int(rng.integers(0, len(hashes)))]
            ok = ref.commit(p, h)
            if ok:
                lib.commit(p, h)
            else:
                with pytest.raises(cb.CbError):
                    lib.commit(p, h)
        elif op == 2:
            k = int(rng.integers(0, 5))
            chain = [hashes[int(i)] for i in rng.integers(0, len(hashes), k)]
            want = ref.match(chain)
            assert lib.match(chain).tolist() == want
            held += want
        elif op == 3 and held:
            k = int(rng.integers(1, min(4, len(held)) + 1))
            pick = [held[int(i)] for i in rng.choice(len(held), k, replace=False)]
            assert ref.release(pick)
            lib.release(pick)
            for p in pick:
                held.remove(p)
        assert lib.stats() == ref.stats()
    for p in range(n_pages):
        refs, reg, h = lib.page_info(p)
        assert refs == ref.ref[p] and reg == (ref.hash[p] is not None) and (h == (ref.hash[p] or 0))
