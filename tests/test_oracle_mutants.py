"""Plant one plausible mistake at a time in the oracle and check that at least one pin fails.

A pin set that lets a dropped term, a wrong sign or index, or a transposed operand through would not be a pin; this
file shows, for each rule of the oracle, a wrong version that the pins reject.
"""
import numpy as np
import pytest

import oracle.attention as A
import oracle.scheduler as S
from tests import oracle_checks as C


def _excl_self(pos, wl):
    return (0 if wl < 0 else max(0, pos - wl)), pos - 1


def _window_short(pos, wl):
    return (0 if wl < 0 else max(0, pos - wl + 1)), pos


def _ring_no_mod(table_row, logical_block, ring_len=0):
    return int(table_row[min(logical_block, len(table_row) - 1)])


def _softmax_by_max(s):
    e = np.exp(s - np.max(s, axis=-1, keepdims=True))
    return e / np.max(e, axis=-1, keepdims=True)


def _softmax_double_scale(s):
    s = 2.0 * s
    e = np.exp(s - np.max(s, axis=-1, keepdims=True))
    return e / np.sum(e, axis=-1, keepdims=True)


def _append_k_into_v(k_cache, v_cache, k_new, v_new, slot_mapping, page_size):
    for t, slot in enumerate(np.asarray(slot_mapping)):
        if slot < 0:
            continue
        k_cache[slot // page_size, slot % page_size] = k_new[t]
        v_cache[slot // page_size, slot % page_size] = k_new[t]


_real_advance = S.advance


def _advance_keeps_old_pages(requests, schedule, free_pages, page_size, *a, **k):
    out, free = _real_advance(requests, schedule, free_pages, page_size, *a, **k)
    for new, old in zip(out, requests):
        new.pages = [np.asarray(p, dtype=np.int32).copy() for p in old.pages]
    return out, free


def _advance_free_list_unmoved(requests, schedule, free_pages, page_size, *a, **k):
    out, _ = _real_advance(requests, schedule, free_pages, page_size, *a, **k)
    return out, [np.asarray(f, dtype=np.int32).copy() for f in free_pages]


def _advance_never_decodes(requests, schedule, free_pages, page_size, *a, **k):
    out, free = _real_advance(requests, schedule, free_pages, page_size, *a, **k)
    for new, old in zip(out, requests):
        if new.state == S.DECODING and old.state != S.DECODING:
            new.state = S.PREFILLING
    return out, free


MUTANTS = {
    "causal bound excludes the query itself": (A, "visible_range", _excl_self),
    "sliding window one key short": (A, "visible_range", _window_short),
    "query head mapped to kv head h % G": (A, "kv_head_of", lambda h, g: h % g),
    "block and offset swapped": (A, "page_of", lambda p, P: (p % P, p // P)),
    "ring slot without modulo": (A, "physical_page", _ring_no_mod),
    "softmax normalised by its max": (A, "softmax", _softmax_by_max),
    "scores scaled twice": (A, "softmax", _softmax_double_scale),
    "append writes K into V": (A, "kv_append", _append_k_into_v),
    "page counts rounded down": (S, "_cdiv", lambda a, b: a // b),
    "ring size never checked": (S, "ring_is_large_enough", lambda *a: True),
    "lifecycle keeps the old pages": (S, "advance", _advance_keeps_old_pages),
    "lifecycle leaves the free list unmoved": (S, "advance", _advance_free_list_unmoved),
    "finished prompt never turns to decoding": (S, "advance", _advance_never_decodes),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    mod, attr, fn = MUTANTS[name]
    monkeypatch.setattr(mod, attr, fn)
    caught = None
    for check in C.ALL_CHECKS:
        try:
            check()
        except Exception as e:  # noqa: BLE001 - any failure of a pin counts
            caught = (check.__name__, type(e).__name__)
            break
    assert caught is not None, f"no pin caught the planted mistake: {name}"
