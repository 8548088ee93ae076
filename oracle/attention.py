"""Plain fp64 CPU attention for one mixed continuous-batching step -- test infrastructure only.

Nothing here is part of the product. Only the tests, the package's smoke check and the benchmark's CPU-baseline leg
may import it. It shares no code with the HIP path.

What is computed (the definition, written out):

* Ragged batch. Query rows of all requests are concatenated; request r owns rows query_start_loc[r] ..
  query_start_loc[r+1]-1 ("Continuous Batching" blog, languisher.top, sections "Attention Mask 构造实现" and
  "优化：偏移实现 Mask": a block-diagonal causal mask over the concatenated tokens, realised with per-request
  offsets instead of a (T,T) matrix).
* Context. seq_lens[r] counts every key of request r after this step; context_len = seq_len - q_len keys were
  computed in earlier steps; row i of the request sits at position context_len + i and sees keys up to that
  position, itself included (same blog, section "扩展：vLLM v1 中的实现": max_kv_pos = context_len + local_q,
  loop kv_pos <= max_kv_pos).
* Paging. Key kv_pos of request r lives in physical block block_table[r][kv_pos / BLOCK_SIZE] at offset
  kv_pos % BLOCK_SIZE (same section; worked example C = [7, 18], BLOCK_SIZE 2, kv_pos 1 -> block 7 offset 1).
* Sliding layers keep only recent keys in a few reused pages (Transformers "continuous batching architecture" page,
  memory-management section). Reading: key kv_pos is visible to position pos iff pos - window_left <= kv_pos <= pos,
  and a ring of R pages stores logical page b in ring slot b mod R.
* Grouped heads: query head h reads kv head h // (Hq / Hkv) (the pages never mention GQA; contiguous grouping is
  the reading taken).
* Per row and head: s_j = scale * <q, k_j>, p = softmax(s) over the visible keys, out = sum_j p_j v_j (the blog's
  kernel sketch: "score = dot(Q, K); softmax accumulate V").

Every helper that encodes one of these rules is a small named function, so a test can plant a mistake in exactly
one rule and check that a pin notices.
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------------------------------------- rules


def visible_range(pos: int, window_left: int):
    """Inclusive [lo, hi] of key positions visible to a query at `pos` (causal; optional sliding window)."""
    lo = 0 if window_left < 0 else max(0, pos - window_left)
    return lo, pos


def kv_head_of(h: int, group: int) -> int:
    """KV head read by query head h when `group` query heads share one kv head."""
    return h // group


def page_of(kv_pos: int, page_size: int):
    """(logical block, offset in block) of a key position."""
    return kv_pos // page_size, kv_pos % page_size


def physical_page(table_row, logical_block: int, ring_len: int = 0) -> int:
    """Physical page of a logical block: direct lookup, or ring slot logical_block mod ring_len."""
    if ring_len > 0:
        return int(table_row[logical_block % ring_len])
    return int(table_row[logical_block])


def softmax(s: np.ndarray) -> np.ndarray:
    """Softmax over the last axis, fp64, with the row maximum subtracted first."""
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


# ------------------------------------------------------------------------------------------------ the definition


def attend(q, k, v, context_len: int, scale: float, window_left: int = -1):
    """Attention of one request's query rows over its own keys, in logical (contiguous) position order.

    q: [q_len, Hq, D]; k, v: [context_len + q_len, Hkv, D] with row j holding key position j.
    Returns fp64 [q_len, Hq, D]. Row i sits at position context_len + i.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    q_len, Hq, D = q.shape
    Hkv = k.shape[1]
    group = Hq // Hkv
    out = np.zeros((q_len, Hq, D), dtype=np.float64)
    for i in range(q_len):
        pos = context_len + i
        lo, hi = visible_range(pos, window_left)
        for h in range(Hq):
            g = kv_head_of(h, group)
            s = scale * (k[lo:hi + 1, g, :] @ q[i, h, :])
            p = softmax(s)
            out[i, h, :] = p @ v[lo:hi + 1, g, :]
    return out


def attend_rows(q_rows, k, v, key_base: int, positions, scale: float, window_left: int = -1):
    """`attend` for selected query rows given by absolute positions.

    q_rows: [n, Hq, D] (row n sits at positions[n]); k, v: [m, Hkv, D] with row j holding key position key_base + j,
    covering at least every key visible to the given rows.
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n_rows, Hq, D = q_rows.shape
    group = Hq // k.shape[1]
    out = np.zeros((n_rows, Hq, D), dtype=np.float64)
    for n, pos in enumerate(positions):
        lo, hi = visible_range(int(pos), window_left)
        a, b = lo - key_base, hi - key_base + 1
        for h in range(Hq):
            g = kv_head_of(h, group)
            s = scale * (k[a:b, g, :] @ q_rows[n, h, :])
            out[n, h, :] = softmax(s) @ v[a:b, g, :]
    return out


# ------------------------------------------------------------------------------------- the paged cache (logical)
#
# The oracle keeps a cache as [num_pages, page_size, Hkv, D]: the pages' k_cache[physical_block][block_offset]
# order with heads and head_dim appended. It never needs the GPU library's byte layout.


def gather(cache, table_row, positions, page_size: int, ring_len: int = 0):
    """Rows of `cache` for logical key positions `positions` of one request, via its block table (or ring)."""
    out = np.empty((len(positions),) + cache.shape[2:], dtype=cache.dtype)
    for n, kv_pos in enumerate(positions):
        blk, off = page_of(int(kv_pos), page_size)
        out[n] = cache[physical_page(table_row, blk, ring_len), off]
    return out


def slot_of(table_row, kv_pos: int, page_size: int, ring_len: int = 0) -> int:
    """Flat cache slot (page * page_size + offset) where key position kv_pos of a request is written."""
    blk, off = page_of(kv_pos, page_size)
    return physical_page(table_row, blk, ring_len) * page_size + off


def kv_append(k_cache, v_cache, k_new, v_new, slot_mapping, page_size: int):
    """Write token t's K/V rows into slot slot_mapping[t] (page = slot // page_size, offset = slot % page_size).

    Tokens with a negative slot are skipped. Copies are exact (no arithmetic on the values).
    """
    for t, slot in enumerate(np.asarray(slot_mapping)):
        slot = int(slot)
        if slot < 0:
            continue
        page, off = slot // page_size, slot % page_size
        k_cache[page, off] = k_new[t]
        v_cache[page, off] = v_new[t]


def copy_pages(dst, dst_pages, src, src_pages):
    """Whole-page copies: page i goes from src[src_pages[i]] to dst[dst_pages[i]] (None stands for i). Pairs with an
    index outside its array are skipped. This is the offloading copy of the Transformers "continuous batching
    architecture" page (section "Offloading"): a request's KV blocks moved to a swap buffer and back, unchanged."""
    n = len(src_pages) if src_pages is not None else (len(dst_pages) if dst_pages is not None
                                                     else min(len(dst), len(src)))
    for i in range(n):
        sp = int(src_pages[i]) if src_pages is not None else i
        dp = int(dst_pages[i]) if dst_pages is not None else i
        if 0 <= sp < len(src) and 0 <= dp < len(dst):
            dst[dp] = src[sp]


def paged_attention(q, k_cache, v_cache, query_start_loc, seq_lens, block_table, page_size: int, scale: float,
                    window_left: int = -1, ring_len=None, rows=None):
    """Attention of every query row of a ragged step, reading K/V through the block table (or ring).

    q: [T, Hq, D]; caches [num_pages, page_size, Hkv, D]; query_start_loc [N+1]; seq_lens [N];
    block_table [N, width]; ring_len [N] or None. Returns fp64 [T, Hq, D] (rows not in `rows`, if given, are 0).
    """
    q = np.asarray(q, dtype=np.float64)
    T = q.shape[0]
    out = np.zeros(q.shape, dtype=np.float64)
    qsl = np.asarray(query_start_loc)
    wanted = None if rows is None else set(int(t) for t in rows)
    for r in range(len(seq_lens)):
        qs, qe = int(qsl[r]), int(qsl[r + 1])
        q_len = qe - qs
        if q_len == 0:
            continue
        ctx = int(seq_lens[r]) - q_len
        rl = 0 if ring_len is None else int(ring_len[r])
        local = [i for i in range(q_len) if wanted is None or (qs + i) in wanted]
        if not local:
            continue
        top = ctx + max(local)
        lo = visible_range(ctx + min(local), window_left)[0]
        pos = np.arange(lo, top + 1)
        kk = gather(k_cache, block_table[r], pos, page_size, rl)
        vv = gather(v_cache, block_table[r], pos, page_size, rl)
        res = attend_rows(q[[qs + i for i in local]], kk, vv, lo, [ctx + i for i in local], scale, window_left)
        for n, i in enumerate(local):
            out[qs + i] = res[n]
    assert out.shape[0] == T
    return out


# ---------------------------------------------------------------------------------------- brute-force reference


def block_diagonal_causal_mask(query_start_loc):
    """Explicit (T, T) mask of a pure-prefill ragged batch: token a may attend token b iff both belong to the same
    request and b is not after a (the blog's block-diagonal causal mask, before the offset optimisation)."""
    qsl = np.asarray(query_start_loc)
    T = int(qsl[-1])
    mask = np.zeros((T, T), dtype=bool)
    for r in range(len(qsl) - 1):
        for a in range(int(qsl[r]), int(qsl[r + 1])):
            for b in range(int(qsl[r]), a + 1):
                mask[a, b] = True
    return mask


def masked_attention(q, k, v, mask, scale: float):
    """Dense attention of every query row over every key row under an explicit boolean mask [Tq, Tk].

    q: [Tq, Hq, D]; k, v: [Tk, Hkv, D]. Fully-masked rows return 0.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Tq, Hq, D = q.shape
    group = Hq // k.shape[1]
    out = np.zeros((Tq, Hq, D))
    for h in range(Hq):
        g = kv_head_of(h, group)
        s = scale * (q[:, h, :] @ k[:, g, :].T)
        s = np.where(mask, s, -np.inf)
        for a in range(Tq):
            if mask[a].any():
                out[a, h] = softmax(s[a]) @ v[:, g, :]
    return out
