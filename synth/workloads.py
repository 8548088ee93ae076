"""Seeded synthetic workloads for one mixed continuous-batching step.

This module only *draws* inputs: request lists (state, computed and pending token counts), shuffled page pools,
the pages each admitted request already owns, and the random Q/K/V values of every token position. It holds none
of the method's arithmetic -- no scheduling, no position-to-page mapping, no attention. Both the HIP-side harness and
the CPU oracle read their inputs here and nowhere else.

Value streams are counter-addressed: the values of tensor `q`/`k`/`v` for request r at token positions
[256*b, 256*b + 256) come from their own PCG64 stream seeded by (seed, layer, tensor, request, b). Any range of
positions can therefore be regenerated on its own, in any order, by either side.

The five workloads follow the shapes the continuous-batching pages describe: the A/B/C ragged example of the
"Continuous Batching" blog (languisher.top, section on building the mask with offsets), a decode-only step, a FIFO
mixed step under a token budget (Transformers "continuous batching architecture" page, sections on chunked prefill
and the FIFO scheduler), a large log-normal decode batch over a pool with reserved padding pages (same page, memory
management section), and a hybrid full + sliding-window layer pair (same page, sliding layers reuse a few pages).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

DECODING, PREFILLING, WAITING = 0, 1, 2
STATE_NAMES = {DECODING: "decoding", PREFILLING: "prefilling", WAITING: "waiting"}

_TENSOR_ID = {"q": 1, "k": 2, "v": 3}
_BLOCK = 256  # token positions per independent value stream


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32 holding bf16-exact values."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-exact."""
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


@dataclass
class LayerSpec:
    """One attention layer type of the step and the page pool its KV lives in."""
    name: str                 # "full" or "sliding"
    layer_id: int             # value-stream id of this layer
    window_left: int          # -1: full attention; else keys pos-window_left .. pos are visible
    ring_len: int             # 0: pages grow with the sequence; >0: each request owns a ring of this many pages
    num_pages: int            # physical pages in the pool, padding pages included
    padding_pages: tuple      # page ids reserved for padded reads/writes; never handed to a request
    free_pages: np.ndarray    # int32, the pool's free pages in allocation order (already shuffled)


@dataclass
class Request:
    id: int
    state: int                # DECODING / PREFILLING / WAITING
    num_computed: int         # tokens whose K/V are already in the cache (context before this step)
    num_pending: int          # tokens to feed: 1 for a decode, the rest of the prompt otherwise
    pages: List[np.ndarray] = field(default_factory=list)   # per layer: owned pages in logical order


@dataclass
class Workload:
    name: str
    index: int
    seed: int
    dtype: str                # "f32" or "bf16"
    Hq: int
    Hkv: int
    D: int
    page_size: int
    scale: float
    max_batch_tokens: int
    max_requests: int
    safety_margin: float
    layers: List[LayerSpec]
    requests: List[Request]
    description: str = ""
    policy: str = "fifo"      # scheduling policy of the step: "fifo" or "prefill_first"

    # ------------------------------------------------------------------ values
    def values(self, tensor: str, r: int, layer: int, lo: int, hi: int) -> np.ndarray:
        """float32 [hi-lo, H, D] values of `tensor` for request index r at positions [lo, hi).

        N(0,1) draws, rounded to bf16 for bf16 workloads. H is Hq for "q" and Hkv for "k"/"v".
        """
        H = self.Hq if tensor == "q" else self.Hkv
        out = np.empty((max(hi - lo, 0), H, self.D), dtype=np.float32)
        if hi <= lo:
            return out
        req_id = self.requests[r].id
        b0, b1 = lo // _BLOCK, (hi - 1) // _BLOCK
        for b in range(b0, b1 + 1):
            rng = np.random.default_rng([self.seed, self.layers[layer].layer_id, _TENSOR_ID[tensor], req_id, b])
            blk = rng.standard_normal((_BLOCK, H, self.D), dtype=np.float32)
            s, e = max(lo, b * _BLOCK), min(hi, (b + 1) * _BLOCK)
            out[s - lo:e - lo] = blk[s - b * _BLOCK:e - b * _BLOCK]
        if self.dtype == "bf16":
            out = round_to_bf16(out)
        return out

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def summary(self) -> dict:
        st = [rq.state for rq in self.requests]
        return {
            "workload": self.name, "requests": len(self.requests),
            "decoding": st.count(DECODING), "prefilling": st.count(PREFILLING), "waiting": st.count(WAITING),
            "Hq": self.Hq, "Hkv": self.Hkv, "D": self.D, "dtype": self.dtype, "page_size": self.page_size,
            "max_batch_tokens": self.max_batch_tokens,
            "layers": [(l.name, l.window_left, l.ring_len, l.num_pages) for l in self.layers],
        }


# ---------------------------------------------------------------------------------------------------------------
# pool construction helpers (random draws only)

def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def _make_pool(rng, n_alloc: int, n_padding: int):
    """Shuffled allocatable page ids n_padding .. n_padding+n_alloc-1; ids 0..n_padding-1 are padding pages."""
    ids = np.arange(n_padding, n_padding + n_alloc, dtype=np.int32)
    return rng.permutation(ids).astype(np.int32)


def _assign(reqs, layer_idx, counts, order):
    """Hand each request the next `counts[i]` pages of the shuffled `order`; return the rest (the free list)."""
    pos = 0
    for rq, c in zip(reqs, counts):
        rq.pages[layer_idx] = order[pos:pos + c].copy()
        pos += c
    return order[pos:].copy()


def ring_pages_needed(window_left: int, max_chunk: int, page_size: int) -> int:
    """Smallest ring that holds every key a chunk of up to `max_chunk` queries can still see, plus the chunk itself.

    Queries of one step sit at positions ctx..ctx+q-1 and see back to ctx-window_left; those
    window_left+q positions may straddle one extra partial page at each end.
    """
    return (window_left + max_chunk + page_size - 2) // page_size + 1


def _full_layer(rng, reqs, P, pool_factor=None, pool_frac=None, n_padding=2, layer_id=0):
    """Full-attention pool: each admitted request owns ceil(num_computed/P) pages; the rest are free.

    The pool is sized from every request's full length (computed + pending tokens), times `pool_factor`, or so that
    those pages fill a fraction `pool_frac` of it.
    """
    hist = [_cdiv(rq.num_computed, P) for rq in reqs]
    need = sum(_cdiv(rq.num_computed + rq.num_pending, P) for rq in reqs)
    if pool_frac is not None:
        n_alloc = _cdiv(need * 100, int(round(pool_frac * 100)))
    else:
        n_alloc = int(math.ceil(pool_factor * need))
    n_alloc = max(n_alloc, need)
    order = _make_pool(rng, n_alloc, n_padding)
    free = _assign(reqs, layer_id, hist, order)
    return LayerSpec("full", 0, -1, 0, n_alloc + n_padding, tuple(range(n_padding)), free)


def _sliding_layer(rng, reqs, P, window_left, ring_len, pool_factor, n_padding=2, layer_idx=1):
    """Sliding pool: every admitted request owns a ring of `ring_len` pages; waiting requests own none yet."""
    hist = [ring_len if rq.state != WAITING else 0 for rq in reqs]
    need = ring_len * len(reqs)
    n_alloc = int(math.ceil(pool_factor * need))
    order = _make_pool(rng, n_alloc, n_padding)
    free = _assign(reqs, layer_idx, hist, order)
    return LayerSpec("sliding", 1, window_left, ring_len, n_alloc + n_padding, tuple(range(n_padding)), free)


# ---------------------------------------------------------------------------------------------------------------
# the five workloads (and reduced "mini" variants the oracle finishes in seconds)

def _decodes(rng, n, ctx_lo, ctx_hi, id0=0):
    ctx = rng.integers(ctx_lo, ctx_hi + 1, size=n)
    return [Request(id0 + i, DECODING, int(c), 1, []) for i, c in enumerate(ctx)]


def workload_1(seed: int = 1001) -> Workload:
    """A/B/C ragged prefill of 4, 2 and 3 new tokens; 32 pages of 2 tokens; C's pages forced to [7, 18]."""
    rng = np.random.default_rng(seed)
    reqs = [Request(0, WAITING, 0, 4, [None]), Request(1, WAITING, 0, 2, [None]), Request(2, WAITING, 0, 3, [None])]
    perm = rng.permutation(32).astype(np.int32)
    rest = perm[(perm != 7) & (perm != 18)]
    # allocation order: A takes two pages, B one, then C gets 7 and 18
    free = np.concatenate([rest[:3], np.array([7, 18], np.int32), rest[3:]]).astype(np.int32)
    for rq in reqs:
        rq.pages = [np.zeros(0, np.int32)]
    layer = LayerSpec("full", 0, -1, 0, 32, (), free)
    return Workload("tiny ragged prefill A/B/C (3 req: 4+2+3 tokens, 2 heads, D64, fp32, page 2)", 1, seed,
                    "f32", 2, 2, 64, 2, 1.0 / math.sqrt(64), 64, 64, 0.0, [layer], reqs)


def workload_2(seed: int = 1002, n=64, ctx_lo=128, ctx_hi=4096, heads=(32, 8), D=128, P=16, name=None) -> Workload:
    """Decode-only step: n requests, one new token each, context uniform in [ctx_lo, ctx_hi]."""
    rng = np.random.default_rng(seed)
    reqs = _decodes(rng, n, ctx_lo, ctx_hi)
    for rq in reqs:
        rq.pages = [None]
    layer = _full_layer(rng, reqs, P, pool_factor=1.25)
    return Workload(name or f"decode-only step ({n} req, ctx U[{ctx_lo},{ctx_hi}], {heads[0]}q/{heads[1]}kv, D{D}, "
                    f"bf16, page {P})", 2, seed, "bf16", heads[0], heads[1], D, P, 1.0 / math.sqrt(D),
                    max(2048, n), max(256, n), 0.0, [layer], reqs)


def workload_3(seed: int = 1003, n_dec=96, dec_ctx=(256, 8192), cont=((1536, 1024), (3584, 3072)), new_prompt=2000,
               budget=2048, heads=(32, 8), D=128, P=16, name=None) -> Workload:
    """Mixed FIFO step: n_dec decodes, continuing prefills (prompt, computed), one new prompt; token budget."""
    rng = np.random.default_rng(seed)
    reqs = _decodes(rng, n_dec, dec_ctx[0], dec_ctx[1])
    rid = n_dec
    for prompt, done in cont:
        reqs.append(Request(rid, PREFILLING, done, prompt - done, []))
        rid += 1
    reqs.append(Request(rid, WAITING, 0, new_prompt, []))
    for rq in reqs:
        rq.pages = [None]
    layer = _full_layer(rng, reqs, P, pool_factor=1.25)
    return Workload(name or f"mixed chunked-prefill step (max_batch_tokens {budget}: {n_dec} decodes ctx "
                    f"U[{dec_ctx[0]},{dec_ctx[1]}], {len(cont)} continuing chunks, 1 new prompt; "
                    f"{heads[0]}q/{heads[1]}kv, D{D}, bf16, page {P})", 3, seed, "bf16", heads[0], heads[1], D, P,
                    1.0 / math.sqrt(D), budget, 256, 0.0, [layer], reqs)


def workload_4(seed: int = 1004, n=256, median=2048, sigma=1.0, clip=(64, 32768), heads=(64, 8), D=128, P=16,
               occupancy=0.6, name=None) -> Workload:
    """Large decode batch with log-normal contexts over a ~60%-occupied shuffled pool with 2 padding pages."""
    rng = np.random.default_rng(seed)
    ctx = np.clip(np.round(np.exp(rng.normal(math.log(median), sigma, size=n))), clip[0], clip[1]).astype(int)
    reqs = [Request(i, DECODING, int(c), 1, [None]) for i, c in enumerate(ctx)]
    layer = _full_layer(rng, reqs, P, pool_frac=occupancy)
    return Workload(name or f"large decode batch ({n} req, log-normal ctx median {median} sigma {sigma} clip "
                    f"[{clip[0]},{clip[1]}], {heads[0]}q/{heads[1]}kv, D{D}, bf16, page {P}, pool "
                    f"{int(occupancy * 100)}% occupied + 2 padding pages)", 4, seed, "bf16", heads[0], heads[1], D, P,
                    1.0 / math.sqrt(D), max(2048, n), max(256, n), 0.0, [layer], reqs)


def workload_5(seed: int = 1005, n_dec=128, dec_ctx=(256, 32768), cont=((6144, 4096), (14336, 12288), (18432, 16384)),
               new_prompt=4000, budget=8192, window_left=4096, heads=(32, 8), D=128, P=32, name=None) -> Workload:
    """Hybrid layer pair over one mixed step: a full layer (block tables) and a sliding layer (page rings)."""
    rng = np.random.default_rng(seed)
    reqs = _decodes(rng, n_dec, dec_ctx[0], dec_ctx[1])
    rid = n_dec
    for prompt, done in cont:
        reqs.append(Request(rid, PREFILLING, done, prompt - done, []))
        rid += 1
    reqs.append(Request(rid, WAITING, 0, new_prompt, []))
    for rq in reqs:
        rq.pages = [None, None]
    full = _full_layer(rng, reqs, P, pool_factor=1.25)
    ring = ring_pages_needed(window_left, budget, P)
    sliding = _sliding_layer(rng, reqs, P, window_left, ring, pool_factor=1.25)
    return Workload(name or f"hybrid full + sliding-window layer pair (max_batch_tokens {budget}: {n_dec} decodes ctx "
                    f"U[{dec_ctx[0]},{dec_ctx[1]}], {len(cont)} continuing chunks, 1 new prompt; window {window_left}; "
                    f"{heads[0]}q/{heads[1]}kv, D{D}, bf16, page {P})", 5, seed, "bf16", heads[0], heads[1], D, P,
                    1.0 / math.sqrt(D), budget, 256, 0.0, [full, sliding], reqs)


def make_workload(index: int, mini: bool = False, seed: Optional[int] = None) -> Workload:
    """Workload 1..5 at full size, or its reduced variant (same structure, lengths the oracle finishes in seconds)."""
    if not mini:
        fn = {1: workload_1, 2: workload_2, 3: workload_3, 4: workload_4, 5: workload_5}[index]
        return fn() if seed is None else fn(seed)
    s = (2000 + index) if seed is None else seed
    if index == 1:
        return workload_1(s)
    if index == 2:
        return workload_2(s, n=8, ctx_lo=1, ctx_hi=300, name="decode-only step, reduced (8 req, ctx U[1,300])")
    if index == 3:
        return workload_3(s, n_dec=6, dec_ctx=(20, 400), cont=((150, 70), (260, 200)), new_prompt=300, budget=256,
                          name="mixed chunked-prefill step, reduced (budget 256: 6 decodes, 2 chunks, 1 new prompt)")
    if index == 4:
        return workload_4(s, n=16, median=128, sigma=1.0, clip=(1, 1000),
                          name="large decode batch, reduced (16 req, log-normal ctx median 128, G=8)")
    if index == 5:
        return workload_5(s, n_dec=8, dec_ctx=(1, 700), cont=((400, 200), (600, 500)), new_prompt=300, budget=512,
                          window_left=128,
                          name="hybrid layer pair, reduced (budget 512: 8 decodes, 2 chunks, 1 new prompt, window 128)")
    raise ValueError(index)
