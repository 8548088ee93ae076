"""Plain Python reference of the prefix cache (page sharing by block hash) -- test infrastructure only.

Rules (Transformers "continuous batching architecture" page, sections "前缀缓存" (prefix cache) and "驱逐"
(eviction)):

* Every full block of a prompt gets a content hash. Reading: a chain hash, so that a block is identified by its tokens
  and everything before it -- FNV-1a 64-bit over the previous block's hash (8 little-endian bytes; the FNV offset
  basis before the first block) followed by the block's token ids (4 little-endian bytes each).
* A later request whose leading blocks are cached reuses their pages (and skips their prefill).
* Shared pages are reference-counted and go back to the free pool only when every request using them has finished.
* Freed pages are not erased: a page holding a registered block stays "initialized" (content and hash kept) for
  later matches. When the empty pool runs out, the manager lazily demotes the most recent initialized page (reading:
  the most recently freed one) to empty, dropping its hash.
* Fresh pages come from the empty pool in free-list order; allocation is all or nothing.

Nothing here is shared with the library's C++ implementation.
"""
from __future__ import annotations

FNV_OFFSET = 14695981039346656037
FNV_PRIME = 1099511628211
MASK = (1 << 64) - 1


def fnv1a64(data: bytes, h: int = FNV_OFFSET) -> int:
    """FNV-1a, 64-bit: for every byte, xor it in, then multiply by the FNV prime (mod 2^64)."""
    for b in data:
        h = ((h ^ b) * FNV_PRIME) & MASK
    return h


def block_hashes(tokens, page_size: int):
    out = []
    prev = FNV_OFFSET
    n_blocks = len(tokens) // page_size
    for b in range(n_blocks):
        data = prev.to_bytes(8, "little") + b"".join(
            (int(t) & 0xFFFFFFFF).to_bytes(4, "little") for t in tokens[b * page_size:(b + 1) * page_size])
        prev = fnv1a64(data)
        out.append(prev)
    return out


class PrefixCache:
    def __init__(self, num_pages: int, free_pages):
        self.num_pages = num_pages
        self.ref = [0] * num_pages
        self.hash = [None] * num_pages          # registered block hash per page, or None
        self.empty = [int(p) for p in free_pages]
        self.initialized = []                   # freed pages that keep a registered block, oldest first
        self.index = {}                         # block hash -> page

    def match(self, hashes):
        pages = []
        for h in hashes:
            p = self.index.get(int(h))
            if p is None:
                break
            if self.ref[p] == 0:
                self.initialized.remove(p)
            self.ref[p] += 1
            pages.append(p)
        return pages

    def lookup(self, hashes):
        """Pages of the leading blocks of `hashes` that are registered, without taking references."""
        pages = []
        for h in hashes:
            p = self.index.get(int(h))
            if p is None:
                break
            pages.append(p)
        return pages

    def n_free(self) -> int:
        """Pages a fresh allocation can take: empty ones plus initialized ones (which it would demote)."""
        return len(self.empty) + len(self.initialized)

    def allocate(self, n: int):
        if len(self.empty) + len(self.initialized) < n:
            return None                          # no space: nothing taken
        out = []
        for _ in range(n):
            if self.empty:
                p = self.empty.pop(0)
            else:
                p = self.initialized.pop()       # the most recently freed initialized page
                del self.index[self.hash[p]]
                self.hash[p] = None
            self.ref[p] = 1
            out.append(p)
        return out

    def commit(self, page: int, h: int) -> bool:
        if not 0 <= page < self.num_pages or self.ref[page] < 1 or self.hash[page] is not None:
            return False
        if int(h) not in self.index:
            self.index[int(h)] = page
            self.hash[page] = int(h)
        return True

    def release(self, pages) -> bool:
        count = {}
        for p in pages:
            if not 0 <= p < self.num_pages:
                return False
            count[p] = count.get(p, 0) + 1
            if count[p] > self.ref[p]:
                return False
        for p in pages:
            self.ref[p] -= 1
            if self.ref[p] == 0:
                (self.initialized if self.hash[p] is not None else self.empty).append(p)
        return True

    def stats(self):
        return len(self.empty), len(self.initialized), len(self.index)
