// Prefix cache: page sharing between requests with a common prompt prefix (Transformers "continuous batching
// architecture" page, sections "前缀缓存" (prefix cache) and "驱逐" (eviction)).
//
// Every full block of a prompt is identified by a chain hash of its tokens and everything before it. A request whose
// leading blocks are cached reuses their pages and skips the prefill of those tokens. Pages carry reference counts
// and go back to a free list only when the last request holding them releases them. A released page that holds a
// hashed block stays "initialized": its content and hash are kept, so a later matching prefix can still reuse it.
// Fresh pages come from the uninitialized free list first; when it runs dry, the most recently freed initialized
// page is demoted (its hash dropped) and handed out instead.
//
// Host only, deterministic, no RNG. The caller owns the token and hash arrays; the cache owns its bookkeeping.

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "cb.h"

struct cb_prefix_cache {
    int32_t num_pages = 0;
    std::vector<int32_t> ref;                    // per page: references held by requests
    std::vector<uint8_t> hashed;                 // per page: holds a registered block
    std::vector<uint64_t> hash;                  // per page: that block's hash
    std::deque<int32_t> uninit;                  // free pages without content, taken from the front
    std::vector<int32_t> init_free;              // free pages that keep a hashed block, most recent last
    std::unordered_map<uint64_t, int32_t> index; // block hash -> page
};

namespace {

// FNV-1a, 64-bit (Fowler, Noll, Vo): start from the offset basis, then for every byte xor it in and multiply by the
// FNV prime.
constexpr uint64_t kFnvOffset = 14695981039346656037ull;
constexpr uint64_t kFnvPrime = 1099511628211ull;

inline uint64_t fnv1a_bytes(uint64_t h, const uint8_t *p, size_t n) {
    for (size_t i = 0; i < n; ++i) {
        h ^= p[i];
        h *= kFnvPrime;
    }
    return h;
}

inline uint64_t fnv1a_u64(uint64_t h, uint64_t v) {
    uint8_t b[8];
    for (int i = 0; i < 8; ++i) b[i] = uint8_t(v >> (8 * i));   // little-endian bytes
    return fnv1a_bytes(h, b, 8);
}

inline uint64_t fnv1a_i32(uint64_t h, int32_t v) {
    const uint32_t u = uint32_t(v);
    uint8_t b[4];
    for (int i = 0; i < 4; ++i) b[i] = uint8_t(u >> (8 * i));
    return fnv1a_bytes(h, b, 4);
}

bool valid_page(const cb_prefix_cache *c, int32_t p) { return p >= 0 && p < c->num_pages; }

}  // namespace

extern "C" uint64_t cb_fnv1a64(const void *data, int64_t n) {
    if (!data || n <= 0) return kFnvOffset;
    return fnv1a_bytes(kFnvOffset, static_cast<const uint8_t *>(data), size_t(n));
}

extern "C" cb_status cb_block_hashes(const int32_t *tokens, int32_t n_tokens, int32_t page_size, uint64_t *out) {
    if (n_tokens < 0 || page_size < 1 || (n_tokens > 0 && !tokens)) return CB_E_INVAL;
    const int32_t blocks = n_tokens / page_size;
    if (blocks > 0 && !out) return CB_E_INVAL;
    uint64_t prev = kFnvOffset;
    for (int32_t b = 0; b < blocks; ++b) {
        uint64_t h = fnv1a_u64(kFnvOffset, prev);
        for (int32_t j = 0; j < page_size; ++j) h = fnv1a_i32(h, tokens[int64_t(b) * page_size + j]);
        out[b] = h;
        prev = h;
    }
    return CB_OK;
}

extern "C" cb_status cb_pcache_create(int32_t num_pages, const int32_t *free_pages, int32_t n_free,
                                      cb_prefix_cache **out) {
    if (!out || num_pages < 1 || n_free < 0 || (n_free > 0 && !free_pages)) return CB_E_INVAL;
    *out = nullptr;
    std::vector<uint8_t> seen(size_t(num_pages), 0);
    for (int32_t i = 0; i < n_free; ++i) {
        const int32_t p = free_pages[i];
        if (p < 0 || p >= num_pages || seen[size_t(p)]) return CB_E_INVAL;
        seen[size_t(p)] = 1;
    }
    cb_prefix_cache *c = new (std::nothrow) cb_prefix_cache();
    if (!c) return CB_E_CAPACITY;
    c->num_pages = num_pages;
    c->ref.assign(size_t(num_pages), 0);
    c->hashed.assign(size_t(num_pages), 0);
    c->hash.assign(size_t(num_pages), 0);
    c->uninit.assign(free_pages, free_pages + n_free);
    *out = c;
    return CB_OK;
}

extern "C" void cb_pcache_destroy(cb_prefix_cache *c) { delete c; }

extern "C" cb_status cb_pcache_match(cb_prefix_cache *c, const uint64_t *hashes, int32_t n_blocks, int32_t *pages_out,
                                     int32_t *n_matched) {
    if (!c || n_blocks < 0 || (n_blocks > 0 && (!hashes || !pages_out)) || !n_matched) return CB_E_INVAL;
    int32_t m = 0;
    for (; m < n_blocks; ++m) {
        const auto it = c->index.find(hashes[m]);
        if (it == c->index.end()) break;
        const int32_t p = it->second;
        if (c->ref[size_t(p)] == 0) {   // a freed block comes back into use
            auto &f = c->init_free;
            f.erase(std::find(f.begin(), f.end(), p));
        }
        ++c->ref[size_t(p)];
        pages_out[m] = p;
    }
    *n_matched = m;
    return CB_OK;
}

extern "C" cb_status cb_pcache_lookup(const cb_prefix_cache *c, const uint64_t *hashes, int32_t n_blocks,
                                      int32_t *pages_out, int32_t *n_found, int32_t *n_free_found) {
    if (!c || n_blocks < 0 || (n_blocks > 0 && (!hashes || !pages_out))) return CB_E_INVAL;
    int32_t m = 0, free_hits = 0;
    for (; m < n_blocks; ++m) {
        const auto it = c->index.find(hashes[m]);
        if (it == c->index.end()) break;
        pages_out[m] = it->second;
        if (c->ref[size_t(it->second)] == 0) ++free_hits;
    }
    if (n_found) *n_found = m;
    if (n_free_found) *n_free_found = free_hits;
    return CB_OK;
}

extern "C" cb_status cb_pcache_allocate(cb_prefix_cache *c, int32_t n, int32_t *pages_out) {
    if (!c || n < 0 || (n > 0 && !pages_out)) return CB_E_INVAL;
    if (int64_t(c->uninit.size()) + int64_t(c->init_free.size()) < n) return CB_E_NOSPACE;
    for (int32_t i = 0; i < n; ++i) {
        int32_t p;
        if (!c->uninit.empty()) {
            p = c->uninit.front();
            c->uninit.pop_front();
        } else {   // lazily demote the most recently freed initialized page
            p = c->init_free.back();
            c->init_free.pop_back();
            c->index.erase(c->hash[size_t(p)]);
            c->hashed[size_t(p)] = 0;
        }
        c->ref[size_t(p)] = 1;
        pages_out[i] = p;
    }
    return CB_OK;
}

extern "C" cb_status cb_pcache_commit(cb_prefix_cache *c, int32_t page, uint64_t hash) {
    if (!c || !valid_page(c, page) || c->ref[size_t(page)] < 1 || c->hashed[size_t(page)]) return CB_E_INVAL;
    if (c->index.count(hash)) return CB_OK;   // the block is already cached elsewhere: this page stays private
    c->index.emplace(hash, page);
    c->hashed[size_t(page)] = 1;
    c->hash[size_t(page)] = hash;
    return CB_OK;
}

extern "C" cb_status cb_pcache_release(cb_prefix_cache *c, const int32_t *pages, int32_t n) {
    if (!c || n < 0 || (n > 0 && !pages)) return CB_E_INVAL;
    // validate first (a page may appear several times if the caller holds several references)
    std::unordered_map<int32_t, int32_t> count;
    for (int32_t i = 0; i < n; ++i) {
        if (!valid_page(c, pages[i])) return CB_E_INVAL;
        if (++count[pages[i]] > c->ref[size_t(pages[i])]) return CB_E_INVAL;
    }
    for (int32_t i = 0; i < n; ++i) {
        const int32_t p = pages[i];
        if (--c->ref[size_t(p)] > 0) continue;
        if (c->hashed[size_t(p)])
            c->init_free.push_back(p);
        else
            c->uninit.push_back(p);
    }
    return CB_OK;
}

extern "C" cb_status cb_pcache_stats(const cb_prefix_cache *c, int32_t *n_uninit, int32_t *n_init_free,
                                     int32_t *n_hashed) {
    if (!c || !n_uninit || !n_init_free || !n_hashed) return CB_E_INVAL;
    *n_uninit = int32_t(c->uninit.size());
    *n_init_free = int32_t(c->init_free.size());
    *n_hashed = int32_t(c->index.size());
    return CB_OK;
}

extern "C" cb_status cb_pcache_page_info(const cb_prefix_cache *c, int32_t page, int32_t *ref, int32_t *hashed,
                                         uint64_t *hash) {
    if (!c || !valid_page(c, page) || !ref || !hashed || !hash) return CB_E_INVAL;
    *ref = c->ref[size_t(page)];
    *hashed = c->hashed[size_t(page)];
    *hash = c->hashed[size_t(page)] ? c->hash[size_t(page)] : 0;
    return CB_OK;
}
