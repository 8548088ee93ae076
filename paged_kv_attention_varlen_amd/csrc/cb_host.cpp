// Host half of the cb library: the step scheduler (cb_build_metadata) and the work planner (cb_plan_attention).
//
// Both are functions of their arguments only: no allocation visible to the caller, no global state, no RNG. Page
// allocation takes pages from the front of the caller's (already shuffled) free lists -- or, when the caller passes a
// prefix cache, from that cache, whose references the scheduler then takes (the one state it changes).

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <vector>

#include "cb.h"

namespace {

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool is_pow2(int32_t x) { return x > 0 && (x & (x - 1)) == 0; }

// Minimum ring (in pages) for a sliding layer: this step's queries at ctx .. ctx+q-1 still see keys back to
// ctx-window_left, and the step writes keys up to ctx+q-1; those window_left+q positions, arbitrarily aligned,
// touch at most (window_left + q + P - 2) / P + 1 pages, which must all sit in distinct ring slots.
int64_t min_ring_pages(int32_t window_left, int32_t max_chunk, int32_t P) {
    return (int64_t(window_left) + max_chunk + P - 2) / P + 1;
}

// Slot of key position pos of a request whose block-table row (or ring of ring_len pages) is `row`: the physical
// page of logical block pos / P (ring slot (pos / P) mod ring_len), times P, plus the offset pos % P.
inline int64_t slot_of(const int32_t *row, int64_t pos, int32_t P, int32_t ring_len) {
    const int64_t logical = pos / P;
    const int32_t page = row[ring_len > 0 ? logical % ring_len : logical];
    return int64_t(page) * P + pos % P;
}

struct Scheduled {
    int32_t req;                        // index into the caller's request array
    int32_t q;                          // tokens of this step
    int32_t new_from[CB_MAX_LAYERS];    // first index into the layer's free list (or the cache's allocations)
    int32_t new_count[CB_MAX_LAYERS];
    int32_t matched;                    // prompt tokens reused from the prefix cache (whole blocks)
    int32_t match_from;                 // first index of its matched pages in the step's list of matches
    int32_t n_match;                    // matched blocks
};

}  // namespace

extern "C" const char *cb_status_str(cb_status s) {
    switch (s) {
        case CB_OK: return "ok";
        case CB_E_INVAL: return "invalid argument";
        case CB_E_NOSPACE: return "no request could be scheduled: out of free pages";
        case CB_E_CAPACITY: return "output buffer too small";
        case CB_E_UNSUPPORTED: return "unsupported shape or dtype";
        case CB_E_WORKSPACE: return "workspace missing or too small";
        case CB_E_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

extern "C" int32_t cb_abi_version(void) { return CB_ABI_VERSION; }

// ------------------------------------------------------------------------------------------------ scheduler

extern "C" cb_status cb_build_metadata(const cb_req *reqs, int32_t n_reqs, const cb_sched_params *params,
                                       const cb_layer_pool *layers, int32_t *out, int64_t out_capacity,
                                       cb_step *step) {
    if (!params || !layers || !step || n_reqs < 0 || (n_reqs > 0 && !reqs)) return CB_E_INVAL;
    const int32_t P = params->page_size;
    const int32_t L = params->n_layers;
    const int32_t budget0 = params->max_batch_tokens;
    const int32_t cap = params->max_requests;
    if (P < 1 || budget0 < 1 || cap < 1 || L < 1 || L > CB_MAX_LAYERS) return CB_E_INVAL;
    if (params->policy != CB_POLICY_FIFO && params->policy != CB_POLICY_PREFILL_FIRST) return CB_E_INVAL;
    for (int l = 0; l < L; ++l) {
        const cb_layer_pool &lay = layers[l];
        if (lay.ring_len < 0 || lay.n_free < 0 || (lay.n_free > 0 && !lay.free_pages)) return CB_E_INVAL;
        if (lay.ring_len > 0 && (lay.window_left < 0 || lay.ring_len < min_ring_pages(lay.window_left, budget0, P)))
            return CB_E_INVAL;
    }
    for (int32_t i = 0; i < n_reqs; ++i) {
        const cb_req &rq = reqs[i];
        if (rq.state != CB_DECODING && rq.state != CB_PREFILLING && rq.state != CB_WAITING) return CB_E_INVAL;
        if (rq.num_computed < 0 || rq.num_pending < 1) return CB_E_INVAL;
        if (rq.state == CB_DECODING && rq.num_pending != 1) return CB_E_INVAL;
        if (rq.n_prompt_blocks < 0 || (rq.n_prompt_blocks > 0 && !rq.prompt_hashes)) return CB_E_INVAL;
        for (int l = 0; l < L; ++l) {
            if (rq.n_pages[l] < 0 || (rq.n_pages[l] > 0 && !rq.pages[l])) return CB_E_INVAL;
            if (layers[l].ring_len > 0) {
                if (rq.state != CB_WAITING && rq.n_pages[l] != layers[l].ring_len) return CB_E_INVAL;
            } else if (rq.n_pages[l] < ceil_div(rq.num_computed, P)) {
                return CB_E_INVAL;
            }
        }
    }

    // Prefix sharing: only with a cache and one full-attention layer type; then the cache allocates every page.
    cb_prefix_cache *pc = (params->prefix_cache && L == 1 && layers[0].ring_len == 0) ? params->prefix_cache : nullptr;
    if (pc) {
        // the scheduler will change the cache, so the output must be known to fit before anything is scheduled:
        // check against a bound (rows, tokens and table width at their largest)
        const int64_t n_max = std::min<int64_t>(n_reqs, cap);
        int64_t w_max = 0;
        for (int32_t i = 0; i < n_reqs; ++i)
            w_max = std::max<int64_t>(w_max, ceil_div(int64_t(reqs[i].num_computed) +
                                                      std::min(reqs[i].num_pending, budget0), P));
        const int64_t bound = 4 * (n_max + 1) + n_reqs + n_max * w_max + budget0 + n_max;
        if (!out || out_capacity < bound) {
            std::memset(step, 0, sizeof(*step));
            step->used = bound;
            return CB_E_CAPACITY;
        }
    }
    auto cache_free = [&]() -> int64_t {
        int32_t a = 0, b = 0, c = 0;
        cb_pcache_stats(pc, &a, &b, &c);
        return int64_t(a) + b;
    };
    std::vector<int32_t> alloc;          // pages the cache allocated, in scheduling order
    std::vector<int32_t> match_pages;    // pages matched at admission, in scheduling order
    int32_t taken[CB_MAX_LAYERS] = {0, 0};
    auto pages_needed = [&](const cb_req &rq, int32_t q, int32_t *need) {
        for (int l = 0; l < L; ++l) {
            const int64_t want = layers[l].ring_len > 0 ? layers[l].ring_len
                                                        : ceil_div(int64_t(rq.num_computed) + q, P);
            need[l] = int32_t(std::max<int64_t>(0, want - rq.n_pages[l]));
        }
    };
    auto free_of = [&](int l) -> int64_t { return pc ? cache_free() : int64_t(layers[l].n_free) - taken[l]; };
    auto available = [&](const int32_t *need) {
        for (int l = 0; l < L; ++l)
            if (need[l] > free_of(l)) return false;
        return true;
    };

    std::vector<Scheduled> rows[3];   // by state: decodes, continuing prefills, admitted requests
    std::vector<int32_t> stalled;
    int32_t first_rejected = -1;
    int32_t held = 0;
    int32_t budget = budget0;
    auto n_rows = [&]() { return int32_t(rows[0].size() + rows[1].size() + rows[2].size()); };
    auto schedule = [&](int32_t group, int32_t i, int32_t q, const int32_t *need, int32_t n_match = 0,
                        int32_t match_from = 0) {
        Scheduled s{};
        s.req = i;
        s.q = q;
        s.n_match = n_match;
        s.matched = n_match * P;
        s.match_from = match_from;
        for (int l = 0; l < L; ++l) {
            s.new_count[l] = need[l];
            if (pc) {   // one layer type: the cache allocates (availability was checked)
                s.new_from[l] = int32_t(alloc.size());
                alloc.resize(alloc.size() + size_t(need[l]));
                if (need[l] > 0) cb_pcache_allocate(pc, need[l], alloc.data() + s.new_from[l]);
            } else {
                s.new_from[l] = taken[l];
            }
            taken[l] += need[l];
        }
        rows[group].push_back(s);
        budget -= q;
    };

    // active decodes, one token each
    auto decodes = [&]() {
        for (int32_t i = 0; i < n_reqs; ++i) {
            if (reqs[i].state != CB_DECODING) continue;
            if (n_rows() >= cap || budget < 1) break;
            int32_t need[CB_MAX_LAYERS];
            pages_needed(reqs[i], 1, need);
            if (!available(need)) {
                stalled.push_back(i);
                continue;
            }
            schedule(0, i, 1, need);
        }
    };
    // active prefills continue where they stopped
    auto prefills = [&]() {
        for (int32_t i = 0; i < n_reqs; ++i) {
            if (reqs[i].state != CB_PREFILLING) continue;
            if (n_rows() >= cap || budget < 1) break;
            const int32_t q = std::min(reqs[i].num_pending, budget);
            int32_t need[CB_MAX_LAYERS];
            pages_needed(reqs[i], q, need);
            if (!available(need)) {
                stalled.push_back(i);
                continue;
            }
            schedule(1, i, q, need);
        }
    };
    // admission of waiting requests, in arrival order
    auto admit = [&]() {
        for (int32_t i = 0; i < n_reqs; ++i) {
            if (reqs[i].state != CB_WAITING) continue;
            if (n_rows() >= cap || budget < 1) break;
            bool low = false;
            for (int l = 0; l < L; ++l) {
                const cb_layer_pool &lay = layers[l];
                if (lay.pool_pages > 0 &&
                    double(free_of(l)) < double(params->safety_margin) * double(lay.pool_pages))
                    low = true;
            }
            if (low) {
                held = 1;
                break;
            }
            const cb_req &rq = reqs[i];
            int32_t found = 0, free_found = 0;
            if (pc && rq.num_computed == 0 && rq.n_pages[0] == 0 && rq.n_prompt_blocks > 0) {
                // leading cached blocks of the prompt, leaving at least one prompt token to compute
                const int32_t n = std::min(rq.n_prompt_blocks, (rq.num_pending - 1) / P);
                std::vector<int32_t> hit(size_t(std::max(n, 1)));
                cb_pcache_lookup(pc, rq.prompt_hashes, n, hit.data(), &found, &free_found);
            }
            const int32_t q = std::min(rq.num_pending - found * P, budget);
            int32_t need[CB_MAX_LAYERS];
            bool ok;
            if (found > 0) {
                need[0] = int32_t(std::max<int64_t>(0, ceil_div(int64_t(found) * P + q, P) - found));
                ok = need[0] <= free_of(0) - free_found;   // matched free pages leave the free pool
            } else {
                pages_needed(rq, q, need);
                ok = available(need);
            }
            if (!ok) {
                first_rejected = i;
                break;
            }
            const int32_t match_from = int32_t(match_pages.size());
            if (found > 0) {
                match_pages.resize(match_pages.size() + size_t(found));
                int32_t got = 0;
                cb_pcache_match(pc, rq.prompt_hashes, found, match_pages.data() + match_from, &got);
            }
            schedule(2, i, q, need, found, match_from);
        }
    };
    if (params->policy == CB_POLICY_FIFO) {
        decodes();
        prefills();
        admit();
    } else {
        prefills();
        admit();
        decodes();
    }
    std::sort(stalled.begin(), stalled.end());
    const int32_t num_decodes = int32_t(rows[0].size());
    // rows laid out decodes first, then continuing prefills, then admitted requests
    rows[0].insert(rows[0].end(), rows[1].begin(), rows[1].end());
    rows[0].insert(rows[0].end(), rows[2].begin(), rows[2].end());
    const std::vector<Scheduled> &all = rows[0];

    // ---- sizes and offsets of the packed output
    const int32_t N = int32_t(all.size());
    int64_t T = 0;
    int32_t max_q = 0, max_seq = 0;
    for (const Scheduled &s : all) {
        T += s.q;
        max_q = std::max(max_q, s.q);
        max_seq = std::max(max_seq, reqs[s.req].num_computed + s.matched + s.q);
    }
    if (T > INT32_MAX) return CB_E_INVAL;
    std::memset(step, 0, sizeof(*step));
    step->num_reqs = N;
    step->num_tokens = int32_t(T);
    step->num_decodes = num_decodes;
    step->max_q_len = max_q;
    step->max_seq_len = max_seq;
    step->n_stalled = int32_t(stalled.size());
    step->first_rejected = first_rejected;
    step->held_by_margin = held;
    step->prefix_sharing = pc ? 1 : 0;
    int64_t off = 0;
    step->off_query_start_loc = off; off += N + 1;
    step->off_seq_lens = off;        off += N;
    step->off_req_index = off;       off += N;
    step->off_stalled = off;         off += int64_t(stalled.size());
    step->off_matched = off;         off += N;
    for (int l = 0; l < L; ++l) {
        step->used_pages[l] = taken[l];
        const int32_t width = layers[l].ring_len > 0 ? layers[l].ring_len : int32_t(ceil_div(max_seq, P));
        step->table_width[l] = width;
        step->off_block_table[l] = off;  off += int64_t(N) * width;
        step->off_slot_mapping[l] = off; off += T;
        step->off_ring_len[l] = off;     off += N;
    }
    step->used = off;
    if (off > out_capacity || !out) return CB_E_CAPACITY;

    // ---- ragged metadata
    int32_t *qsl = out + step->off_query_start_loc;
    int32_t *seq = out + step->off_seq_lens;
    int32_t *idx = out + step->off_req_index;
    qsl[0] = 0;
    for (int32_t r = 0; r < N; ++r) {
        qsl[r + 1] = qsl[r] + all[r].q;
        seq[r] = reqs[all[r].req].num_computed + all[r].matched + all[r].q;
        idx[r] = all[r].req;
        out[step->off_matched + r] = all[r].matched;
    }
    std::copy(stalled.begin(), stalled.end(), out + step->off_stalled);

    // ---- per layer: block table, slot mapping, ring length
    for (int l = 0; l < L; ++l) {
        const cb_layer_pool &lay = layers[l];
        const int32_t width = step->table_width[l];
        const int32_t R = lay.ring_len;
        int32_t *table = out + step->off_block_table[l];
        int32_t *slots = out + step->off_slot_mapping[l];
        int32_t *rlen = out + step->off_ring_len[l];
        for (int32_t r = 0; r < N; ++r) {
            const Scheduled &s = all[r];
            const cb_req &rq = reqs[s.req];
            int32_t *row = table + int64_t(r) * width;
            // the row's pages: those owned, those matched in the prefix cache, then the fresh ones (from the free
            // list, or allocated by the cache)
            const int32_t used = R > 0 ? R : int32_t(ceil_div(seq[r], P));
            const int32_t own = rq.n_pages[l];
            const int32_t *fresh = pc ? alloc.data() : lay.free_pages;
            for (int32_t b = 0; b < width; ++b) {
                int32_t page = params->pad_page;
                if (b < used) {
                    if (b < own) page = rq.pages[l][b];
                    else if (b - own < s.n_match) page = match_pages[size_t(s.match_from + b - own)];
                    else page = fresh[s.new_from[l] + (b - own - s.n_match)];
                }
                row[b] = page;
            }
            rlen[r] = R;
            for (int32_t j = 0; j < s.q; ++j)
                slots[qsl[r] + j] = int32_t(slot_of(row, int64_t(rq.num_computed) + s.matched + j, P, R));
        }
    }
    const bool blocked = !stalled.empty() || first_rejected >= 0;
    return (N == 0 && blocked) ? CB_E_NOSPACE : CB_OK;
}

// ------------------------------------------------------------------------------------- schedule and plan at once

extern "C" cb_status cb_build_step(const cb_req *reqs, int32_t n_reqs, const cb_sched_params *params,
                                   const cb_layer_pool *layers, const cb_attn_shape *shapes, int32_t *out,
                                   int64_t meta_capacity, int64_t out_capacity, cb_step *step, cb_plan *plans,
                                   int64_t *plan_offsets) {
    if (!params || !shapes || !plans || !plan_offsets || !out || !step || meta_capacity < 0 ||
        out_capacity < meta_capacity)
        return CB_E_INVAL;
    const cb_status st = cb_build_metadata(reqs, n_reqs, params, layers, out, meta_capacity, step);
    if (st != CB_OK) return st;
    const int32_t N = step->num_reqs;
    int64_t at = 0;
    for (int l = 0; l < params->n_layers; ++l) {
        const int32_t *ring = layers[l].ring_len > 0 ? out + step->off_ring_len[l] : nullptr;
        plan_offsets[l] = at;
        const cb_status ps = cb_plan_attention(out + step->off_query_start_loc, out + step->off_seq_lens, ring, N,
                                               &shapes[l], out + meta_capacity + at, out_capacity - meta_capacity - at,
                                               &plans[l]);
        if (ps != CB_OK) return ps;
        at += plans[l].used;
    }
    return CB_OK;
}

// ------------------------------------------------------------------------------------------ request lifecycle

extern "C" cb_status cb_advance(cb_req *reqs, int32_t n_reqs, const cb_sched_params *params, cb_layer_pool *layers,
                                const int32_t *buf, const cb_step *step, int32_t *page_store, int32_t store_stride) {
    if (!params || !layers || !buf || !step || n_reqs < 0 || (n_reqs > 0 && !reqs) || store_stride < 0)
        return CB_E_INVAL;
    const int32_t P = params->page_size;
    const int32_t L = params->n_layers;
    const int32_t N = step->num_reqs;
    if (P < 1 || L < 1 || L > CB_MAX_LAYERS || N < 0 || N > n_reqs) return CB_E_INVAL;
    if (N > 0 && !page_store) return CB_E_INVAL;
    cb_prefix_cache *pc = step->prefix_sharing ? params->prefix_cache : nullptr;
    if (step->prefix_sharing && !pc) return CB_E_INVAL;
    const int32_t *qsl = buf + step->off_query_start_loc;
    const int32_t *seq = buf + step->off_seq_lens;
    const int32_t *idx = buf + step->off_req_index;
    auto pages_after = [&](int l, int32_t s) -> int64_t {
        return layers[l].ring_len > 0 ? layers[l].ring_len : ceil_div(s, P);
    };
    // blocks [first, end) of row r's prompt that this step completed (registered when the step shared prefixes)
    auto completed = [&](int32_t r, int32_t &first, int32_t &end) {
        const cb_req &rq = reqs[idx[r]];
        first = (seq[r] - (qsl[r + 1] - qsl[r])) / P;
        end = std::min(seq[r] / P, rq.prompt_hashes ? rq.n_prompt_blocks : 0);
    };

    // everything is checked before anything changes
    if (qsl[0] != 0) return CB_E_INVAL;
    std::vector<uint8_t> seen(size_t(n_reqs), 0);
    for (int32_t r = 0; r < N; ++r) {
        const int32_t i = idx[r];
        if (i < 0 || i >= n_reqs || seen[size_t(i)]) return CB_E_INVAL;
        seen[size_t(i)] = 1;
        const cb_req &rq = reqs[i];
        const int32_t q = qsl[r + 1] - qsl[r];
        const int32_t ctx = seq[r] - q;
        if (q < 0 || ctx < rq.num_computed) return CB_E_INVAL;
        for (int l = 0; l < L; ++l) {
            const int64_t n = pages_after(l, seq[r]);
            if (n > step->table_width[l]) return CB_E_INVAL;
            if (n > store_stride) return CB_E_CAPACITY;
        }
        if (pc) {
            int32_t b0, b1;
            completed(r, b0, b1);
            const int32_t *row = buf + step->off_block_table[0] + int64_t(r) * step->table_width[0];
            for (int32_t b = b0; b < b1; ++b) {
                int32_t refs = 0, registered = 0;
                uint64_t h = 0;
                if (cb_pcache_page_info(pc, row[b], &refs, &registered, &h) != CB_OK || refs < 1 || registered)
                    return CB_E_INVAL;
            }
        }
    }
    if (!step->prefix_sharing)
        for (int l = 0; l < L; ++l)
            if (step->used_pages[l] < 0 || step->used_pages[l] > layers[l].n_free) return CB_E_INVAL;

    for (int32_t r = 0; r < N; ++r) {
        const int32_t i = idx[r];
        cb_req &rq = reqs[i];
        if (pc) {
            int32_t b0, b1;
            completed(r, b0, b1);
            const int32_t *row = buf + step->off_block_table[0] + int64_t(r) * step->table_width[0];
            for (int32_t b = b0; b < b1; ++b) cb_pcache_commit(pc, row[b], rq.prompt_hashes[b]);
        }
        // the keys up to seq_len are in the cache now: this step's tokens and any prompt tokens reused from the cache
        rq.num_pending -= seq[r] - rq.num_computed;
        rq.num_computed = seq[r];
        if (rq.num_pending <= 0) {
            rq.state = CB_DECODING;   // the prompt is done: the token this step produced is fed next
            rq.num_pending = 1;
        } else {
            rq.state = CB_PREFILLING;
        }
        for (int l = 0; l < L; ++l) {
            const int64_t n = pages_after(l, seq[r]);
            int32_t *dst = page_store + (int64_t(i) * L + l) * store_stride;
            std::memcpy(dst, buf + step->off_block_table[l] + int64_t(r) * step->table_width[l], size_t(n) * 4);
            rq.pages[l] = dst;
            rq.n_pages[l] = int32_t(n);
        }
    }
    if (!step->prefix_sharing)
        for (int l = 0; l < L; ++l) {
            layers[l].free_pages += step->used_pages[l];
            layers[l].n_free -= step->used_pages[l];
        }
    return CB_OK;
}

extern "C" cb_status cb_slot_mapping(const int32_t *pages, int32_t n_pages, int32_t ring_len, int32_t page_size,
                                     int32_t lo, int32_t hi, int32_t *out) {
    if (page_size < 1 || n_pages < 0 || ring_len < 0 || lo < 0 || hi < lo) return CB_E_INVAL;
    if (hi == lo) return CB_OK;
    if (!pages || !out) return CB_E_INVAL;
    // the largest table index any position reads must exist
    const int64_t need = ring_len > 0 ? std::min<int64_t>(ring_len, ceil_div(hi, page_size)) : ceil_div(hi, page_size);
    if (need > n_pages || (ring_len > 0 && ring_len > n_pages)) return CB_E_INVAL;
    for (int32_t p = lo; p < hi; ++p) out[p - lo] = int32_t(slot_of(pages, p, page_size, ring_len));
    return CB_OK;
}

extern "C" cb_status cb_validate_metadata(const int32_t *qsl, const int32_t *seq_lens, int32_t N,
                                          const int32_t *table, int32_t width, const int32_t *ring_len,
                                          const int32_t *slots, int32_t T, int32_t num_pages, int32_t P,
                                          int32_t n_reserved, int32_t *bad_what, int32_t *bad_index) {
    auto fail = [&](int32_t what, int64_t index) {
        if (bad_what) *bad_what = what;
        if (bad_index) *bad_index = int32_t(index);
        return CB_E_INVAL;
    };
    if (bad_what) *bad_what = 0;
    if (bad_index) *bad_index = -1;
    if (N < 0 || T < 0 || width < 0 || num_pages < 1 || P < 1 || n_reserved < 0) return fail(0, -1);
    if (!qsl || (N > 0 && (!seq_lens || (width > 0 && !table)))) return fail(0, -1);
    if (qsl[0] != 0) return fail(1, 0);
    for (int32_t r = 0; r < N; ++r)
        if (qsl[r + 1] < qsl[r]) return fail(1, r + 1);
    if (qsl[N] != T) return fail(1, N);
    for (int32_t r = 0; r < N; ++r) {
        const int32_t q = qsl[r + 1] - qsl[r];
        if (seq_lens[r] < q) return fail(2, r);
        const int32_t R = ring_len ? ring_len[r] : 0;
        if (R < 0) return fail(3, r);
        const int64_t used = R > 0 ? R : ceil_div(seq_lens[r], P);
        if (used > width) return fail(3, r);
        const int32_t *row = table + int64_t(r) * width;
        for (int64_t b = 0; b < used; ++b)
            if (row[b] < n_reserved || row[b] >= num_pages) return fail(3, r);
        if (!slots) continue;
        const int64_t ctx = int64_t(seq_lens[r]) - q;
        for (int32_t j = 0; j < q; ++j) {
            const int32_t s = slots[qsl[r] + j];
            if (s >= 0 && s != slot_of(row, ctx + j, P, R)) return fail(4, qsl[r] + j);
        }
    }
    return CB_OK;
}

// -------------------------------------------------------------------------------------------------- planner
//
// Work items, 8 int32 each:
//   decode / row-wise item:  {row, token, pos, kv_lo, kv_hi, slot, ring_len, 0}
//   prefill tile item:       {row, token0, pos0, q_count, kv_lo, kv_hi, slot_base, ring_len}
// Merge item, 4 int32:       {token, first_slot, n_splits, slot_stride}
// [kv_lo, kv_hi) is the item's key range (absolute positions). slot < 0: the item owns the whole visible range of
// its rows and writes the output; otherwise it writes unnormalised partial results into workspace slots.

namespace {

constexpr int kPrefillRowsNarrow = 128;  // query rows (token x grouped head) of a 4-wave prefill work group
constexpr int kPrefillRowsWide = 256;    // ... of an 8-wave one
constexpr int kPrefillMaxPages = 1536;  // page ids of one prefill item the device kernel stages in LDS
constexpr int kDecodeMaxPages = 1040;   // page ids of one decode split the device kernel stages in LDS
constexpr int kNumCUs = 256;

struct Item {
    int32_t v[8];
};

}  // namespace

extern "C" cb_status cb_plan_attention(const int32_t *qsl, const int32_t *seq_lens, const int32_t *ring_len,
                                       int32_t N, const cb_attn_shape *sh, int32_t *out, int64_t out_capacity,
                                       cb_plan *plan) {
    if (!sh || !plan || N < 0 || (N > 0 && (!qsl || !seq_lens))) return CB_E_INVAL;
    const int32_t Hq = sh->num_q_heads, Hkv = sh->num_kv_heads, D = sh->head_dim, P = sh->page_size;
    if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || sh->window_left < -1) return CB_E_INVAL;
    if (sh->decode_split < 0 || sh->decode_split % 64 != 0) return CB_E_INVAL;
    if (sh->prefill_split < 0 || sh->prefill_split % 64 != 0) return CB_E_INVAL;
    if (sh->prefill_rows != 0 && sh->prefill_rows != kPrefillRowsNarrow && sh->prefill_rows != kPrefillRowsWide)
        return CB_E_INVAL;
    if ((D != 64 && D != 128) || !is_pow2(P) || P > 256) return CB_E_UNSUPPORTED;
    if (sh->dtype != CB_DTYPE_F32 && sh->dtype != CB_DTYPE_BF16) return CB_E_UNSUPPORTED;
    if (N > 0 && qsl[0] != 0) return CB_E_INVAL;
    for (int32_t r = 0; r < N; ++r) {
        const int32_t q = qsl[r + 1] - qsl[r];
        if (q < 0 || seq_lens[r] < q) return CB_E_INVAL;
        if (ring_len && ring_len[r] < 1) return CB_E_INVAL;
    }
    const int32_t G = Hq / Hkv;
    const int32_t W = sh->window_left;
    const bool bf16 = sh->dtype == CB_DTYPE_BF16;
    const bool fast_decode = bf16 && P >= 8 && G <= 16;
    auto lo_of = [&](int64_t pos) -> int64_t { return W < 0 ? 0 : std::max<int64_t>(0, pos - W); };
    // Prefill tile rows. 256-row tiles (8 waves) copy each K/V tile into LDS once for twice the rows of a 128-row
    // tile, but give half as many work groups and run one per CU: chosen when the step's chunks fill the CUs with
    // at least three of them each.
    int32_t rows = sh->prefill_rows;
    if (rows == 0) {
        rows = kPrefillRowsNarrow;
        if (bf16 && P >= 8 && kPrefillRowsWide % G == 0) {
            int64_t wide_tiles = 0;
            for (int32_t r = 0; r < N; ++r) {
                const int32_t q = qsl[r + 1] - qsl[r];
                if (q > 1) wide_tiles += ceil_div(q, kPrefillRowsWide / G);
            }
            if (wide_tiles * Hkv >= 3 * kNumCUs) rows = kPrefillRowsWide;
        }
    }
    const bool fast_prefill = bf16 && P >= 8 && G <= rows && rows % G == 0;
    const int32_t tile_tokens = fast_prefill ? rows / G : 0;

    // ---- split sizes. Decode: enough (row, split, kv head) work groups to give every CU several; prefill: tiles
    // with long key ranges are cut so that no work group carries many times the average work.
    int64_t dec_keys = 0, tile_work = 0;
    for (int32_t r = 0; r < N; ++r) {
        const int32_t q = qsl[r + 1] - qsl[r];
        const int64_t ctx = int64_t(seq_lens[r]) - q;
        const bool as_rows = (q == 1) ? !fast_decode : !fast_prefill;
        if (q == 1 || as_rows) {
            for (int32_t i = 0; i < q; ++i) dec_keys += ctx + i + 1 - lo_of(ctx + i);
        } else {
            for (int32_t i0 = 0; i0 < q; i0 += tile_tokens) {
                const int64_t hi = ctx + std::min(q, i0 + tile_tokens);
                tile_work += hi - lo_of(ctx + i0);
            }
        }
    }
    int32_t S = sh->decode_split;
    if (S == 0) {
        const int64_t target_groups = 6 * kNumCUs;                       // work groups across all kv heads
        const int64_t per = ceil_div(dec_keys * Hkv, target_groups);
        S = int32_t(std::min<int64_t>(4096, std::max<int64_t>(256, ceil_div(per, 256) * 256)));
    }
    // the decode kernel stages a split's page ids in LDS: at most kDecodeMaxPages - 2 pages of keys per split (a cap
    // that depends on the page size only, so a caller-fixed split stays independent of the batch)
    if (fast_decode) S = int32_t(std::min<int64_t>(S, int64_t(kDecodeMaxPages - 2) * P / 64 * 64));
    int32_t PS = sh->prefill_split;
    if (PS == 0) {
        // Split a tile's key range only as far as load balance needs: every split writes fp32 partial rows that the
        // merge reads back. Items may be up to ~1.25x the average work of one work-group slot (two per CU with
        // 128-row tiles, one with 256-row tiles).
        const int64_t slots = (rows == kPrefillRowsWide ? 1 : 2) * kNumCUs;
        const int64_t per_slot = ceil_div(tile_work * Hkv, slots);
        PS = int32_t(std::min<int64_t>(1 << 20, std::max<int64_t>(512, ceil_div(per_slot * 5 / 4, 64) * 64)));
    }
    // a prefill item's page ids are staged in LDS: at most kPrefillMaxPages - 2 pages of keys per split
    PS = int32_t(std::min<int64_t>(PS, int64_t(kPrefillMaxPages - 2) * P / 64 * 64));
    if (PS < 64) return CB_E_UNSUPPORTED;

    std::vector<Item> dec, pre, rowwise;
    std::vector<int32_t> comb;
    int64_t slots = 0;
    int64_t max_block = -1;
    auto split_row = [&](std::vector<Item> &dst, int32_t r, int32_t t, int64_t pos, int32_t ring) {
        const int64_t lo = lo_of(pos), hi = pos + 1;
        const int64_t first = (lo / S) * S;
        const int64_t n = ceil_div(hi - first, S);
        const int64_t base = n > 1 ? slots : -1;
        for (int64_t s = 0; s < n; ++s) {
            const int64_t a = std::max(lo, first + s * S), b = std::min(hi, first + (s + 1) * S);
            Item it{{r, t, int32_t(pos), int32_t(a), int32_t(b), int32_t(n > 1 ? base + s : -1), ring, 0}};
            dst.push_back(it);
        }
        if (n > 1) {
            comb.insert(comb.end(), {t, int32_t(base), int32_t(n), 1});
            slots += n;
        }
        max_block = std::max<int64_t>(max_block, ring > 0 ? ring - 1 : (hi - 1) / P);
    };

    for (int32_t r = 0; r < N; ++r) {
        const int32_t q = qsl[r + 1] - qsl[r];
        if (q == 0) continue;
        const int64_t ctx = int64_t(seq_lens[r]) - q;
        const int32_t ring = ring_len ? ring_len[r] : 0;
        if (q == 1 && fast_decode) {
            split_row(dec, r, qsl[r], ctx, ring);
        } else if (q > 1 && fast_prefill) {
            for (int32_t i0 = 0; i0 < q; i0 += tile_tokens) {
                const int32_t qc = std::min(tile_tokens, q - i0);
                const int64_t pos0 = ctx + i0;
                const int64_t lo = lo_of(pos0), hi = pos0 + qc;
                // split boundaries: at multiples of a caller-fixed PS, so that a request's split points (and its
                // output bits) do not depend on the rest of the batch; with the planner's own PS, from the tile's
                // first 64-key tile, so that a tile whose keys fit one split is never cut (a sliding window's range
                // would otherwise straddle a multiple of PS)
                const int64_t first = sh->prefill_split > 0 ? (lo / PS) * PS : (lo / 64) * 64;
                const int64_t n = ceil_div(hi - first, PS);
                const int64_t base = n > 1 ? slots : -1;
                for (int64_t s = 0; s < n; ++s) {
                    const int64_t a = std::max(lo, first + s * PS), b = std::min(hi, first + (s + 1) * PS);
                    Item it{{r, qsl[r] + i0, int32_t(pos0), qc, int32_t(a), int32_t(b),
                             int32_t(n > 1 ? base + s * qc : -1), ring}};
                    pre.push_back(it);
                }
                if (n > 1) {
                    for (int32_t i = 0; i < qc; ++i)
                        comb.insert(comb.end(), {qsl[r] + i0 + i, int32_t(base + i), int32_t(n), qc});
                    slots += n * qc;
                }
                max_block = std::max<int64_t>(max_block, ring > 0 ? ring - 1 : (hi - 1) / P);
            }
        } else {
            for (int32_t i = 0; i < q; ++i) split_row(rowwise, r, qsl[r] + i, ctx + i, ring);
        }
    }
    if (slots > INT32_MAX / 2) return CB_E_UNSUPPORTED;
    // heaviest items first: work groups are dispatched roughly in index order, so this packs the CUs like
    // longest-processing-time-first scheduling and keeps long items out of the tail
    auto by_keys = [](const Item &a, const Item &b) { return a.v[4] - a.v[3] > b.v[4] - b.v[3]; };
    std::stable_sort(dec.begin(), dec.end(), by_keys);
    std::stable_sort(rowwise.begin(), rowwise.end(), by_keys);
    std::stable_sort(pre.begin(), pre.end(), [](const Item &a, const Item &b) {
        return int64_t(a.v[5] - a.v[4]) * a.v[3] > int64_t(b.v[5] - b.v[4]) * b.v[3];
    });

    std::memset(plan, 0, sizeof(*plan));
    plan->n_decode = int32_t(dec.size());
    plan->n_prefill = int32_t(pre.size());
    plan->n_rowwise = int32_t(rowwise.size());
    plan->n_combine = int32_t(comb.size() / 4);
    plan->n_partials = int32_t(slots);
    plan->decode_split = S;
    plan->prefill_split = PS;
    plan->prefill_tokens = tile_tokens;
    plan->num_tokens = N > 0 ? qsl[N] : 0;
    plan->max_page_index = int32_t(max_block);
    int64_t off = 0;
    plan->off_decode = off;  off += 8 * int64_t(dec.size());
    plan->off_prefill = off; off += 8 * int64_t(pre.size());
    plan->off_rowwise = off; off += 8 * int64_t(rowwise.size());
    plan->off_combine = off; off += int64_t(comb.size());
    plan->used = off;
    if (off > out_capacity || (off > 0 && !out)) return CB_E_CAPACITY;
    auto put = [&](const std::vector<Item> &v, int64_t at) {
        for (size_t k = 0; k < v.size(); ++k) std::memcpy(out + at + 8 * int64_t(k), v[k].v, sizeof(Item));
    };
    put(dec, plan->off_decode);
    put(pre, plan->off_prefill);
    put(rowwise, plan->off_rowwise);
    if (!comb.empty()) std::memcpy(out + plan->off_combine, comb.data(), comb.size() * sizeof(int32_t));
    return CB_OK;
}
