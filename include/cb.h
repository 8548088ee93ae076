/*
 * cb.h -- C ABI of the mixed-batch paged attention step of continuous batching, for AMD Instinct MI355X (gfx950).
 *
 * One forward step of a continuously batched model holds a ragged concatenation of decode tokens and prefill-chunk
 * tokens. The scheduler builds the step's metadata on the host (query_start_loc, seq_lens, slot_mapping,
 * block_table) and the attention kernels only check bounds and map logical key positions to physical pages
 * ("Continuous Batching" blog, languisher.top, section "扩展：vLLM v1 中的实现"). This library provides:
 *
 *   cb_build_metadata   host: FIFO fill under a token budget, page allocation, ragged metadata
 *   cb_plan_attention   host: split the step into kernel work items (decode splits, prefill tiles, merges)
 *   cb_kv_append        device: write the step's new K/V rows into the paged cache through slot_mapping
 *   cb_paged_attention  device: attention of every query row of the step over its request's paged keys
 *
 * Conventions shared by all calls
 *   - Every integer array is int32, row-major, densely packed. Device pointers are plain HIP device addresses;
 *     host pointers are ordinary process memory. The library never frees or keeps any pointer it is given.
 *   - A step has N requests ("rows" of the metadata) and T query tokens. Request r owns tokens
 *     query_start_loc[r] .. query_start_loc[r+1]-1; query_start_loc has N+1 entries, [0] = 0, [N] = T.
 *   - seq_lens[r] = number of keys of request r after this step = context_len + q_len, where context_len keys were
 *     computed in earlier steps. Token i of request r sits at position context_len + i and attends keys
 *     [lo, context_len + i] (inclusive; itself included), lo = 0 for full layers, max(0, pos - window_left) for
 *     sliding layers.
 *   - Paging: key position p of request r lives in physical page block_table[r][p / page_size] at offset
 *     p % page_size; in ring mode (sliding layers) in page block_table[r][(p / page_size) % ring_len[r]].
 *   - Cache layout (one tensor per layer for K and one for V, element type = the dtype). NOTE: this is NOT the
 *     plain [num_pages][page_size][num_kv_heads][head_dim] order; V is transposed inside each page:
 *        k_cache  [num_pages][num_kv_heads][page_size][head_dim]   (key rows, head_dim contiguous)
 *        v_cache  [num_pages][num_kv_heads][head_dim][page_size]   (value columns, page offsets contiguous)
 *     Callers state it with the tag CB_LAYOUT_KD_VT on every cache call (see "cache layout" below); the plain
 *     order has its own tag, CB_LAYOUT_PAGED_NHD, which the kernels refuse. One kv head's slice of one page is a
 *     single contiguous run of page_size*head_dim elements in each tensor.
 *   - Q and O are [T][num_q_heads][head_dim]; new K/V rows are [T][num_kv_heads][head_dim]. Query head h reads kv
 *     head h / (num_q_heads / num_kv_heads).
 *   - dtype: CB_DTYPE_F32 (float) or CB_DTYPE_BF16 (bfloat16). Attention accumulates in fp32; bf16 outputs are
 *     rounded to nearest even.
 *   - Device calls are asynchronous on the given stream (a hipStream_t passed as void*, NULL = the null stream).
 *     They validate arguments synchronously and return before any launch on error.
 */
#ifndef CB_H
#define CB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CB_ABI_VERSION 8

typedef int32_t cb_status;
#define CB_OK 0
#define CB_E_INVAL 1        /* inconsistent arguments (lengths, shapes, metadata)                          */
#define CB_E_NOSPACE 2      /* cb_build_metadata: nothing could be scheduled for lack of free pages        */
#define CB_E_CAPACITY 3     /* output buffer too small; the needed size is written back                    */
#define CB_E_UNSUPPORTED 4  /* valid but not implemented (head_dim, page_size, dtype, head ratio)          */
#define CB_E_WORKSPACE 5    /* cb_paged_attention: workspace missing or too small                          */
#define CB_E_HIP 6          /* a HIP runtime call or kernel launch failed                                  */

#define CB_DTYPE_F32 0
#define CB_DTYPE_BF16 1

/* request states, in the order of the request lifecycle (Transformers "continuous batching architecture" page,
 * section "请求生命周期"): waiting in the queue, prefilling the prompt in chunks, decoding one token per step. */
#define CB_DECODING 0
#define CB_PREFILLING 1
#define CB_WAITING 2

#define CB_MAX_LAYERS 2     /* attention layer types per step: full, and optionally sliding */

/* ------------------------------------------------------------------------------------------- cb_build_metadata */

typedef struct cb_prefix_cache cb_prefix_cache;   /* prefix cache (see "prefix cache" below), opaque */

/* One request known to the scheduler, given in arrival (FIFO) order. */
typedef struct cb_req {
    int64_t id;                          /* caller's id; not interpreted                                         */
    int32_t state;                       /* CB_DECODING, CB_PREFILLING or CB_WAITING                            */
    int32_t num_computed;                /* keys already in the cache (context before this step), >= 0          */
    int32_t num_pending;                 /* tokens to feed: exactly 1 for CB_DECODING, >= 1 otherwise            */
    int32_t n_pages[CB_MAX_LAYERS];      /* pages already owned per layer type                                   */
    const int32_t *pages[CB_MAX_LAYERS]; /* host arrays of owned page ids, logical order (full) or ring order    */
    const uint64_t *prompt_hashes;       /* chain hashes of the prompt's full blocks (cb_block_hashes), or NULL:
                                            looked up in the prefix cache when the request is admitted          */
    int32_t n_prompt_blocks;             /* entries of prompt_hashes                                            */
} cb_req;

/* One layer type's page pool. */
typedef struct cb_layer_pool {
    int32_t ring_len;          /* 0: full attention, pages grow with the sequence; > 0: sliding layer, each
                                  request owns a ring of exactly ring_len pages from admission on              */
    int32_t window_left;       /* sliding layers: keys pos-window_left..pos are visible; -1 for full layers     */
    int32_t pool_pages;        /* allocatable pages of the pool (denominator of the safety margin)              */
    int32_t n_free;            /* entries of free_pages                                                         */
    const int32_t *free_pages; /* host array: free pages in allocation order; pages are taken from the front   */
} cb_layer_pool;

/* Scheduling policies (Transformers "continuous batching architecture" page, sections "FIFO" and "PrefillFirst"). */
#define CB_POLICY_FIFO 0           /* active decodes, then active prefills, then waiting requests                 */
#define CB_POLICY_PREFILL_FIRST 1  /* active prefills, then waiting requests, then decodes with what budget is left */

typedef struct cb_sched_params {
    int32_t max_batch_tokens;  /* token budget of one forward pass, >= 1                                        */
    int32_t max_requests;      /* request cap of one forward pass, >= 1                                         */
    int32_t page_size;         /* tokens per page, >= 1                                                         */
    int32_t pad_page;          /* page id written into unused block-table entries (a reserved padding page)     */
    int32_t n_layers;          /* 1 or 2 layer types                                                            */
    int32_t policy;            /* CB_POLICY_FIFO or CB_POLICY_PREFILL_FIRST                                     */
    float safety_margin;       /* hold new prefills while any pool's free fraction is below this (0 disables);
                                  the page gives 0.15 as the FIFO default and 0 for PrefillFirst              */
    cb_prefix_cache *prefix_cache; /* NULL, or a prefix cache over layer 0's pool: prefix sharing at admission
                                  (see cb_build_metadata)                                                      */
} cb_sched_params;

/* Header of the packed int32 buffer cb_build_metadata writes. Offsets count int32 elements from the buffer start;
 * per scheduled row r (rows laid out decodes first, then continuing prefills, then admitted requests, each group in
 * scheduling order, whatever the policy): */
typedef struct cb_step {
    int32_t num_reqs;                        /* N rows scheduled                                                 */
    int32_t num_tokens;                      /* T                                                                */
    int32_t num_decodes;                     /* rows 0..num_decodes-1 are the decodes                            */
    int32_t max_q_len, max_seq_len;
    int32_t n_stalled;                       /* active requests left out for lack of pages                       */
    int32_t first_rejected;                  /* input index of the waiting request refused admission, or -1      */
    int32_t held_by_margin;                  /* 1 if new prefills were held by the safety margin                 */
    int32_t prefix_sharing;                  /* 1 if the step scheduled with prefix sharing on                   */
    int32_t used_pages[CB_MAX_LAYERS];       /* pages taken from the front of each free list                     */
    int32_t table_width[CB_MAX_LAYERS];      /* row stride of each layer's block table                           */
    int64_t off_query_start_loc;             /* [N+1]                                                            */
    int64_t off_seq_lens;                    /* [N]                                                              */
    int64_t off_req_index;                   /* [N] input index of each row                                      */
    int64_t off_stalled;                     /* [n_stalled] input indices, ascending                             */
    int64_t off_block_table[CB_MAX_LAYERS];  /* [N][table_width]; unused entries hold pad_page                   */
    int64_t off_slot_mapping[CB_MAX_LAYERS]; /* [T] page * page_size + offset of each new token's K/V            */
    int64_t off_ring_len[CB_MAX_LAYERS];     /* [N] ring length per row (0 for full layers)                      */
    int64_t off_matched;                     /* [N] prompt tokens each row reused from the prefix cache          */
    int64_t used;                            /* int32 elements written, or needed when CB_E_CAPACITY            */
} cb_step;

/*
 * Schedule one step (Transformers "continuous batching architecture" page, sections "调度器", "FIFO",
 * "PrefillFirst", "准入" and "分块预填充"; "Continuous Batching" blog, section "扩展：与 Chunked Prefill 结合").
 * Three passes, in the order of the policy (FIFO: D, P, A; PrefillFirst: P, A, D):
 *   D. active decodes in arrival order, one token each;
 *   P. active prefills, each continuing with min(num_pending, budget left) tokens;
 *   A. waiting requests in arrival order: held while a pool's free fraction is below safety_margin; admitted
 *      all-or-nothing across layer types (pages for the chunk, plus a whole ring for sliding layers); the first
 *      refusal stops admission.
 *   Every pass stops at max_requests rows or an exhausted budget, and takes its pages from the front of the free
 *   lists in that order. Active requests whose pages cannot be allocated are reported stalled and left out.
 * Prefix sharing (same page, sections "前缀缓存" and "准入"), when params->prefix_cache is set and the step has one
 * layer type, a full-attention one (the page: sharing is on only when every allocator supports it, so sliding and
 * hybrid models run without it; with a ring layer the cache is ignored):
 *   - every page the step takes comes from the cache's allocator (cb_pcache_allocate order: empty pages first,
 *     then demoted initialized ones), not from layers[0].free_pages;
 *   - a waiting request with num_computed 0 and no pages first looks up the leading blocks of its prompt_hashes,
 *     at most (num_pending - 1) / page_size of them, so that at least one prompt token is still computed; their
 *     pages become its first pages (references taken) and its context starts at matched * page_size;
 *   - admission stays all-or-nothing: the match is taken only if the fresh pages for the rest of the chunk can be
 *     allocated too, counting matched pages that sat free in the cache as leaving its free pool;
 *   - the safety margin and every availability check use the cache's free pages.
 * The call then changes the cache (references taken, pages allocated); the caller registers completed prompt blocks
 * (cb_pcache_commit) after the step and releases a finished request's pages. To keep a failed call from changing
 * the cache, the output capacity is checked first against a bound of the output size (step->used = that bound on
 * CB_E_CAPACITY).
 * Without a prefix cache the call is a pure host function: reads reqs/params/layers, writes `out` (capacity
 * out_capacity int32 elements) and `step`.
 * Returns CB_OK, CB_E_INVAL (inconsistent input, including a ring too small for max_batch_tokens), CB_E_NOSPACE
 * (no row could be scheduled because pages ran out; out/step are still valid) or CB_E_CAPACITY (step->used tells
 * the size needed).
 */
cb_status cb_build_metadata(const cb_req *reqs, int32_t n_reqs, const cb_sched_params *params,
                            const cb_layer_pool *layers, int32_t *out, int64_t out_capacity, cb_step *step);

/*
 * Request lifecycle after a step has run (Transformers "continuous batching architecture" page, section "请求生命周期":
 * a waiting request is admitted and prefilled in chunks, then decodes one token per step), done in place on the
 * arrays the next cb_build_metadata call reads, so that a serving loop's host half stays in native code.
 * buf/step: the step's metadata as cb_build_metadata wrote it from these same reqs/params/layers. For every row r
 * the step scheduled (request i = req_index[r]):
 *   - the keys up to seq_len[r] are in the cache: num_pending drops by seq_len[r] - num_computed (this step's
 *     tokens plus any prompt tokens reused from the prefix cache) and num_computed becomes seq_len[r];
 *   - a request whose prompt is done decodes next (CB_DECODING, one pending token: the token this step produced),
 *     otherwise it keeps prefilling (CB_PREFILLING);
 *   - per layer type its pages become its block-table row: the first ceil(seq_len / page_size) entries, or its
 *     whole ring. They are copied to page_store + (i * n_layers + l) * store_stride and reqs[i].pages[l] points
 *     there (page_store: host int32 [n_reqs][n_layers][store_stride], caller-owned, must outlive every later use
 *     of reqs);
 *   - when the step shared prefixes (step->prefix_sharing), every prompt block the step completed (blocks
 *     ctx / page_size .. min(seq_len / page_size, n_prompt_blocks) - 1) is registered in params->prefix_cache under
 *     its hash (cb_pcache_commit), so that later requests can reuse it.
 * Requests the step did not schedule are unchanged. Unless the step shared prefixes (its pages then came from the
 * cache's allocator), each pool's free list moves past the pages the step took: layers[l].free_pages +=
 * used_pages[l], layers[l].n_free -= used_pages[l] (the caller's array itself is not written).
 * Everything is checked before anything changes: CB_E_INVAL (a row index out of range or repeated, a seq_len
 * below the request's context, more used pages than a free list holds, a completed block's page not held or
 * already registered) or CB_E_CAPACITY (a row needs more than store_stride pages) leave all arguments unchanged.
 * Host only; allocates nothing the caller sees.
 */
cb_status cb_advance(cb_req *reqs, int32_t n_reqs, const cb_sched_params *params, cb_layer_pool *layers,
                     const int32_t *buf, const cb_step *step, int32_t *page_store, int32_t store_stride);

/*
 * Cache slots of key positions lo .. hi-1 of one request: out[i] = page * page_size + (p % page_size) for p = lo + i,
 * where page = pages[p / page_size] (full layers, ring_len 0) or pages[(p / page_size) % ring_len] (ring mode). This
 * is the rule slot_mapping follows ("Continuous Batching" blog, section "扩展：vLLM v1 中的实现": logical block
 * kv_pos / BLOCK_SIZE, offset kv_pos % BLOCK_SIZE, physical block from block_table), exposed for callers that write
 * keys the scheduler did not schedule (a request's history, a swapped-in prompt). Host only.
 * pages: host [n_pages], the request's block-table row (or ring). out: host [hi - lo], caller-owned.
 * Returns CB_E_INVAL if a position needs an entry beyond n_pages, or on bad sizes (nothing is written then).
 */
cb_status cb_slot_mapping(const int32_t *pages, int32_t n_pages, int32_t ring_len, int32_t page_size, int32_t lo,
                          int32_t hi, int32_t *out);

/*
 * Debug check of one layer's step metadata before it goes to the device (the kernels trust it and only clamp page
 * ids into the pool, so a corrupt table gives meaningless rows instead of a fault). Checks, on host arrays:
 * query_start_loc [N+1] starts at 0, never decreases and ends at num_tokens; seq_lens[r] >= q_len[r]; every
 * block-table entry a row reads (its logical blocks 0 .. ceil(seq_len/page_size)-1, or its whole ring) is a page in
 * [n_reserved, num_pages), i.e. inside the pool and not one of the reserved padding pages 0 .. n_reserved-1; every
 * slot_mapping entry (if given) is the slot of its token's position under the same table, or negative (skipped).
 * ring_len [N] or NULL (full layer). On failure returns CB_E_INVAL and writes to *bad_what a code (1 query_start_loc,
 * 2 seq_lens, 3 block table, 4 slot_mapping) and to *bad_index the offending row or token (either pointer may be
 * NULL). Host only, O(metadata).
 */
cb_status cb_validate_metadata(const int32_t *query_start_loc, const int32_t *seq_lens, int32_t num_reqs,
                               const int32_t *block_table, int32_t table_width, const int32_t *ring_len,
                               const int32_t *slot_mapping, int32_t num_tokens, int32_t num_pages, int32_t page_size,
                               int32_t n_reserved, int32_t *bad_what, int32_t *bad_index);

/* ------------------------------------------------------------------------------------------- cb_plan_attention */

typedef struct cb_attn_shape {
    int32_t num_q_heads;       /* Hq, a multiple of num_kv_heads                                               */
    int32_t num_kv_heads;      /* Hkv                                                                          */
    int32_t head_dim;          /* D: 64 or 128                                                                 */
    int32_t page_size;         /* P: a power of two, 1..256                                                    */
    int32_t dtype;             /* CB_DTYPE_F32 or CB_DTYPE_BF16                                                */
    int32_t window_left;       /* -1: full attention; >= 0: sliding window                                     */
    int32_t decode_split;      /* keys per decode split (a multiple of 64), 0 = chosen by the planner from the
                                  whole step's decode keys. Splits are merged in a fixed order, so a fixed value
                                  makes a request's output bits independent of the rest of its batch; with 0 they
                                  may change with the batch (the values stay within rounding of each other).
                                  On the decode kernel's path (bf16, pages of 8 or more keys, up to 16 grouped
                                  heads) capped at 1038 pages of keys (rounded down to a multiple of 64), the
                                  page ids it stages per split; the plan reports the size used                 */
    int32_t prefill_split;     /* keys per prefill-tile split (a multiple of 64), 0 = chosen by the planner
                                  (batch-dependent in the same way as decode_split). Capped at 1534 pages of
                                  keys (rounded down to a multiple of 64), the page ids the prefill kernel stages
                                  per item                                                                     */
    int32_t prefill_rows;      /* query rows (tokens x grouped heads) per prefill work group: 128 (4 waves, two
                                  work groups per CU), 256 (8 waves sharing each K/V tile, one per CU) or 0 =
                                  chosen by the planner (256 when the step has enough such tiles to fill the
                                  CUs several times over). Any other value is CB_E_INVAL. The rows of a tile see
                                  the same keys either way; outputs agree to rounding                          */
} cb_attn_shape;

/* Header of the packed int32 plan. Work items (8 int32 each) and merge items (4 int32 each) start at the given
 * element offsets. */
typedef struct cb_plan {
    int32_t n_decode;          /* split-KV decode items (rows with q_len 1, fast kernels)                     */
    int32_t n_prefill;         /* prefill tile items (rows with q_len > 1, fast kernels)                      */
    int32_t n_rowwise;         /* per-token items of the general kernel (fp32, or shapes the fast kernels skip)*/
    int32_t n_combine;         /* output tokens merged from partial results                                    */
    int32_t n_partials;        /* partial-result slots the workspace must hold                                 */
    int32_t decode_split, prefill_split, prefill_tokens;  /* the sizes used                                    */
    int32_t num_tokens;        /* T                                                                            */
    int32_t max_page_index;    /* largest logical block index any item reads (block_table width check)         */
    int64_t off_decode, off_prefill, off_rowwise, off_combine;
    int64_t used;              /* int32 elements written, or needed when CB_E_CAPACITY                        */
} cb_plan;

/*
 * Split a step into kernel work items: every query row's visible key range [lo, pos] is cut into splits; a row
 * with one split is written directly, a row with several gets partial results merged by a final pass. Host only.
 * query_start_loc [N+1], seq_lens [N] (host); ring_len [N] host array or NULL (full layer).
 * Returns CB_OK, CB_E_INVAL, CB_E_UNSUPPORTED or CB_E_CAPACITY (plan->used tells the size needed).
 */
cb_status cb_plan_attention(const int32_t *query_start_loc, const int32_t *seq_lens, const int32_t *ring_len,
                            int32_t num_reqs, const cb_attn_shape *shape, int32_t *out, int64_t out_capacity,
                            cb_plan *plan);

/*
 * Schedule one step and plan every layer type of it, in one call, into one caller buffer: cb_build_metadata into
 * out[0 .. meta_capacity), then cb_plan_attention of layer l (shape shapes[l]; its ring lengths from the step's
 * metadata for a sliding layer) on the rows the step scheduled, into out[meta_capacity + plan_offsets[l] ..), the
 * plans packed back to back within out_capacity. For serving loops that prepare a step per forward pass: one call
 * instead of 1 + n_layers, with the plans placed where one copy to the device takes them with the metadata.
 * shapes: [params->n_layers]; plans, plan_offsets: [params->n_layers] (caller-owned outputs). Host only.
 * Returns CB_OK, or the first failing call's status with its outputs as that call leaves them (CB_E_CAPACITY:
 * step->used, or plans[l].used for the layer that did not fit, tells the size needed; CB_E_NOSPACE from the
 * scheduler stops before planning). CB_E_INVAL for missing pointers or meta_capacity > out_capacity.
 */
cb_status cb_build_step(const cb_req *reqs, int32_t n_reqs, const cb_sched_params *params,
                        const cb_layer_pool *layers, const cb_attn_shape *shapes, int32_t *out, int64_t meta_capacity,
                        int64_t out_capacity, cb_step *step, cb_plan *plans, int64_t *plan_offsets);

/* ------------------------------------------------------------------------------------------------ cache layout */

/*
 * Cache layout tags. Every call that reads or writes a cache takes one, and refuses (CB_E_UNSUPPORTED, before any
 * launch) a tag it does not implement, so a caller cannot silently pair its tensors with the wrong byte order.
 *
 *   CB_LAYOUT_PAGED_NHD (0)  k_cache and v_cache both [num_pages][page_size][num_kv_heads][head_dim]: the pages'
 *                            own order k_cache[physical_block][block_offset] ("Continuous Batching" blog, section
 *                            "扩展：vLLM v1 中的实现"), heads and head_dim appended. NOT implemented by the device
 *                            kernels: passing it returns CB_E_UNSUPPORTED. It is 0 so that an argument block left
 *                            zeroed is refused rather than misread.
 *   CB_LAYOUT_KD_VT (1)      the layout this library implements. Page-major like the pages' order, with the inner
 *                            order chosen for the bf16 matrix cores of gfx950:
 *                              k_cache [num_pages][num_kv_heads][page_size][head_dim]   key rows, head_dim contiguous
 *                              v_cache [num_pages][num_kv_heads][head_dim][page_size]   value columns, offsets contiguous
 *                            Both contractions (q.k over head_dim, p.v over key offsets) then read their reduction
 *                            index contiguously, 8 elements per lane, which is what an MFMA operand holds; the
 *                            transposition of V is paid once per new token in the append instead of in every
 *                            attention tile. One kv head's slice of a page is one contiguous run in each tensor.
 */
#define CB_LAYOUT_PAGED_NHD 0
#define CB_LAYOUT_KD_VT 1

/* ------------------------------------------------------------------------------------------------ cb_kv_append */

/*
 * For every token t with 0 <= slot_mapping[t] < num_pages*page_size, copy k_new[t] and v_new[t] (all kv heads) into
 * page slot_mapping[t] / page_size at offset slot_mapping[t] % page_size, bit for bit. Tokens with a negative (or
 * out-of-pool) slot are skipped. slot_mapping is the scheduler's (Continuous Batching blog, section "扩展：vLLM v1
 * 中的实现": the scheduler builds slot_mapping with the rest of the metadata). Must be enqueued before
 * cb_paged_attention of the same step: the step's own keys are read back from the cache. (cb_paged_attention can
 * instead do the same append itself, in its own launches: see k_new in cb_attn_args.)
 * Device pointers: k_cache, v_cache (layouts above), k_new, v_new [T][Hkv][D], d_slot_mapping [T].
 * layout: CB_LAYOUT_KD_VT (anything else: CB_E_UNSUPPORTED).
 * Two tokens with the same slot race (last writer wins, unspecified which).
 */
cb_status cb_kv_append(void *k_cache, void *v_cache, const void *k_new, const void *v_new,
                       const int32_t *d_slot_mapping, int32_t num_tokens, int32_t num_pages, int32_t page_size,
                       int32_t num_kv_heads, int32_t head_dim, int32_t dtype, int32_t layout, void *stream);

/* -------------------------------------------------------------------------------------------- cb_kv_copy_pages */

/*
 * Copy whole pages between two page arrays on the device: page i goes from src + src_pages[i] * page_bytes to
 * dst + dst_pages[i] * page_bytes (a NULL list stands for 0, 1, ..., n-1). With a contiguous device buffer on one
 * side this is the batched gather / scatter of a request's cache pages that swapping to host memory needs
 * (Transformers "continuous batching architecture" page, section "Offloading": the KV blocks of offloaded requests
 * are copied to a pre-allocated pinned CPU buffer in one transfer, and copied back when GPU cache space frees up);
 * the transfer between that buffer and pinned host memory is an ordinary asynchronous copy. Call once for the K
 * tensor and once for the V tensor: a page is Hkv * page_size * head_dim elements in either layout.
 * Device pointers: dst, src, d_dst_pages [n], d_src_pages [n]; dst_slots / src_slots are the pages each array holds.
 * Pairs with an index outside its array are skipped. Pages of src and dst must not overlap. Async on `stream`.
 * Returns CB_OK, CB_E_INVAL (negative sizes, page_bytes not a multiple of 16, null buffers, n above an array without
 * an index list), CB_E_UNSUPPORTED (page_bytes above 1 GiB) or CB_E_HIP.
 */
cb_status cb_kv_copy_pages(void *dst, const int32_t *d_dst_pages, int32_t dst_slots, const void *src,
                           const int32_t *d_src_pages, int32_t src_slots, int32_t n, int64_t page_bytes, void *stream);

/* ------------------------------------------------------------------------------------------ cb_paged_attention */

typedef struct cb_attn_args {
    void *out;                    /* device [T][Hq][D], written for every token of the plan                       */
    const void *q;                /* device [T][Hq][D]                                                           */
    const void *k_cache;          /* device, layout above                                                        */
    const void *v_cache;          /* device, layout above                                                        */
    int32_t layout;               /* cache layout tag: must be CB_LAYOUT_KD_VT (else CB_E_UNSUPPORTED)           */
    const int32_t *block_table;   /* device [N][table_width]: physical page per logical block (or ring slot)     */
    const int32_t *plan;          /* device copy of the int32 plan written by cb_plan_attention                 */
    cb_plan plan_info;            /* host copy of that plan's header                                             */
    cb_attn_shape shape;          /* the shape the plan was made for                                             */
    int32_t num_pages;            /* pages in each cache tensor                                                  */
    int32_t table_width;          /* row stride of block_table                                                   */
    float scale;                  /* softmax scale applied to q.k                                                */
    void *workspace;              /* device scratch of cb_paged_attention_workspace_size() bytes (256-aligned)  */
    size_t workspace_bytes;
    int32_t phases;               /* 0 = the whole step; else a mask of CB_PHASE_* launching only those kernels,
                                     in the fixed order (lets a caller bracket one kernel with events)           */
    /* Optional fused append. With k_new set, the call also writes the step's new K/V rows into the caches, exactly
     * as cb_kv_append would with the same arguments, and the caller does not call cb_kv_append for this step. The
     * append runs in the call that launches the plan's first cache-reading phase (decode if the plan has decode
     * items, else the per-token phase, else the prefill phase): inside the decode launch its work groups follow
     * the decode work groups, and each decode row takes its own new key and value from k_new / v_new instead of
     * the cache; otherwise it is a launch of its own ahead of the per-token and prefill kernels. All NULL / 0: the
     * caches are only read. */
    const void *k_new;            /* device [num_new][Hkv][D], the caches' element type                          */
    const void *v_new;            /* device [num_new][Hkv][D]                                                    */
    const int32_t *slot_mapping;  /* device [num_new]; negative or out-of-pool slots are skipped                 */
    int32_t num_new;              /* must equal the plan's token count when k_new is set                         */
    /* Optional device-resident item counts, for launches whose shape must not change from step to step (a HIP graph
     * captured once and replayed for every step that pads to the same shape: Transformers "continuous batching
     * architecture" page, section "CUDA 图"). NULL: plan_info's counts are the items. Else device int32[4] =
     * {n_decode, n_prefill, n_rowwise, n_combine} of THIS step, each <= the matching plan_info count, which is then
     * only a capacity: the grids cover the capacities, the plan's sections are laid out at those capacities (the
     * off_* offsets), and work groups past this step's counts exit at once. plan_info.n_partials must likewise be
     * a capacity that stays the same across such steps: it fixes where the workspace's second region starts.
     * Everything else the launches read (plan items, block table, slot mapping) is read from device memory too,
     * so one captured launch serves every step whose metadata is written to the same addresses. */
    const int32_t *counts;
    /* Optional timing events (hipEvent_t created with timing enabled), for callers that time the kernels: the call's
     * first kernel records timing_start when it begins executing and its last kernel records timing_stop when it
     * ends, so that the pair brackets the kernels alone. Events recorded on the stream around the call would also
     * count the dispatch after the previous work and the completion signal after the last kernel. A call that
     * launches no kernel (its phases have no items) records both on the stream. NULL: none. */
    void *timing_start;
    void *timing_stop;
} cb_attn_args;

#define CB_PHASE_DECODE 1         /* split-KV decode kernel                                                     */
#define CB_PHASE_ROWWISE 2        /* general per-token kernel                                                   */
#define CB_PHASE_PREFILL 4        /* prefill-tile kernel                                                        */
#define CB_PHASE_COMBINE 8        /* merge of split rows; needs the phases that wrote its partials to have run  */

/* Bytes of device workspace cb_paged_attention needs for this plan (0 if none). */
size_t cb_paged_attention_workspace_size(const cb_attn_args *args);

/*
 * Attention of every token of the plan ("Continuous Batching" blog, sections "优化：偏移实现 Mask" and "扩展：vLLM
 * v1 中的实现": per request, keys 0..context_len+local_q through block_table; no mask is materialised).
 * Launches, in order on `stream`: the split-KV decode kernel, the general per-token kernel, the prefill-tile kernel,
 * then the merge of split rows. Reads the caches only, unless the fused append is requested (k_new above). Page ids
 * read from block_table are clamped into
 * [0, num_pages) so a corrupt table cannot fault the device (results are then meaningless).
 * Returns CB_OK, CB_E_INVAL, CB_E_UNSUPPORTED, CB_E_WORKSPACE or CB_E_HIP.
 */
cb_status cb_paged_attention(const cb_attn_args *args, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): cb_paged_attention with the workspace taken from a static device array of
 * CB_NOALLOC_WORKSPACE_BYTES, one per device, which the library holds from the load of its code object until the
 * process ends. args->workspace and args->workspace_bytes are ignored. The caller still passes every input and
 * output. Allocates nothing (no hipMalloc / hipFree, no allocating library call). Returns CB_E_WORKSPACE, before any
 * launch, if the plan's workspace (cb_paged_attention_workspace_size) exceeds the array; CB_E_INVAL if `stream`
 * belongs to a device other than the current one; otherwise what cb_paged_attention returns. All calls on one
 * device share its array: calls that overlap on one device (on different streams, or enqueued before an earlier
 * one has finished reading its partial results) race.
 */
#define CB_NOALLOC_WORKSPACE_BYTES (96u << 20)
cb_status cb_paged_attention_noalloc(const cb_attn_args *args, void *stream);

/* ------------------------------------------------------------------------------------------------ prefix cache */

/*
 * Page sharing between requests with a common prompt prefix (Transformers "continuous batching architecture" page,
 * sections "前缀缓存" (prefix cache) and "驱逐" (eviction)): every full block of a prompt gets a content hash; a later
 * request whose leading blocks are cached reuses their pages and skips their prefill; shared pages carry reference
 * counts and return to a free list only when the last holder releases them; a freed page that holds a hashed block
 * keeps it ("initialized") for later matches, until fresh pages run out and the most recently freed one is demoted
 * (its hash dropped). Host only, deterministic; page ids are the caller's pool (full-attention layers: the page says
 * sliding and hybrid models do not share). All functions return CB_E_INVAL on null or out-of-range arguments.
 */
/* cb_prefix_cache (declared at the top) is opaque, owned by the library between create and destroy. */

/* FNV-1a 64-bit hash of n bytes (offset basis 14695981039346656037, prime 1099511628211). */
uint64_t cb_fnv1a64(const void *data, int64_t n);

/* Chain hashes of the n_tokens / page_size full blocks of a token sequence: block b hashes, with FNV-1a 64, the
 * 8 little-endian bytes of block b-1's hash (the FNV offset basis for b = 0) followed by the block's token ids as
 * 4 little-endian bytes each. out: [n_tokens / page_size] (caller-owned). */
cb_status cb_block_hashes(const int32_t *tokens, int32_t n_tokens, int32_t page_size, uint64_t *out);

/* A cache over pages 0 .. num_pages-1, of which free_pages (distinct, in allocation order) start free and empty.
 * Returns CB_E_CAPACITY if the host allocation of the bookkeeping fails. */
cb_status cb_pcache_create(int32_t num_pages, const int32_t *free_pages, int32_t n_free, cb_prefix_cache **out);
void cb_pcache_destroy(cb_prefix_cache *cache);

/* Longest cached prefix: the leading blocks whose hashes are registered. Their pages go to pages_out [n_blocks] and
 * each gains a reference (a freed one comes back into use); *n_matched tells how many. */
cb_status cb_pcache_match(cb_prefix_cache *cache, const uint64_t *hashes, int32_t n_blocks, int32_t *pages_out,
                          int32_t *n_matched);

/* Pages of the leading registered blocks of hashes [n_blocks], into pages_out, WITHOUT taking references: *n_found
 * tells how many, *n_free_found how many of those pages are currently free (initialized, no reference), i.e. would
 * leave the free pool if matched. Either count pointer may be NULL. */
cb_status cb_pcache_lookup(const cb_prefix_cache *cache, const uint64_t *hashes, int32_t n_blocks, int32_t *pages_out,
                           int32_t *n_found, int32_t *n_free_found);

/* n fresh pages with one reference each, into pages_out [n]: empty pages first, in free-list order, then demoted
 * initialized pages, most recently freed first. All or nothing: CB_E_NOSPACE, and nothing taken, if fewer exist. */
cb_status cb_pcache_allocate(cb_prefix_cache *cache, int32_t n, int32_t *pages_out);

/* Page `page` (held, not yet registered) now holds the full block with this hash: register it. If another page
 * already holds that block, this page stays unregistered (private). */
cb_status cb_pcache_commit(cb_prefix_cache *cache, int32_t page, uint64_t hash);

/* Drop one reference per entry of pages [n] (a page may appear as often as references are held; the whole call is
 * checked first). A page left with none becomes free: initialized if it holds a registered block, empty otherwise. */
cb_status cb_pcache_release(cb_prefix_cache *cache, const int32_t *pages, int32_t n);

/* Counts: empty free pages, initialized free pages, registered blocks. */
cb_status cb_pcache_stats(const cb_prefix_cache *cache, int32_t *n_empty, int32_t *n_initialized_free,
                          int32_t *n_registered);

/* One page's references, whether it holds a registered block, and that block's hash (0 if none). */
cb_status cb_pcache_page_info(const cb_prefix_cache *cache, int32_t page, int32_t *refs, int32_t *registered,
                              uint64_t *hash);

/* --------------------------------------------------------------------------------------------------- utilities */

const char *cb_status_str(cb_status status);
int32_t cb_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CB_H */
