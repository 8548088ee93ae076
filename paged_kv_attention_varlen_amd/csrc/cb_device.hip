// Device half of the cb library for gfx950 (MI355X): KV append, split-KV decode, per-token general kernel,
// prefill tiles, and the merge of split rows. All kernels read their work from the host-built plan.
//
// Layouts (see include/cb.h):
//   k_cache [page][kv_head][offset][d]    -- a key row is D contiguous elements
//   v_cache [page][kv_head][d][offset]    -- a value column over the page's offsets is contiguous
// so both contractions (q.k over d, p.v over keys) read their reduction index contiguously per lane, which is what
// the MFMA operand layouts want: 8 consecutive bf16 of the reduction dimension per lane.
//
// Softmax runs in the log2 domain: scores are multiplied by scale*log2(e) once and exponentiated with exp2;
// partial results store the running maximum in those units.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "cb.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -INFINITY;

__device__ __forceinline__ u32x4 load16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ void store16(void *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }
// streaming load (non-temporal hint): for data read exactly once, such as the K/V pages of a decode split
__device__ __forceinline__ u32x4 load16_stream(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// Physical page of a logical block of one request (ring slot in ring mode), clamped into the pool so that a
// corrupt table cannot send a load outside the cache tensors.
__device__ __forceinline__ int lookup_page(const int32_t *bt_row, int logical, int ring, int num_pages) {
    const int idx = ring > 0 ? logical % ring : logical;
    const int p = bt_row[idx];
    return p < 0 ? 0 : (p >= num_pages ? num_pages - 1 : p);
}

// Work groups are dispatched to the 8 XCDs round-robin by linear block index, and each XCD has its own L2. The work
// groups of one kv head read the same K/V pages, so they are placed on the same XCD: linear block L runs on XCD L % 8
// and is given a (work item, kv head) pair whose head belongs to that XCD. Returns false for the padding blocks of
// the grid (grid size from xcd_grid).
constexpr int kXcds = 8;
__host__ __device__ inline int xcd_grid(int n_items, int n_heads) {
    if (n_heads % kXcds == 0 || kXcds % n_heads != 0) return n_items * n_heads;
    const int r = kXcds / n_heads;   // XCDs sharing one head
    return (n_items + r - 1) / r * kXcds;
}
__device__ __forceinline__ bool xcd_item(int L, int n_items, int n_heads, int &item, int &head) {
    const int x = L % kXcds, j = L / kXcds;
    if (n_heads % kXcds == 0) {
        const int per = n_heads / kXcds;   // heads per XCD
        item = j / per;
        head = x + kXcds * (j % per);
    } else if (kXcds % n_heads == 0) {
        const int r = kXcds / n_heads;
        head = x % n_heads;
        item = j * r + x / n_heads;
    } else {
        item = L % n_items;
        head = L / n_items;
    }
    return item < n_items;
}

// Zero the bf16 elements of an 8-wide group whose key (key0 + e) lies outside [lo, hi).
__device__ __forceinline__ u32x4 mask_keys8(u32x4 v, int key0, int lo, int hi) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const int k = key0 + 2 * w;
        uint32_t m = 0;
        if (k >= lo && k < hi) m |= 0x0000FFFFu;
        if (k + 1 >= lo && k + 1 < hi) m |= 0xFFFF0000u;
        v[w] &= m;
    }
    return v;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) x = fmaxf(x, __shfl_xor(x, s));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) x += __shfl_xor(x, s);
    return x;
}

// ============================================================================================== KV append
//
// One work group per (group of 16 consecutive tokens of the step, kv head). K rows are copied in 16-byte chunks.
// V goes into d-major pages. The group is cut into runs of R = min(16, page size) tokens; a run whose tokens fill R
// consecutive, R-aligned offsets of one page (the usual case inside a prefill chunk) gives every d-row of that page
// R contiguous elements, written as 16-byte stores. With R = 16 both halves of a 32-byte d-row come from the same
// work group, so whole 32-byte pieces of memory are written. Tokens outside such runs are written element by
// element. Tokens whose slot is negative or outside the pool are skipped.

constexpr int kAppendGroup = 16;
constexpr int kAppendThreads = 256;

template <typename T>
__device__ __forceinline__ void append_group(T *__restrict__ kc, T *__restrict__ vc, const T *__restrict__ kn,
                                             const T *__restrict__ vn, const int32_t *__restrict__ slots,
                                             int num_tokens, int num_pages, int P, int Hkv, int D, int group, int g) {
    constexpr int E = 16 / sizeof(T);   // elements per 16 bytes
    constexpr int TG = kAppendGroup;
    __shared__ int64_t s_slot[TG];
    __shared__ int s_run[TG];           // run r is a whole aligned run inside one page
    const int64_t t0 = int64_t(group) * TG;
    const int nt = int(min(int64_t(TG), int64_t(num_tokens) - t0));
    const int64_t pool = int64_t(num_pages) * P;
    const int R = min(TG, P);
    if (threadIdx.x < TG) {
        int64_t sl = threadIdx.x < nt ? int64_t(slots[t0 + threadIdx.x]) : -1;
        s_slot[threadIdx.x] = (sl >= 0 && sl < pool) ? sl : -1;
    }
    __syncthreads();
    if (threadIdx.x < TG / R) {
        const int i0 = threadIdx.x * R;
        const int64_t s0 = s_slot[i0];
        bool ok = R * int(sizeof(T)) >= 16 && i0 + R <= nt && s0 >= 0 && (s0 % P) % R == 0;
        for (int i = 1; i < R; ++i) ok = ok && s_slot[i0 + i] == s0 + i;
        s_run[threadIdx.x] = ok;
    }
    __syncthreads();
    // Each pass issues all of a thread's loads (one K chunk; E tokens of one V d-row, a wave covering 64
    // consecutive d) before its stores, so a work group waits for memory about once per pass.
    const int cpr = D / E;             // 16-byte chunks per K row
    const int nk = nt * cpr;           // K chunks
    const int nv = (TG / E) * D;       // V chunks of E tokens
    for (int base = 0; base < max(nk, nv); base += blockDim.x) {
        const int c = base + int(threadIdx.x);
        u32x4 kval = {0, 0, 0, 0};
        int64_t kdst = -1;
        if (c < nk) {
            const int i = c / cpr, cc = c % cpr;
            const int64_t slot = s_slot[i];
            if (slot >= 0) {
                kval = load16(kn + ((t0 + i) * Hkv + g) * D + int64_t(cc) * E);
                kdst = ((slot / P * Hkv + g) * P + slot % P) * D + int64_t(cc) * E;
            }
        }
        const int qa = c / D, d = c % D;
        const int i0 = qa * E;   // first token of the V chunk
        const bool vact = c < nv && i0 < nt;
        T vals[E];
#pragma unroll
        for (int e = 0; e < E; ++e)
            vals[e] = (vact && i0 + e < nt) ? vn[((t0 + i0 + e) * Hkv + g) * D + d] : T(0);
        if (kdst >= 0) store16(kc + kdst, kval);
        if (!vact) continue;
        if (s_run[i0 / R]) {
            const int64_t s0 = s_slot[i0];
            store16(vc + ((s0 / P * Hkv + g) * D + d) * P + s0 % P, *reinterpret_cast<const u32x4 *>(vals));
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const int64_t slot = i0 + e < nt ? s_slot[i0 + e] : -1;
                if (slot >= 0) vc[((slot / P * Hkv + g) * D + d) * P + slot % P] = vals[e];
            }
        }
    }
}

template <typename T>
__global__ __launch_bounds__(kAppendThreads) void kv_append_kernel(T *__restrict__ kc, T *__restrict__ vc,
                                                                   const T *__restrict__ kn, const T *__restrict__ vn,
                                                                   const int32_t *__restrict__ slots, int num_tokens,
                                                                   int num_pages, int P, int Hkv, int D) {
    append_group(kc, vc, kn, vn, slots, num_tokens, num_pages, P, Hkv, D, int(blockIdx.x), int(blockIdx.y));
}

// ============================================================================================ page copies
//
// Whole pages between two page arrays (cache <-> contiguous swap buffer, or cache <-> cache): page i goes from
// src[src_pages[i]] to dst[dst_pages[i]] (a null list means page i itself). One work group per (page, 16 KB piece);
// every thread moves four 16-byte chunks with streaming loads. Pairs with an index outside its array are skipped.

constexpr int kCopyPiece = 16384;   // bytes per work group

__global__ __launch_bounds__(256) void copy_pages_kernel(uint8_t *__restrict__ dst, const int32_t *__restrict__ dst_pages,
                                                         int dst_slots, const uint8_t *__restrict__ src,
                                                         const int32_t *__restrict__ src_pages, int src_slots,
                                                         int64_t page_bytes) {
    const int i = blockIdx.x;
    const int sp = src_pages ? src_pages[i] : i;
    const int dp = dst_pages ? dst_pages[i] : i;
    if (sp < 0 || sp >= src_slots || dp < 0 || dp >= dst_slots) return;
    const int64_t lo = int64_t(blockIdx.y) * kCopyPiece;
    const int64_t hi = min(page_bytes, lo + kCopyPiece);
    const uint8_t *s = src + int64_t(sp) * page_bytes;
    uint8_t *d = dst + int64_t(dp) * page_bytes;
    u32x4 v[4];
    int64_t o = lo + 16 * threadIdx.x;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        if (o + 4096 * k < hi) v[k] = load16_stream(s + o + 4096 * k);
#pragma unroll
    for (int k = 0; k < 4; ++k)
        if (o + 4096 * k < hi) store16(d + o + 4096 * k, v[k]);
}

// ===================================================================== split-KV decode (bf16, MFMA 16x16x32)
//
// Work group = one (decode row split, kv head); 4 waves take the split's 32-key tiles round-robin and merge their
// online-softmax states through LDS at the end. All G query heads of the kv head ride in the N dimension of the
// MFMAs (padded to 16), so each K/V byte is read once for the whole group.
//
// Per 32-key tile and wave:
//   scores  S[key][head] = K[key][:] . Q[head][:]      2 x D/32 MFMAs; A = K rows, B = Q^T
//   output  O[d][head]  += V^T[d][key] . P[key][head]  D/16 MFMAs;     A = V^T (d-major page), B = P^T
// MFMA 16x16x32 bf16 operands: lane l holds A[l%16][8(l/16) .. +8] and B[8(l/16) .. +8][l%16]; the result gives
// lane l the entries [4(l/16) .. +4][l%16]. The key order inside the tile is permuted so that after the QK product
// lane l owns the scores of keys 8(l/16) .. 8(l/16)+7 for head l%16 -- exactly its B operand of the PV product --
// and a V^T operand of 8 consecutive keys is one 16-byte load.

constexpr int kDecodeMaxPages = 1040;   // page ids of one decode split staged in LDS (split / page + 2)

// decode splits of at least this many keys run the decode kernel with one tile in flight per wave (see decode_kernel)
constexpr int kDecodeSingleBufferSplit = 2560;

template <int D>
struct DecodeTile {
    u32x4 k[2][D / 32];   // K rows of both 16-key halves, d = 32kb + 8(l/16) .. +8
    u32x4 v[D / 16];      // V^T rows d = 16b + l%16, keys 8(l/16) .. +8
};

// NBUF: 32-key K/V tiles each wave holds in registers. Two (one computed while the next loads) at two work groups
// per CU; one at three work groups per CU, which the launch picks for long splits (kDecodeSingleBufferSplit).
template <int D, int NBUF>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NBUF == 2 ? 2 : 3, NBUF == 2 ? 2 : 3))) void decode_kernel(const uint16_t *__restrict__ q, uint16_t *__restrict__ out,
                                                     const uint16_t *__restrict__ kc, const uint16_t *__restrict__ vc,
                                                     const int32_t *__restrict__ block_table, int table_width,
                                                     int num_pages, const int32_t *__restrict__ items,
                                                     float *__restrict__ part_o, float *__restrict__ part_ml, int Hq,
                                                     int Hkv, int P_log2, float scale_log2e, int n_decode_groups,
                                                     uint16_t *kc_w, uint16_t *vc_w, const uint16_t *kn,
                                                     const uint16_t *vn, const int32_t *slots, int num_new,
                                                     const int32_t *__restrict__ counts) {
    constexpr int KB = D / 32;   // QK MFMAs per 16-key half tile
    constexpr int DB = D / 16;   // PV MFMAs (16 d-rows each)
    __shared__ float sm_o[4][D][17];
    __shared__ float sm_m[4][16];
    __shared__ float sm_l[4][16];
    __shared__ int sm_page[kDecodeMaxPages];
    __shared__ __attribute__((aligned(16))) uint16_t sm_new[2][D];   // the row's own new K and V (fused append)

    // Fused append (kn != null): the work groups after the decode work groups write the step's new K/V into the
    // caches, running in the decode tail. Decode rows then must not read their own new key from the cache, where it
    // may not have landed yet: the work group whose split ends at the row's position takes it from kn / vn.
    if (int(blockIdx.x) >= n_decode_groups) {
        const int L = int(blockIdx.x) - n_decode_groups;
        append_group(kc_w, vc_w, kn, vn, slots, num_new, num_pages, 1 << P_log2, Hkv, D, L / Hkv, L % Hkv);
        return;
    }

    // the kv head varies fastest in the linear block index, so work groups start in the plan's heaviest-first order
    // across all heads (blocks are dispatched in index order)
    const int item = int(blockIdx.x) / Hkv;
    const int g = int(blockIdx.x) - item * Hkv;
    if (counts && item >= counts[0]) return;   // a launch sized for a capacity: past the step's decode items
    const int32_t *it = items + int64_t(item) * 8;
    const int r = it[0], t = it[1], pos = it[2], kv_lo = it[3], kv_hi = it[4], slot = it[5], ring = it[6];
    const bool own_new = kn != nullptr && kv_hi == pos + 1;
    const int G = Hq / Hkv;
    const int P = 1 << P_log2;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15;   // head in the group (N index) and A row index
    const int rg = lane >> 4;    // 0..3

    // the split's page ids, once, into LDS
    const int blk0 = kv_lo >> P_log2;
    {
        const int32_t *bt = block_table + int64_t(r) * table_width;
        const int nblk = ((kv_hi - 1) >> P_log2) - blk0 + 1;
        for (int i = threadIdx.x; i < nblk; i += 256) sm_page[i] = lookup_page(bt, blk0 + i, ring, num_pages);
    }

    if (own_new && threadIdx.x < D / 4) {   // 16-byte pieces of the new K row, then of the new V row
        const int half = int(threadIdx.x) / (D / 8), c = int(threadIdx.x) % (D / 8);
        const uint16_t *src = (half ? vn : kn) + (int64_t(t) * Hkv + g) * D + 8 * c;
        *reinterpret_cast<u32x4 *>(&sm_new[half][8 * c]) = load16(src);
    }

    // Q as the B operand of the QK product: head `col`, d = 32kb + 8rg .. +8
    bf16x8 qf[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        u32x4 v = {0, 0, 0, 0};
        if (col < G) v = load16(q + (int64_t(t) * Hq + g * G + col) * D + 32 * kb + 8 * rg);
        qf[kb] = as_bf16x8(v);
    }
    __syncthreads();

    // K row handled by this lane in each half tile: A row `col` of half hf holds key 8(col/4) + 4hf + col%4
    const int krow0 = 8 * (col >> 2) + (col & 3);
    const int64_t head_k = int64_t(g) * P * D;      // offset of kv head g inside a K page
    const int64_t head_v = int64_t(g) * D * P;      // and inside a V page
    const int64_t page_elems = int64_t(Hkv) * P * D;

    auto load_tile = [&](int tile, DecodeTile<D> &b) {
        const int base = tile << 5;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const int key = base + krow0 + 4 * hf;
            if (key >= kv_lo && key < kv_hi) {
                const int page = sm_page[(key >> P_log2) - blk0];
                const uint16_t *src = kc + page * page_elems + head_k + int64_t(key & (P - 1)) * D + 8 * rg;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) b.k[hf][kb] = load16_stream(src + 32 * kb);
            } else {
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) b.k[hf][kb] = u32x4{0, 0, 0, 0};
            }
        }
        const int key8 = base + 8 * rg;
        if (key8 + 8 > kv_lo && key8 < kv_hi) {
            const int first = key8 < kv_lo ? kv_lo : key8;   // any valid key of the group locates the page
            const int page = sm_page[(first >> P_log2) - blk0];
            const uint16_t *src = vc + page * page_elems + head_v + int64_t(col) * P + (key8 & (P - 1));
#pragma unroll
            for (int bb = 0; bb < DB; ++bb) b.v[bb] = load16_stream(src + int64_t(16 * bb) * P);
        } else {
#pragma unroll
            for (int bb = 0; bb < DB; ++bb) b.v[bb] = u32x4{0, 0, 0, 0};
        }
    };

    float m = kNegInf, l = 0.f;
    f32x4 acc[DB];
#pragma unroll
    for (int bb = 0; bb < DB; ++bb) acc[bb] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute_tile = [&](int tile, DecodeTile<D> &b) {
        const int base = tile << 5;
        const int key8 = base + 8 * rg;
        const bool edge = base < kv_lo || base + 32 > kv_hi;
        if (own_new && tile == (pos >> 5)) {   // the row's own new key: K row and V column from the staged copy
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
                if (base + krow0 + 4 * hf == pos)
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb)
                        b.k[hf][kb] = *reinterpret_cast<const u32x4 *>(&sm_new[0][32 * kb + 8 * rg]);
            if (pos >= key8 && pos < key8 + 8) {
                const int e = pos - key8;
#pragma unroll
                for (int bb = 0; bb < DB; ++bb) {
                    const uint32_t v = sm_new[1][16 * bb + col];
                    u32x4 x = b.v[bb];
                    const uint32_t w = x[e >> 1];
                    x[e >> 1] = (e & 1) ? ((w & 0x0000FFFFu) | (v << 16)) : ((w & 0xFFFF0000u) | v);
                    b.v[bb] = x;
                }
            }
        }
        if (edge) {
#pragma unroll
            for (int bb = 0; bb < DB; ++bb) b.v[bb] = mask_keys8(b.v[bb], key8, kv_lo, kv_hi);
        }
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(b.k[0][kb]), qf[kb], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(b.k[1][kb]), qf[kb], s1, 0, 0, 0);
        }
        float s[8];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            s[u] = s0[u] * scale_log2e;
            s[4 + u] = s1[u] * scale_log2e;
        }
        if (edge) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int key = key8 + e;
                if (key < kv_lo || key >= kv_hi) s[e] = kNegInf;
            }
        }
        // online softmax for head `col` (its 32 keys sit in lanes col, col+16, col+32, col+48)
        float tmax = s[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) tmax = fmaxf(tmax, s[e]);
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float m_new = fmaxf(m, tmax);
        const float m_use = m_new == kNegInf ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m - m_use);
        bf16x8 pf;
        float psum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float p = __builtin_amdgcn_exp2f(s[e] - m_use);
            psum += p;
            pf[e] = static_cast<__bf16>(p);
        }
        l = l * alpha + psum;
        m = m_new;
#pragma unroll
        for (int bb = 0; bb < DB; ++bb) {
            acc[bb] *= alpha;
            acc[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(b.v[bb]), pf, acc[bb], 0, 0, 0);
        }
    };

    // tiles of 32 keys, round-robin over the 4 waves; the next tile's loads are in flight while one is computed
    const int tile_last = (kv_hi - 1) >> 5;
    int tile = (kv_lo >> 5) + wave;
    if constexpr (NBUF == 2) {
        if (tile <= tile_last) {
            DecodeTile<D> ta, tb;
            load_tile(tile, ta);
            while (true) {
                const int t1 = tile + 4;
                if (t1 <= tile_last) load_tile(t1, tb);
                compute_tile(tile, ta);
                if (t1 > tile_last) break;
                const int t2 = t1 + 4;
                if (t2 <= tile_last) load_tile(t2, ta);
                compute_tile(t1, tb);
                if (t2 > tile_last) break;
                tile = t2;
            }
        }
    } else {
        for (; tile <= tile_last; tile += 4) {
            DecodeTile<D> ta;
            load_tile(tile, ta);
            compute_tile(tile, ta);
        }
    }
    // ---- per-wave totals, then merge the 4 waves
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (rg == 0) {
        sm_m[wave][col] = m;
        sm_l[wave][col] = l;
    }
#pragma unroll
    for (int bb = 0; bb < DB; ++bb)
#pragma unroll
        for (int u = 0; u < 4; ++u) sm_o[wave][16 * bb + 4 * rg + u][col] = acc[bb][u];
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * D; idx += 256) {
        const int n = idx / D, d = idx % D;
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_m[w][n]);
        float L = 0.f, O = 0.f;
        if (M != kNegInf) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float f = __builtin_amdgcn_exp2f(sm_m[w][n] - M);
                L += sm_l[w][n] * f;
                O += sm_o[w][d][n] * f;
            }
        }
        const int h = g * G + n;
        if (slot < 0) {
            out[(int64_t(t) * Hq + h) * D + d] = f32_to_bf16(L > 0.f ? O / L : 0.f);
        } else {
            part_o[(int64_t(slot) * Hq + h) * D + d] = O;
            if (d == 0) {
                part_ml[(int64_t(slot) * Hq + h) * 2 + 0] = M;
                part_ml[(int64_t(slot) * Hq + h) * 2 + 1] = L;
            }
        }
    }
}

// ========================================================================= general per-token kernel (VALU)
//
// One wave per (token split, kv head, group of up to 16 query heads). Used for fp32 and for shapes the MFMA
// kernels do not cover. Keys are taken 64 at a time, one per lane: each lane computes its key's scores for all the
// group's heads; the wave then folds the chunk into the running softmax, and the lanes switch to one d each for
// the weighted sum of V.

template <typename T>
__device__ __forceinline__ float to_f32(T x);
template <>
__device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ float to_f32<uint16_t>(uint16_t x) { return bf16_to_f32(x); }
template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ uint16_t from_f32<uint16_t>(float x) { return f32_to_bf16(x); }

template <typename T, int D>
__global__ __launch_bounds__(64) void rowwise_kernel(const T *__restrict__ q, T *__restrict__ out,
                                                     const T *__restrict__ kc, const T *__restrict__ vc,
                                                     const int32_t *__restrict__ block_table, int table_width,
                                                     int num_pages, const int32_t *__restrict__ items,
                                                     float *__restrict__ part_o, float *__restrict__ part_ml, int Hq,
                                                     int Hkv, int P_log2, float scale_log2e,
                                                     const int32_t *__restrict__ counts) {
    constexpr int HG = 16;        // query heads per wave
    if (counts && int(blockIdx.x) >= counts[2]) return;
    constexpr int DPL = D / 64;   // d values per lane in the V sum
    __shared__ float sq[HG][D];
    __shared__ float sp[HG][64];

    const int32_t *it = items + int64_t(blockIdx.x) * 8;
    const int r = it[0], t = it[1], kv_lo = it[3], kv_hi = it[4], slot = it[5], ring = it[6];
    const int g = blockIdx.y;
    const int G = Hq / Hkv;
    const int h0 = blockIdx.z * HG;
    const int nh = min(HG, G - h0);
    const int P = 1 << P_log2;
    const int lane = threadIdx.x;
    const int32_t *bt = block_table + int64_t(r) * table_width;

    for (int idx = lane; idx < HG * D; idx += 64) {
        const int n = idx / D, d = idx % D;
        sq[n][d] = n < nh ? to_f32(q[(int64_t(t) * Hq + g * G + h0 + n) * D + d]) : 0.f;
    }
    __syncthreads();

    float m[HG], l[HG], acc[HG][DPL];
#pragma unroll
    for (int n = 0; n < HG; ++n) {
        m[n] = kNegInf;
        l[n] = 0.f;
#pragma unroll
        for (int j = 0; j < DPL; ++j) acc[n][j] = 0.f;
    }

    for (int base = kv_lo; base < kv_hi; base += 64) {
        const int key = base + lane;
        float s[HG];
#pragma unroll
        for (int n = 0; n < HG; ++n) s[n] = 0.f;
        if (key < kv_hi) {
            const int page = lookup_page(bt, key >> P_log2, ring, num_pages);
            const T *krow = kc + ((int64_t(page) * Hkv + g) * P + (key & (P - 1))) * D;
            for (int d = 0; d < D; ++d) {
                const float kv = to_f32(krow[d]);
#pragma unroll
                for (int n = 0; n < HG; ++n) s[n] = fmaf(sq[n][d], kv, s[n]);
            }
        }
        const int nkeys = min(64, kv_hi - base);
#pragma unroll
        for (int n = 0; n < HG; ++n) {
            const float sc = key < kv_hi ? s[n] * scale_log2e : kNegInf;
            const float cmax = wave_max(sc);
            const float m_new = fmaxf(m[n], cmax);
            const float alpha = exp2f(m[n] - m_new);
            const float p = exp2f(sc - m_new);
            l[n] = l[n] * alpha + wave_sum(p);
            m[n] = m_new;
            sp[n][lane] = p;
#pragma unroll
            for (int j = 0; j < DPL; ++j) acc[n][j] *= alpha;
        }
        __syncthreads();
        for (int j = 0; j < nkeys; ++j) {
            const int kk = base + j;
            const int page = lookup_page(bt, kk >> P_log2, ring, num_pages);
            const T *vcol = vc + (int64_t(page) * Hkv + g) * D * P + (kk & (P - 1));
#pragma unroll
            for (int jj = 0; jj < DPL; ++jj) {
                const float vv = to_f32(vcol[int64_t(lane + 64 * jj) * P]);
#pragma unroll
                for (int n = 0; n < HG; ++n) acc[n][jj] = fmaf(sp[n][j], vv, acc[n][jj]);
            }
        }
        __syncthreads();
    }
    for (int n = 0; n < nh; ++n) {
        const int h = g * G + h0 + n;
#pragma unroll
        for (int jj = 0; jj < DPL; ++jj) {
            const int d = lane + 64 * jj;
            if (slot < 0) {
                out[(int64_t(t) * Hq + h) * D + d] = from_f32<T>(l[n] > 0.f ? acc[n][jj] / l[n] : 0.f);
            } else {
                part_o[(int64_t(slot) * Hq + h) * D + d] = acc[n][jj];
            }
        }
        if (slot >= 0 && lane == 0) {
            part_ml[(int64_t(slot) * Hq + h) * 2 + 0] = m[n];
            part_ml[(int64_t(slot) * Hq + h) * 2 + 1] = l[n];
        }
    }
}

// ======================================================================= prefill tiles (bf16, MFMA 32x32x16)
//
// Work group = one (tile of query tokens x the G heads of a kv head = 32 NW rows, KV range, kv head); rows are
// token-major (row = token * G + head) and each of the NW waves owns 32 of them. Every SIMD runs two waves: two
// 4-wave work groups share a CU (128-row tiles), or one 8-wave work group has it alone (256-row tiles, where each K/V
// tile copied into LDS serves twice the rows). Either way one wave's softmax arithmetic runs beside the other's
// matrix work. Per 64-key tile and wave:
//   S^T[key][row] = K[key][:] . Q[row][:]         A = K rows (LDS), B = Q^T (registers)   2 halves x D/16 MFMAs
//   O^T[d][row]  += V^T[d][key] . P^T[key][row]   A = V^T (LDS), B = P^T (registers)      4 k-steps x D/32 MFMAs
// MFMA 32x32x16 bf16 operands: lane l holds A[l%32][8(l/32) .. +8] and B[8(l/32) .. +8][l%32]; the result gives lane l
// column l%32 and rows 8(v/4) + 4(l/32) + v%4 for v = 0..15. The K rows of a 32-key half are fed with bits 2 and 3 of
// the key index swapped, so that lane l's 16 scores are keys 8(l/32) + 16kk + 0..7 (kk = 0, 1): each group of 8 is
// one B operand of the PV product.
//
// LDS holds the K and V^T tiles in 1 KB blocks. Each block is filled by one direct global->LDS copy (lane L's 16 bytes
// land at offset 16 L) and read back with 16-byte reads at offset 16 l, so fills and reads are linear and
// conflict-free, and each copy reads one page (pages of >= 16 keys: the page id is wave-uniform and the address is
// scalar; with 8-key pages a copy spans two):
//   K block (half s, k-step pair p, key quarter qq): slot 32 kbp + 16 h + j = K[32s + 16qq + j][16(2p + kbp) + 8h ..]
//   V block (k-step kk, d block b):                 slot 32 h + i          = V^T[32b + i][16kk + 8h ..]
// Key quarter qq (keys 16qq .. 16qq + 15 of the tile: its K blocks and V k-step qq) is copied by wave qq, or with 8
// waves by waves qq and qq + 4, each taking half of the quarter's blocks.
//
// Per tile, with the next tile's copies in flight (double buffering):
//   QK(half 0) | QK(half 1) beside softmax(half 0) | PV(half 0) beside softmax(half 1) | PV(half 1)
// Softmax in the log2 domain with a lazily moved running maximum: the weights are computed speculatively against the
// current maximum, and only when some row's weights could exceed 2^8 (its sum does) does a rare path move
// it, rescale that row's accumulators and recompute the weights. Tiles every row sees completely skip the mask.
// Q is multiplied by scale * log2(e) once, when it is loaded, and rounded to bf16; the score accumulators start at
// -mu (mu: the running maximum, 0 before the row has one), so the QK product yields each weight's exponent and the
// common path spends one exp2 and no other arithmetic per score.

constexpr int kPfKeys = 64;    // keys per tile
constexpr int kPrefillMaxPages = 1536;   // page ids of one prefill item staged in LDS (split / page + 2)
// the running maximum may lag 8 (log2 units) behind the true one: a half's weight sum above 2^8 sends the row to the
// rare path
constexpr float kWeightSumBound = 256.f;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Sum of 8 bf16 values in fp32 (the same rounded weights the PV product uses).
__device__ __forceinline__ float sum_bf16x8(bf16x8 p, float acc) {
    const bf16x2 one = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bf16x2 pr = {p[2 * i], p[2 * i + 1]};
        acc = __builtin_amdgcn_fdot2_f32_bf16(pr, one, acc, false);
    }
    return acc;
}

// Direct global -> LDS copy of 16 bytes per lane: lane L's bytes land at lds_base + 16 L (lds_base wave-uniform).
__device__ __forceinline__ void load_lds16(const void *src, void *lds_base) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                     (__attribute__((address_space(3))) void *)lds_base, 16, 0, 0);
}
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)

// max of x over lanes l and l ^ 32
__device__ __forceinline__ float max_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <int D, int PL, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_kernel(
    const uint16_t *__restrict__ q, uint16_t *__restrict__ out, const uint16_t *__restrict__ kc,
    const uint16_t *__restrict__ vc, const int32_t *__restrict__ block_table, int table_width, int num_pages,
    const int32_t *__restrict__ items, int n_items, float *__restrict__ part_o, float *__restrict__ part_ml, int Hq,
    int Hkv, float scale_log2e, int window_left, const int32_t *__restrict__ counts) {
    constexpr int P = 1 << PL;
    constexpr int KB = D / 16;          // k-steps of the QK product
    constexpr int DB = D / 32;          // 32-row d blocks of the output
    constexpr int NK = KB / 2;          // K blocks per key quarter
    constexpr int KQ = NW / 4;          // waves sharing the copies of one key quarter
    constexpr int NT = NW * 64;         // threads
    static_assert((NW == 4 || NW == 8) && NK % KQ == 0 && DB % KQ == 0, "copies must split evenly over the waves");
    constexpr int KT = 2 * KB * 1024;   // one K tile (64 keys)
    constexpr int VT = 4 * DB * 1024;   // one V tile (64 keys)
    // distinct LDS objects per buffer: the copies streaming into one provably do not alias reads of the other, so
    // the compiler does not wait for them before reading
    __shared__ __attribute__((aligned(1024))) uint8_t s_k0[KT];
    __shared__ __attribute__((aligned(1024))) uint8_t s_k1[KT];
    __shared__ __attribute__((aligned(1024))) uint8_t s_v0[VT];
    __shared__ __attribute__((aligned(1024))) uint8_t s_v1[VT];
    __shared__ int s_pages[kPrefillMaxPages];

    int item, g;
    if (!xcd_item(blockIdx.x, n_items, Hkv, item, g)) return;
    if (counts && item >= counts[1]) return;   // a launch sized for a capacity: past the step's prefill items
    const int32_t *it = items + int64_t(item) * 8;
    const int r = it[0], t0 = it[1], pos0 = it[2], qc = it[3], kv_lo = it[4], kv_hi = it[5];
    const int slot_base = it[6], ring = it[7];
    const int G = Hq / Hkv;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c32 = lane & 31, h = lane >> 5;
    const int32_t *bt = block_table + int64_t(r) * table_width;
    const int64_t page_elems = int64_t(Hkv) * P * D;
    const uint16_t *kc_g = kc + int64_t(g) * P * D;
    const uint16_t *vc_g = vc + int64_t(g) * D * P;
    auto lo_of = [&](int p) { return window_left < 0 ? 0 : max(0, p - window_left); };

    // this lane's row and the keys it sees; a row that sees nothing gets an empty range
    const int row = 32 * w + c32;
    const int ti = row / G, hn = row - ti * G;
    const bool ok = ti < qc;
    int rlo, rspan;
    {
        const int pos = pos0 + ti;
        const int lo = max(kv_lo, lo_of(pos)), hi = min(pos, kv_hi - 1);
        const bool none = !ok || hi < lo;
        rlo = none ? 0x7fffffff : lo;
        rspan = none ? 0 : hi - lo;
    }

    // keys any row of the group sees; tiles every row sees completely need no mask
    const int ulo = max(kv_lo, lo_of(pos0));
    const int uhi = min(kv_hi, pos0 + qc);   // exclusive
    const int lo_max = max(kv_lo, lo_of(pos0 + qc - 1));
    const int hi_min = min(pos0, kv_hi - 1);
    const int tile_first = ulo / kPfKeys;
    const int ntiles = uhi > ulo ? (uhi - 1) / kPfKeys - tile_first + 1 : 0;
    auto clean = [&](int tile) { return tile * kPfKeys >= lo_max && tile * kPfKeys + kPfKeys - 1 <= hi_min; };
    auto needs_vfix = [&](int tile) { return tile * kPfKeys < ulo || tile * kPfKeys + kPfKeys > uhi; };

    float m = kNegInf, l = 0.f;
    f32x16 acc[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[b][v] = 0.f;

    if (ntiles > 0) {
        // ---- the item's page ids into LDS
        const int blk0 = ulo >> PL;
        const int nblk = ((uhi - 1) >> PL) - blk0 + 1;
        for (int i = tid; i < nblk; i += NT) s_pages[i] = lookup_page(bt, blk0 + i, ring, num_pages);
        // keys outside the item's blocks read the nearest staged page: a real page of the pool, so the copy stays in
        // bounds; those keys are masked (K) or zeroed (V) before use
        auto page_at = [&](int key) { return s_pages[min(max((key >> PL) - blk0, 0), nblk - 1)]; };

        // ---- copies of one tile into LDS: wave w copies its part (w / 4) of key quarter w % 4
        const int qw = w & 3, part = w >> 2;
        const int k_cp = (lane & (P >= 16 ? 15 : 7)) * D + 16 * (lane >> 5) + 8 * ((lane >> 4) & 1);
        const int v_cp = (lane & 31) * P + (P >= 16 ? 8 * (lane >> 5) : 0);
        auto issue_k = [&](int tile, uint8_t *kbuf) {
            const int key0 = tile * kPfKeys + 16 * qw;
            uint8_t *dst = kbuf + ((qw >> 1) * NK * 2 + (qw & 1)) * 1024;
            const uint16_t *src;
            if constexpr (P >= 16) {
                const int pg = __builtin_amdgcn_readfirstlane(page_at(key0));
                src = kc_g + int64_t(pg) * page_elems + (key0 & (P - 1)) * D + k_cp;
            } else {
                const int pg = page_at(key0 + 8 * ((lane >> 3) & 1));
                src = kc_g + int64_t(pg) * page_elems + k_cp;
            }
#pragma unroll
            for (int i = 0; i < NK / KQ; ++i) {
                const int p = part * (NK / KQ) + i;
                load_lds16(src + 32 * p, dst + p * 2048);
            }
        };
        auto issue_v = [&](int tile, uint8_t *vbuf) {
            const int key0 = tile * kPfKeys + 16 * qw;
            uint8_t *dst = vbuf + qw * DB * 1024;
            const uint16_t *src;
            if constexpr (P >= 16) {
                const int pg = __builtin_amdgcn_readfirstlane(page_at(key0));
                src = vc_g + int64_t(pg) * page_elems + (key0 & (P - 1)) + v_cp;
            } else {
                const int pg = page_at(key0 + 8 * h);
                src = vc_g + int64_t(pg) * page_elems + v_cp;
            }
#pragma unroll
            for (int i = 0; i < DB / KQ; ++i) {
                const int b = part * (DB / KQ) + i;
                load_lds16(src + 32 * b * P, dst + b * 1024);
            }
        };
        // zero V^T entries of keys outside [ulo, uhi) (their pages may hold anything, NaN included)
        auto fix_v = [&](int tile, uint8_t *vbuf) {
            for (int e = tid; e < 4 * DB * 64; e += NT) {
                const int key8 = tile * kPfKeys + 16 * ((e >> 6) / DB) + 8 * ((e >> 5) & 1);
                if (key8 >= ulo && key8 + 8 <= uhi) continue;
                u32x4 *p = reinterpret_cast<u32x4 *>(vbuf + e * 16);
                *p = mask_keys8(*p, key8, ulo, uhi);
            }
        };

        // ---- compute pieces
        const int krow = (((c32 >> 3) & 1) << 2) | (((c32 >> 2) & 1) << 3) | (c32 & ~12);   // bits 2, 3 swapped
        const int k_rd = (c32 >> 4) * 1024 + (16 * h + (krow & 15)) * 16;
        // this lane's Q row as B operands of the QK product: Q[row][16kb + 8h .. +8]
        bf16x8 qf[KB];
        {
            const uint16_t *qrow = q + (int64_t(t0 + ti) * Hq + g * G + hn) * D + 8 * h;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                u32x4 v = {0, 0, 0, 0};
                if (ok) v = load16(qrow + 16 * kb);
                const bf16x8 raw = as_bf16x8(v);
                bf16x8 sc;
#pragma unroll
                for (int e = 0; e < 8; ++e) sc[e] = static_cast<__bf16>(static_cast<float>(raw[e]) * scale_log2e);
                qf[kb] = sc;
            }
        }
        // the score accumulators start at -mu_c, so that S = scale log2(e) q.k - mu_c is the exponent of the weight;
        // mu_c is the running maximum m, or 0 while the row has none
        float mu_c = 0.f;
        f32x16 cm;
#pragma unroll
        for (int v = 0; v < 16; ++v) cm[v] = 0.f;
        // S^T of one 32-key half
        auto qk_half = [&](const uint8_t *kbuf, int s, f32x16 &S) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const bf16x8 a = as_bf16x8(load16(kbuf + k_rd + (s * NK + kb / 2) * 2048 + (kb & 1) * 512));
                S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kb], kb == 0 ? cm : S, 0, 0, 0);
            }
        };
        // O^T += V^T P^T over one 32-key half (k-steps 2s, 2s+1)
        auto pv_half = [&](const uint8_t *vbuf, int s, const bf16x8 (&pf)[2]) {
            const uint8_t *v_rd = vbuf + lane * 16;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int b = 0; b < DB; ++b) {
                    const bf16x8 a = as_bf16x8(load16(v_rd + ((2 * s + kk) * DB + b) * 1024));
                    acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kk], acc[b], 0, 0, 0);
                }
        };
        // scores of keys the row does not see -> -inf (tiles on the causal diagonal or at the window's edge)
        auto mask_half = [&](f32x16 &S, int key_base) {
            const int base = key_base + 8 * h - rlo;
#pragma unroll
            for (int v = 0; v < 16; ++v)
                if (unsigned(base + 16 * (v >> 3) + (v & 7)) > unsigned(rspan)) S[v] = kNegInf;
        };
        auto weights = [&](const f32x16 &S, float delta, bool shift, bf16x8 (&pf)[2]) {
            float sum = 0.f;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                bf16x8 p;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    p[e] = static_cast<__bf16>(__builtin_amdgcn_exp2f(shift ? S[8 * kk + e] + delta : S[8 * kk + e]));
                pf[kk] = p;
                sum = sum_bf16x8(p, sum);
            }
            return sum;
        };
        // Softmax of one half against the current running maximum (speculative): the bf16 weights (the B operands
        // of the PV product) and their sum. The weights are trusted when the row already has a maximum and their sum
        // stays below kWeightSumBound, which bounds every weight; otherwise (first visible keys of the row, or scores
        // that climbed past the running maximum) the rare path below settles the row. No row maximum is computed on
        // the common path.
        auto softmax_half = [&](const f32x16 &S, bf16x8 (&pf)[2], float &lsum) {
            lsum = weights(S, 0.f, false, pf);
            // pin the speculative results here, beside the matrix work of this region: otherwise the compiler sinks
            // them past the rare-path branch that follows and they no longer overlap the MFMAs
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                u32x4 t = __builtin_bit_cast(u32x4, pf[kk]);
                asm volatile("" : "+v"(t));
                pf[kk] = as_bf16x8(t);
            }
            asm volatile("" : "+v"(lsum));
            // !(lsum <= bound) also catches a sum that overflowed to inf or NaN
            return (m == kNegInf && lsum > 0.f) || !(lsum <= kWeightSumBound);
        };
        // Rare path for the rows that asked for it: take the half's true row maximum (both lanes of the row), move
        // the running maximum up to it if it is higher, rescale the row's accumulators and recompute its weights.
        // Scores already computed against the old mu_c (this half, and `other`: the tile's second half when the first
        // is settled) are shifted to the new one, and later tiles' accumulators start at the new -mu_c.
        auto settle = [&](bool want, f32x16 &S, bf16x8 (&pf)[2], float &lsum, f32x16 *other) {
            // a loop of at most one trip rather than a branch, so that the compiler keeps the rescale out of line
            const int trips = __builtin_amdgcn_ballot_w64(want) ? 1 : 0;
#pragma nounroll
            for (int t = 0; t < trips; ++t) {
                float x = S[0];
#pragma unroll
                for (int v = 1; v < 16; ++v) x = __builtin_elementwise_maximum(x, S[v]);
                // the partner lane of the row decides too: both see the same maximum
                const float tmax = max_xor32(x) + mu_c;
                const bool bump = __shfl_xor(int(want), 32) != 0 || want;
                const float m_new = bump ? fmaxf(m, tmax) : m;
                const float alpha = m_new > m ? __builtin_amdgcn_exp2f(m - m_new) : 1.f;
                l *= alpha;
#pragma unroll
                for (int b = 0; b < DB; ++b) acc[b] *= alpha;
                m = m_new;
                const float mu_new = m_new == kNegInf ? 0.f : m_new;
                const float delta = mu_c - mu_new;
                lsum = weights(S, delta, true, pf);
                if (other) {
#pragma unroll
                    for (int v = 0; v < 16; ++v) (*other)[v] += delta;
                }
                mu_c = mu_new;
#pragma unroll
                for (int v = 0; v < 16; ++v) cm[v] = -mu_c;
            }
            l += lsum;
        };

        // One tile from (kcur, vcur); the next tile's copies go to (knxt, vnxt).
        auto tile = [&](int j, const uint8_t *kcur, const uint8_t *vcur, uint8_t *knxt, uint8_t *vnxt) {
            const int tile = tile_first + j;
            const bool more = j + 1 < ntiles;
            const bool edge = !clean(tile);
            if (more) {
                issue_k(tile + 1, knxt);
                issue_v(tile + 1, vnxt);
            }
            f32x16 S0, S1;
            bf16x8 p0[2], p1[2];
            float ls0, ls1;
            // the compute of a tile runs at raised wave priority: while this work group's waves compute, the other
            // work group on the CU, if it is copying, waiting or at its barrier, does not take issue slots first
            __builtin_amdgcn_s_setprio(1);
            qk_half(kcur, 0, S0);
            if (edge) mask_half(S0, tile * kPfKeys);
            qk_half(kcur, 1, S1);
            const bool b0 = softmax_half(S0, p0, ls0);
            settle(b0, S0, p0, ls0, &S1);
            if (edge) mask_half(S1, tile * kPfKeys + 32);
            pv_half(vcur, 0, p0);
            const bool b1 = softmax_half(S1, p1, ls1);
            settle(b1, S1, p1, ls1, nullptr);
            pv_half(vcur, 1, p1);
            __builtin_amdgcn_s_setprio(0);
            // the next tile has landed for every wave; every wave is done with this one
            wait_vmem();
            __syncthreads();
            if (more && needs_vfix(tile + 1)) {
                fix_v(tile + 1, vnxt);
                __syncthreads();
            }
        };

        // ---- the first tile into LDS, then the tiles (buffers named statically: the loop is unrolled by two)
        __syncthreads();   // page ids
        issue_k(tile_first, s_k0);
        issue_v(tile_first, s_v0);
        wait_vmem();
        __syncthreads();
        if (needs_vfix(tile_first)) {
            fix_v(tile_first, s_v0);
            __syncthreads();
        }
        for (int j = 0; j < ntiles; j += 2) {
            tile(j, s_k0, s_v0, s_k1, s_v1);
            if (j + 1 < ntiles) tile(j + 1, s_k1, s_v1, s_k0, s_v0);
        }
    }

    // ---- results: lane holds O^T[d][row] for d = 32b + 8(v/4) + 4h + v%4
    l += __shfl_xor(l, 32);
    if (!ok) return;
    const int hh = g * G + hn;
    const int tok = t0 + ti;
    if (slot_base < 0) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        uint16_t *orow = out + (int64_t(tok) * Hq + hh) * D;
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) {
                const int d = 32 * b + 8 * v4 + 4 * h;
                const uint32_t lo2 = uint32_t(f32_to_bf16(acc[b][4 * v4 + 0] * inv)) |
                                     uint32_t(f32_to_bf16(acc[b][4 * v4 + 1] * inv)) << 16;
                const uint32_t hi2 = uint32_t(f32_to_bf16(acc[b][4 * v4 + 2] * inv)) |
                                     uint32_t(f32_to_bf16(acc[b][4 * v4 + 3] * inv)) << 16;
                *reinterpret_cast<uint2 *>(orow + d) = make_uint2(lo2, hi2);
            }
    } else {
        const int64_t sl = int64_t(slot_base) + ti;
        float *po = part_o + (sl * Hq + hh) * D;
#pragma unroll
        for (int b = 0; b < DB; ++b)
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) {
                const int d = 32 * b + 8 * v4 + 4 * h;
                *reinterpret_cast<f32x4 *>(po + d) =
                    f32x4{acc[b][4 * v4 + 0], acc[b][4 * v4 + 1], acc[b][4 * v4 + 2], acc[b][4 * v4 + 3]};
            }
        if (h == 0) {
            part_ml[(sl * Hq + hh) * 2 + 0] = m;
            part_ml[(sl * Hq + hh) * 2 + 1] = l;
        }
    }
}

// =========================================================================================== merge of splits
//
// out = sum_s O_s 2^(m_s - M) / sum_s l_s 2^(m_s - M), M = max_s m_s, for each (token, head). One work group per
// (merged token, group of 256 / (D/4) heads): each thread owns (head, 4 consecutive d), so the split maxima and sums
// it needs and its 16-byte partial rows are independent loads that all go out at once.

template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(T *__restrict__ out, const float *__restrict__ part_o,
                                                      const float *__restrict__ part_ml,
                                                      const int32_t *__restrict__ items, int Hq, int D,
                                                      const int32_t *__restrict__ counts) {
    if (counts && int(blockIdx.x) >= counts[3]) return;
    const int32_t *it = items + int64_t(blockIdx.x) * 4;
    const int t = it[0], first = it[1], n = it[2], stride = it[3];
    const int quads = D / 4;
    const int h = blockIdx.y * (256 / quads) + threadIdx.x / quads;
    const int d = 4 * (threadIdx.x % quads);
    if (h >= Hq) return;
    // both loops are unrolled so that several splits' loads are in flight at once: the merge is latency-bound
    float M = kNegInf;
#pragma unroll 4
    for (int s = 0; s < n; ++s) M = fmaxf(M, part_ml[((int64_t(first) + int64_t(s) * stride) * Hq + h) * 2]);
    float L = 0.f;
    f32x4 O = {0.f, 0.f, 0.f, 0.f};
    if (M != kNegInf) {
#pragma unroll 4
        for (int s = 0; s < n; ++s) {
            const int64_t sl = int64_t(first) + int64_t(s) * stride;
            const float f = exp2f(part_ml[(sl * Hq + h) * 2] - M);
            L += part_ml[(sl * Hq + h) * 2 + 1] * f;
            O += *reinterpret_cast<const f32x4 *>(part_o + (sl * Hq + h) * D + d) * f;
        }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    T *o = out + (int64_t(t) * Hq + h) * D + d;
    T res[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) res[e] = from_f32<T>(O[e] * inv);
    if constexpr (sizeof(T) == 2) {
        *reinterpret_cast<uint2 *>(o) = *reinterpret_cast<const uint2 *>(res);
    } else {
        *reinterpret_cast<u32x4 *>(o) = *reinterpret_cast<const u32x4 *>(res);
    }
}

inline int ilog2(int x) {
    int s = 0;
    while ((1 << s) < x) ++s;
    return s;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool shape_ok(const cb_attn_shape &s) {
    return s.num_q_heads > 0 && s.num_kv_heads > 0 && s.num_q_heads % s.num_kv_heads == 0 &&
           (s.head_dim == 64 || s.head_dim == 128) && s.page_size >= 1 && s.page_size <= 256 &&
           (s.page_size & (s.page_size - 1)) == 0 && (s.dtype == CB_DTYPE_F32 || s.dtype == CB_DTYPE_BF16) &&
           s.window_left >= -1;
}

}  // namespace

// A kernel launch on stream `s`, the call's launch number `k_launch` of `n_launch`. The call's first kernel records
// the caller's start event when it begins executing and its last kernel the stop event when it ends
// (hipExtLaunchKernel), so that the pair times the kernels themselves: events recorded on the stream around the call
// would also count the dispatch after the previous work and the completion signal after the last kernel.
#define CB_LAUNCH(K, GRID, BLOCK, ...)                                                                         \
    do {                                                                                                       \
        hipEvent_t ev_a = k_launch == 0 ? ev_start : nullptr;                                                  \
        hipEvent_t ev_b = k_launch == n_launch - 1 ? ev_stop : nullptr;                                        \
        if (ev_a || ev_b)                                                                                      \
            hipExtLaunchKernelGGL(K, GRID, BLOCK, 0, s, ev_a, ev_b, 0, __VA_ARGS__);                           \
        else                                                                                                   \
            hipLaunchKernelGGL(K, GRID, BLOCK, 0, s, __VA_ARGS__);                                              \
        ++k_launch;                                                                                            \
    } while (0)

// Launch of the append kernel over all tokens (sizes already checked); the events as for CB_LAUNCH, with this
// launch as a call's only one.
static hipError_t launch_append(void *k_cache, void *v_cache, const void *k_new, const void *v_new, const int32_t *slots,
                         int32_t num_tokens, int32_t num_pages, int32_t page_size, int32_t num_kv_heads,
                         int32_t head_dim, int32_t dtype, hipStream_t s, hipEvent_t ev_start = nullptr,
                         hipEvent_t ev_stop = nullptr) {
    int k_launch = 0;
    const int n_launch = 1;
    const int64_t groups = (int64_t(num_tokens) + kAppendGroup - 1) / kAppendGroup;
    const dim3 grid{static_cast<unsigned>(groups), static_cast<unsigned>(num_kv_heads), 1u};
    if (dtype == CB_DTYPE_F32) {
        CB_LAUNCH(kv_append_kernel<float>, grid, dim3(kAppendThreads), static_cast<float *>(k_cache),
                  static_cast<float *>(v_cache), static_cast<const float *>(k_new),
                  static_cast<const float *>(v_new), slots, num_tokens, num_pages, page_size, num_kv_heads, head_dim);
    } else {
        CB_LAUNCH(kv_append_kernel<uint16_t>, grid, dim3(kAppendThreads), static_cast<uint16_t *>(k_cache),
                  static_cast<uint16_t *>(v_cache), static_cast<const uint16_t *>(k_new),
                  static_cast<const uint16_t *>(v_new), slots, num_tokens, num_pages, page_size, num_kv_heads,
                  head_dim);
    }
    return hipGetLastError();
}

// ================================================================================================== C ABI

extern "C" cb_status cb_kv_append(void *k_cache, void *v_cache, const void *k_new, const void *v_new,
                                  const int32_t *d_slot_mapping, int32_t num_tokens, int32_t num_pages,
                                  int32_t page_size, int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                                  int32_t layout, void *stream) {
    if (num_tokens < 0 || num_pages < 1 || page_size < 1 || num_kv_heads < 1 || head_dim < 1) return CB_E_INVAL;
    if (dtype != CB_DTYPE_F32 && dtype != CB_DTYPE_BF16) return CB_E_UNSUPPORTED;
    if (layout != CB_LAYOUT_KD_VT) return CB_E_UNSUPPORTED;
    const int esz = dtype == CB_DTYPE_F32 ? 4 : 2;
    if ((head_dim * esz) % 16 != 0) return CB_E_UNSUPPORTED;
    if (num_tokens == 0) return CB_OK;
    if (!k_cache || !v_cache || !k_new || !v_new || !d_slot_mapping) return CB_E_INVAL;
    const int64_t groups = (int64_t(num_tokens) + kAppendGroup - 1) / kAppendGroup;
    if (groups > INT32_MAX || num_kv_heads > 65535) return CB_E_UNSUPPORTED;
    return launch_append(k_cache, v_cache, k_new, v_new, d_slot_mapping, num_tokens, num_pages, page_size,
                         num_kv_heads, head_dim, dtype, static_cast<hipStream_t>(stream)) == hipSuccess
               ? CB_OK
               : CB_E_HIP;
}

extern "C" cb_status cb_kv_copy_pages(void *dst, const int32_t *d_dst_pages, int32_t dst_slots, const void *src,
                                      const int32_t *d_src_pages, int32_t src_slots, int32_t n, int64_t page_bytes,
                                      void *stream) {
    if (n < 0 || dst_slots < 0 || src_slots < 0 || page_bytes < 16 || page_bytes % 16 != 0) return CB_E_INVAL;
    if (n == 0) return CB_OK;
    if (!dst || !src) return CB_E_INVAL;
    if (!d_dst_pages && n > dst_slots) return CB_E_INVAL;
    if (!d_src_pages && n > src_slots) return CB_E_INVAL;
    const int64_t pieces = (page_bytes + kCopyPiece - 1) / kCopyPiece;
    if (pieces > 65535) return CB_E_UNSUPPORTED;
    const dim3 grid{static_cast<unsigned>(n), static_cast<unsigned>(pieces), 1u};
    hipLaunchKernelGGL(copy_pages_kernel, grid, dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<uint8_t *>(dst), d_dst_pages, dst_slots, static_cast<const uint8_t *>(src),
                       d_src_pages, src_slots, page_bytes);
    return hipGetLastError() == hipSuccess ? CB_OK : CB_E_HIP;
}

extern "C" size_t cb_paged_attention_workspace_size(const cb_attn_args *a) {
    if (!a) return 0;
    const size_t n = size_t(a->plan_info.n_partials);
    const size_t hq = size_t(a->shape.num_q_heads), d = size_t(a->shape.head_dim);
    if (n == 0) return 0;
    return align256(n * hq * d * sizeof(float)) + align256(n * hq * 2 * sizeof(float));
}

extern "C" cb_status cb_paged_attention(const cb_attn_args *a, void *stream) {
    if (!a || a->phases < 0 || a->phases > 15) return CB_E_INVAL;
    const cb_attn_shape &sh = a->shape;
    const cb_plan &pl = a->plan_info;
    if (!shape_ok(sh) || a->layout != CB_LAYOUT_KD_VT) return CB_E_UNSUPPORTED;
    if (pl.n_decode < 0 || pl.n_prefill < 0 || pl.n_rowwise < 0 || pl.n_combine < 0 || pl.n_partials < 0)
        return CB_E_INVAL;
    const int64_t n_work = int64_t(pl.n_decode) + pl.n_prefill + pl.n_rowwise + pl.n_combine;
    if (n_work == 0) {   // nothing to launch: the timing events are recorded where the kernels would have run
        for (void *ev : {a->timing_start, a->timing_stop})
            if (ev && hipEventRecord(static_cast<hipEvent_t>(ev), static_cast<hipStream_t>(stream)) != hipSuccess)
                return CB_E_HIP;
        return CB_OK;
    }
    if (!a->out || !a->q || !a->k_cache || !a->v_cache || !a->block_table || !a->plan) return CB_E_INVAL;
    if (a->num_pages < 1 || a->table_width <= pl.max_page_index) return CB_E_INVAL;
    const int Hq = sh.num_q_heads, Hkv = sh.num_kv_heads, D = sh.head_dim;
    const int G = Hq / Hkv;
    const bool bf16 = sh.dtype == CB_DTYPE_BF16;
    if ((pl.n_decode > 0 || pl.n_prefill > 0) && (!bf16 || sh.page_size < 8)) return CB_E_INVAL;
    if (pl.n_decode > 0 && (G > 16 || pl.decode_split / sh.page_size + 2 > kDecodeMaxPages)) return CB_E_INVAL;
    // prefill tiles: prefill_tokens tokens x G heads = 128 rows (4-wave work groups) or 256 (8 waves)
    const int64_t pf_rows = int64_t(pl.prefill_tokens) * G;
    if (pl.n_prefill > 0 && (pl.prefill_tokens < 1 || (pf_rows != 128 && pf_rows != 256) ||
                             pl.prefill_split / sh.page_size + 2 > kPrefillMaxPages))
        return CB_E_INVAL;
    const size_t need = cb_paged_attention_workspace_size(a);
    if (need > 0 && (!a->workspace || a->workspace_bytes < need)) return CB_E_WORKSPACE;
    // fused append: the call that runs the first cache-reading phase of the plan also appends the step's new K/V
    const bool fuse = a->k_new != nullptr;
    if (fuse && (!a->v_new || !a->slot_mapping || a->num_new != pl.num_tokens)) return CB_E_INVAL;
    const int first_reader = pl.n_decode > 0    ? CB_PHASE_DECODE
                             : pl.n_rowwise > 0 ? CB_PHASE_ROWWISE
                             : pl.n_prefill > 0 ? CB_PHASE_PREFILL
                                                : 0;
    float *part_o = static_cast<float *>(a->workspace);
    float *part_ml = need ? reinterpret_cast<float *>(static_cast<char *>(a->workspace) +
                                                      align256(size_t(pl.n_partials) * Hq * D * sizeof(float)))
                          : nullptr;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipEvent_t ev_start = static_cast<hipEvent_t>(a->timing_start), ev_stop = static_cast<hipEvent_t>(a->timing_stop);
    const int Pl = ilog2(sh.page_size);
    const float sl2e = a->scale * 1.4426950408889634f;   // scale * log2(e): softmax in base 2
    const int32_t *plan = a->plan;
    const int32_t ph = a->phases == 0 ? (CB_PHASE_DECODE | CB_PHASE_ROWWISE | CB_PHASE_PREFILL | CB_PHASE_COMBINE)
                                      : a->phases;

    const bool append_here = fuse && (ph & first_reader) != 0;
    // the launches this call makes, in order (the timing events go to the first and the last)
    const bool l_dec = pl.n_decode > 0 && (ph & CB_PHASE_DECODE);
    const bool l_row = pl.n_rowwise > 0 && (ph & CB_PHASE_ROWWISE);
    const bool l_pre = pl.n_prefill > 0 && (ph & CB_PHASE_PREFILL);
    const bool l_com = pl.n_combine > 0 && (ph & CB_PHASE_COMBINE);
    const int n_launch = int(l_dec) + int(!l_dec && append_here) + int(l_row) + int(l_pre) + int(l_com);
    int k_launch = 0;
    const int64_t append_groups = append_here ? (int64_t(a->num_new) + kAppendGroup - 1) / kAppendGroup * Hkv : 0;
    if (int64_t(pl.n_decode) * Hkv + append_groups > INT32_MAX) return CB_E_UNSUPPORTED;
    if (l_dec) {
        // with the fused append, its work groups follow the decode work groups in the same grid
        const int n_dec = pl.n_decode * Hkv;
        const dim3 grid{unsigned(n_dec + append_groups), 1u, 1u};
        const uint16_t *qq = static_cast<const uint16_t *>(a->q);
        uint16_t *oo = static_cast<uint16_t *>(a->out);
        const uint16_t *kk = static_cast<const uint16_t *>(a->k_cache);
        const uint16_t *vv = static_cast<const uint16_t *>(a->v_cache);
        uint16_t *kw = append_here ? static_cast<uint16_t *>(const_cast<void *>(a->k_cache)) : nullptr;
        uint16_t *vw = append_here ? static_cast<uint16_t *>(const_cast<void *>(a->v_cache)) : nullptr;
        const uint16_t *kn = append_here ? static_cast<const uint16_t *>(a->k_new) : nullptr;
        const uint16_t *vn = append_here ? static_cast<const uint16_t *>(a->v_new) : nullptr;
        const int32_t *sm = append_here ? a->slot_mapping : nullptr;
        // long splits: one tile in flight per wave and three work groups per CU; short ones: two tiles per wave
        const bool single = pl.decode_split >= kDecodeSingleBufferSplit;
#define CB_DECODE(DD, NB)                                                                                         \
    CB_LAUNCH((decode_kernel<DD, NB>), grid, dim3(256), qq, oo, kk, vv, a->block_table, a->table_width, a->num_pages, \
              plan + pl.off_decode, part_o, part_ml, Hq, Hkv, Pl, sl2e, n_dec, kw, vw, kn, vn, sm, a->num_new, a->counts)
        if (D == 128) {
            if (single)
                CB_DECODE(128, 1);
            else
                CB_DECODE(128, 2);
        } else {
            if (single)
                CB_DECODE(64, 1);
            else
                CB_DECODE(64, 2);
        }
#undef CB_DECODE
    } else if (append_here) {
        // the plan's first cache reader is the per-token or the prefill kernel: append on its own launch first
        const hipError_t e = launch_append(const_cast<void *>(a->k_cache), const_cast<void *>(a->v_cache), a->k_new,
                                           a->v_new, a->slot_mapping, a->num_new, a->num_pages, sh.page_size, Hkv, D,
                                           sh.dtype, s, k_launch == 0 ? ev_start : nullptr,
                                           k_launch == n_launch - 1 ? ev_stop : nullptr);
        ++k_launch;
        if (e != hipSuccess)
            return CB_E_HIP;
    }
    if (l_row) {
        const dim3 grid(unsigned(pl.n_rowwise), unsigned(Hkv), unsigned((G + 15) / 16));
#define CB_ROWWISE(T, DD)                                                                                         \
    CB_LAUNCH((rowwise_kernel<T, DD>), grid, dim3(64), static_cast<const T *>(a->q), static_cast<T *>(a->out),  \
              static_cast<const T *>(a->k_cache), static_cast<const T *>(a->v_cache), a->block_table,          \
              a->table_width, a->num_pages, plan + pl.off_rowwise, part_o, part_ml, Hq, Hkv, Pl, sl2e, a->counts)
        if (bf16) {
            if (D == 128) CB_ROWWISE(uint16_t, 128); else CB_ROWWISE(uint16_t, 64);
        } else {
            if (D == 128) CB_ROWWISE(float, 128); else CB_ROWWISE(float, 64);
        }
#undef CB_ROWWISE
    }
    if (l_pre) {
        const dim3 grid(unsigned(xcd_grid(pl.n_prefill, Hkv)));
        const uint16_t *qq = static_cast<const uint16_t *>(a->q);
        uint16_t *oo = static_cast<uint16_t *>(a->out);
        const uint16_t *kk = static_cast<const uint16_t *>(a->k_cache);
        const uint16_t *vv = static_cast<const uint16_t *>(a->v_cache);
        const bool wide = pf_rows == 256;   // 8-wave work groups
#define CB_PREFILL(DD, PLOG)                                                                                   \
    if (wide)                                                                                                  \
        CB_LAUNCH((prefill_kernel<DD, PLOG, 8>), grid, dim3(512), qq, oo, kk, vv, a->block_table, a->table_width, \
                  a->num_pages, plan + pl.off_prefill, pl.n_prefill, part_o, part_ml, Hq, Hkv, sl2e,             \
                  sh.window_left, a->counts);                                                                  \
    else                                                                                                       \
        CB_LAUNCH((prefill_kernel<DD, PLOG, 4>), grid, dim3(256), qq, oo, kk, vv, a->block_table, a->table_width, \
                  a->num_pages, plan + pl.off_prefill, pl.n_prefill, part_o, part_ml, Hq, Hkv, sl2e,             \
                  sh.window_left, a->counts)
#define CB_PREFILL_D(DD)                                                                                       \
    switch (Pl) {                                                                                              \
        case 3: CB_PREFILL(DD, 3); break;                                                                      \
        case 4: CB_PREFILL(DD, 4); break;                                                                      \
        case 5: CB_PREFILL(DD, 5); break;                                                                      \
        case 6: CB_PREFILL(DD, 6); break;                                                                      \
        case 7: CB_PREFILL(DD, 7); break;                                                                      \
        default: CB_PREFILL(DD, 8); break;                                                                     \
    }
        if (D == 128) {
            CB_PREFILL_D(128)
        } else {
            CB_PREFILL_D(64)
        }
#undef CB_PREFILL_D
#undef CB_PREFILL
    }
    if (l_com) {
        const int heads_per_group = 256 / (D / 4);
        const dim3 grid(unsigned(pl.n_combine), unsigned((Hq + heads_per_group - 1) / heads_per_group));
        if (bf16)
            CB_LAUNCH(combine_kernel<uint16_t>, grid, dim3(256), static_cast<uint16_t *>(a->out), part_o, part_ml,
                      plan + pl.off_combine, Hq, D, a->counts);
        else
            CB_LAUNCH(combine_kernel<float>, grid, dim3(256), static_cast<float *>(a->out), part_o, part_ml,
                      plan + pl.off_combine, Hq, D, a->counts);
    }
    // a call whose phases launch no kernel still records the timing events, where its kernels would have run
    if (n_launch == 0) {
        if (ev_start && hipEventRecord(ev_start, s) != hipSuccess) return CB_E_HIP;
        if (ev_stop && hipEventRecord(ev_stop, s) != hipSuccess) return CB_E_HIP;
    }
    return hipGetLastError() == hipSuccess ? CB_OK : CB_E_HIP;
}

// ============================================================================ allocation-free entry point
//
// The same launches as cb_paged_attention, with the partial results of split rows kept in `scratch`, a static
// device array of fixed size: one copy per device, allocated when the code object is loaded and held until the
// process ends. Host code never passes `scratch` itself to a kernel (in host code the name stands for a host-side
// shadow, not a device address): its device address is taken once per device with hipGetSymbolAddress and kept
// in g_scratch. Every split slot is written by the work group that owns it before the merge reads it, so nothing in
// the array has to start at zero; two calls that overlap on one device share the array and race.

static __device__ __align__(256) uint8_t scratch[CB_NOALLOC_WORKSPACE_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices];   // device address of `scratch` on each device, looked up at the first call there
}  // namespace

extern "C" cb_status cb_paged_attention_noalloc(const cb_attn_args *a, void *stream) {
    if (!a) return CB_E_INVAL;
    if (cb_paged_attention_workspace_size(a) > size_t(CB_NOALLOC_WORKSPACE_BYTES)) return CB_E_WORKSPACE;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CB_E_HIP;
    if (stream) {   // the scratch address below is the current device's: the stream must belong to it
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess) return CB_E_HIP;
        if (int(sdev) != dev) return CB_E_INVAL;
    }
    void *ptr = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        if (!g_scratch[dev]) {
            void *p = nullptr;
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CB_E_HIP;
            g_scratch[dev] = p;
        }
        ptr = g_scratch[dev];
    }
    cb_attn_args b = *a;
    b.workspace = ptr;
    b.workspace_bytes = size_t(CB_NOALLOC_WORKSPACE_BYTES);
    return cb_paged_attention(&b, stream);
}
