// Global dedup across lists into a compacted pool (README "60+ inference
// optimizations & kernels", section "4-bit KV cache": dedup compaction, read
// across all lists at once).  Every entry of every list is translated as the
// attention kernels translate it; U = the distinct valid slots in increasing
// order; cpool row i = pool row U[i]; each entry is rewritten as the index of
// its slot in U (-1 when skipped).  Attention over cpool with the rewritten
// lists as physical slots then gathers from |U| contiguous rows instead of
// scattered ones and equals attention over the original, entry for entry.
//
// A bitmap over the pool's slots carries the set.  Launches mark the entries
// (when the bitmap fits in 64 KB, each workgroup into an LDS copy stored as a
// partial bitmap, then OR-ed together; otherwise one global atomic per entry
// into a cleared bitmap), scan it (per word, then per block of 4096 words,
// then over the blocks: inside the rewrite's workgroups when there are at
// most 1024 blocks, else a launch of its own), list U and rewrite the
// entries (a slot's index is
// its block's base plus its word's base plus the set bits below it in the
// word; for small bitmaps the rewrite is a launch of its own that reads the
// word table from LDS), and copy the rows, one 16-byte piece per lane.
#include "kv4_device.h"
#include "kv4_launch.h"

#include <algorithm>

namespace kv4 {

constexpr int kCompactThreads = 256;
constexpr int kScanWords = 4096;                 // bitmap words per scan block
constexpr int kLdsMarkWords = 16384;             // bitmaps up to 64 KB are marked in LDS first
constexpr int kMarkThreads = 512;                // LDS marking: lanes per workgroup,
constexpr int kMarkParts = 512;                  // at most this many workgroups (partial bitmaps),
constexpr int kMarkPer = 32;                     // and entries per lane per round
constexpr int kEmitPer = 4;                      // entries per lane when rewriting the lists
constexpr int kLdsEmitWords = 8192;              // word tables up to 64 KB are read from LDS when rewriting
constexpr int kInlineBlocks = 1024;              // up to this many scan blocks, each rewriting workgroup
                                                 // scans the block totals itself (no launch of its own)

// A query row's translation: through its page-table row, or physical slots
// (no page table), or none at all (its request lies outside the table: every
// entry >= 0 is skipped and flagged).
struct RowCtx {
    const int32_t *pt_row;
    bool bad;
};

__device__ __forceinline__ RowCtx row_ctx(const CompactParams &p, int32_t r) {
    RowCtx c{nullptr, false};
    if (p.page_table) {
        const int32_t req = p.row_req ? p.row_req[r] : r;
        if (req < 0 || req >= p.pt_n_rows)
            c.bad = true;
        else
            c.pt_row = p.page_table + (int64_t)req * p.pt_row_stride;
    }
    return c;
}

// list entry pos of a row -> slot or -1 (flags into err)
__device__ __forceinline__ int64_t entry_slot(const CompactParams &p, const RowCtx &c, int32_t pos, uint32_t &err) {
    if (c.bad) {
        if (pos >= 0) err |= kErrPage;
        return -1;
    }
    return translate_slot(pos, c.pt_row, p.pt_n_pages, p.page_shift, p.n_slots, err);
}

__global__ __launch_bounds__(kCompactThreads) void compact_clear_kernel(uint32_t *__restrict__ bitmap,
                                                                         int64_t n_words) {
    // n_words is a multiple of 4 (the workspace rounds it up)
    for (int64_t i = 4 * ((int64_t)blockIdx.x * kCompactThreads + threadIdx.x); i < n_words;
         i += 4 * (int64_t)gridDim.x * kCompactThreads)
        *reinterpret_cast<uint4 *>(bitmap + i) = uint4{0, 0, 0, 0};
}

// Small pools: workgroup b marks whole rows [b * rows_per_part, ...) into an
// LDS copy of the bitmap (n_words words of dynamic LDS), so repeated slots
// cost LDS atomics only, and stores it as partial bitmap b; a second launch
// ORs the partials into the bitmap.  No global atomics: with a few thousand
// bitmap words shared by every workgroup, they would serialize.
__global__ __launch_bounds__(kMarkThreads) void compact_mark_lds_kernel(CompactParams p, uint32_t *__restrict__ parts,
                                                                         int64_t n_words, int32_t rows_per_part) {
    extern __shared__ uint32_t local[];
    uint32_t err = 0;
    for (int i = threadIdx.x; i < n_words; i += kMarkThreads) local[i] = 0;
    __syncthreads();
    // wavefront w takes rows r0 + w, r0 + w + waves, ...: a row's translation
    // is uniform across the wavefront
    constexpr int kWaves = kMarkThreads / 64;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int32_t r0 = blockIdx.x * rows_per_part, r1 = min(p.n_rows, r0 + rows_per_part);
    for (int32_t r = r0 + wave; r < r1; r += kWaves) {
        const RowCtx c = row_ctx(p, r);
        const int32_t *lst = p.topk + (int64_t)r * p.topk_row_stride;
        for (int32_t j0 = 0; j0 < p.k; j0 += kMarkPer * 64) {
            int32_t pos[kMarkPer];
#pragma unroll
            for (int v = 0; v < kMarkPer; ++v) {
                const int32_t j = j0 + v * 64 + lane;
                pos[v] = j < p.k ? lst[j] : -1;
            }
#pragma unroll
            for (int v = 0; v < kMarkPer; ++v) {
                const int64_t sl = entry_slot(p, c, pos[v], err);
                if (sl >= 0)
                    (void)__hip_atomic_fetch_or(&local[sl >> 5], 1u << (sl & 31), __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_WORKGROUP);
            }
        }
    }
    __syncthreads();
    uint4 *dst = reinterpret_cast<uint4 *>(parts + (int64_t)blockIdx.x * n_words);   // n_words is a multiple of 4
    for (int i = threadIdx.x; 4 * i < n_words; i += kMarkThreads)
        dst[i] = uint4{local[4 * i], local[4 * i + 1], local[4 * i + 2], local[4 * i + 3]};
    if (err && p.err_word) atomicOr(p.err_word, err);
}

// bitmap = OR of the n_parts partial bitmaps: 16 four-word columns per
// workgroup, the partials split over 64 lane groups, eight loads in flight
__global__ __launch_bounds__(1024) void compact_reduce_kernel(const uint32_t *__restrict__ parts, int32_t n_parts,
                                                              int64_t n_words, uint32_t *__restrict__ bitmap) {
    __shared__ uint4 red[64][16];
    const int col = threadIdx.x & 15, grp = threadIdx.x >> 4;
    const int64_t n4 = n_words / 4, q = (int64_t)blockIdx.x * 16 + col;
    uint4 acc{0, 0, 0, 0};
    if (q < n4) {
        const uint4 *src = reinterpret_cast<const uint4 *>(parts) + q;
        for (int32_t b0 = grp; b0 < n_parts; b0 += 64 * 8) {
            uint4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int32_t b = b0 + 64 * u;
                v[u] = b < n_parts ? src[(int64_t)b * n4] : uint4{0, 0, 0, 0};
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                acc.x |= v[u].x;
                acc.y |= v[u].y;
                acc.z |= v[u].z;
                acc.w |= v[u].w;
            }
        }
    }
    red[grp][col] = acc;
    __syncthreads();
    for (int half = 32; half > 0; half >>= 1) {
        if (grp < half) {
            const uint4 o = red[grp + half][col];
            acc.x |= o.x;
            acc.y |= o.y;
            acc.z |= o.z;
            acc.w |= o.w;
            red[grp][col] = acc;
        }
        __syncthreads();
    }
    if (grp == 0 && q < n4) reinterpret_cast<uint4 *>(bitmap)[q] = acc;
}

// Large pools: one global atomic per entry; workgroup b takes row b / chunks,
// entries [256 (b % chunks), +256) of it.
__global__ __launch_bounds__(kCompactThreads) void compact_mark_global_kernel(CompactParams p,
                                                                               uint32_t *__restrict__ bitmap,
                                                                               int32_t chunks) {
    uint32_t err = 0;
    const int32_t r = blockIdx.x / chunks, ch = blockIdx.x - r * chunks;
    const int32_t j = ch * kCompactThreads + threadIdx.x;
    if (j < p.k) {
        const RowCtx c = row_ctx(p, r);
        const int64_t sl = entry_slot(p, c, p.topk[(int64_t)r * p.topk_row_stride + j], err);
        if (sl >= 0) atomicOr(bitmap + (sl >> 5), 1u << (sl & 31));
    }
    if (err && p.err_word) atomicOr(p.err_word, err);
}

// per block of kScanWords words: each word with the exclusive prefix of set
// bits before it (within the block), and the block's total
__global__ __launch_bounds__(kCompactThreads) void compact_scan_kernel(const uint32_t *__restrict__ bitmap,
                                                                        int64_t n_words,
                                                                        uint2 *__restrict__ word_info,
                                                                        uint32_t *__restrict__ block_sum) {
    constexpr int kPer = kScanWords / kCompactThreads;   // 16 consecutive words per lane
    __shared__ uint32_t wave_tot[kCompactThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t w0 = (int64_t)blockIdx.x * kScanWords + (int64_t)tid * kPer;
    uint32_t bits[kPer], sum = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        bits[i] = w0 + i < n_words ? bitmap[w0 + i] : 0u;
        sum += __builtin_popcount(bits[i]);
    }
    uint32_t incl = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t t = __shfl_up(incl, off);
        if (lane >= off) incl += t;
    }
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    uint32_t base = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kCompactThreads / 64; ++w) {
        base += w < wave ? wave_tot[w] : 0u;
        total += wave_tot[w];
    }
    uint32_t run = base + incl - sum;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        if (w0 + i < n_words) word_info[w0 + i] = make_uint2(bits[i], run);
        run += __builtin_popcount(bits[i]);
    }
    if (tid == 0) block_sum[blockIdx.x] = total;
}

// Exclusive prefix of the n_blocks (<= kInlineBlocks) block totals into
// base[] (LDS) by the THREADS lanes of a workgroup, consecutive blocks per
// lane; returns the total |U| in every lane.  Holds a barrier: every lane
// calls it.
template <int THREADS>
__device__ __forceinline__ uint32_t block_prefix_lds(const uint32_t *__restrict__ block_sum, int32_t n_blocks,
                                                     uint32_t *base, uint32_t *wave_tot) {
    constexpr int kPer = kInlineBlocks / THREADS;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint32_t v[kPer], sum = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int b = tid * kPer + i;
        v[i] = b < n_blocks ? block_sum[b] : 0u;
        sum += v[i];
    }
    uint32_t incl = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t t = __shfl_up(incl, off);
        if (lane >= off) incl += t;
    }
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    uint32_t run = 0, total = 0;
#pragma unroll
    for (int w = 0; w < THREADS / 64; ++w) {
        run += w < wave ? wave_tot[w] : 0u;
        total += wave_tot[w];
    }
    run += incl - sum;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int b = tid * kPer + i;
        if (b < n_blocks) base[b] = run;
        run += v[i];
    }
    __syncthreads();
    return total;
}

// one workgroup: exclusive prefix over the blocks, and the total |U|
// (when there are more blocks than the rewriting workgroups scan themselves)
__global__ __launch_bounds__(1024) void compact_top_kernel(const uint32_t *__restrict__ block_sum, int32_t n_blocks,
                                                           uint32_t *__restrict__ block_base,
                                                           int32_t *__restrict__ count) {
    __shared__ uint32_t wave_tot[16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int per = (n_blocks + 1023) / 1024;             // consecutive blocks per lane
    uint32_t sum = 0;
    for (int i = 0; i < per; ++i) {
        const int b = tid * per + i;
        sum += b < n_blocks ? block_sum[b] : 0u;
    }
    uint32_t incl = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t t = __shfl_up(incl, off);
        if (lane >= off) incl += t;
    }
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    uint32_t base = 0, total = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
        base += w < wave ? wave_tot[w] : 0u;
        total += wave_tot[w];
    }
    uint32_t run = base + incl - sum;
    for (int i = 0; i < per; ++i) {
        const int b = tid * per + i;
        if (b < n_blocks) {
            block_base[b] = run;
            run += block_sum[b];
        }
    }
    if (tid == 0) *count = (int32_t)total;
}

// blocks [0, word_blocks): list U (lane per word, its set bits in order);
// the rest: rewrite the entries, block word_blocks + b taking row b / chunks,
// entries [kEmitPer * 256 (b % chunks), ...) of it, kEmitPer per lane.
// INLINE: every workgroup first scans the n_blocks block totals into LDS (and
// workgroup 0 writes |U|); otherwise block_base holds them, from
// compact_top_kernel.
template <bool INLINE>
__global__ __launch_bounds__(kCompactThreads) void compact_emit_kernel(CompactParams p,
                                                                        const uint2 *__restrict__ word_info,
                                                                        int64_t n_words,
                                                                        const uint32_t *__restrict__ block_sum,
                                                                        int32_t n_blocks,
                                                                        const uint32_t *__restrict__ block_base,
                                                                        int64_t word_blocks, int32_t chunks,
                                                                        int32_t *__restrict__ uslots) {
    __shared__ uint32_t s_base[INLINE ? kInlineBlocks : 1];
    __shared__ uint32_t s_wave_tot[kCompactThreads / 64];
    if constexpr (INLINE) {
        const uint32_t total = block_prefix_lds<kCompactThreads>(block_sum, n_blocks, s_base, s_wave_tot);
        if (blockIdx.x == 0 && threadIdx.x == 0) *p.out_count = (int32_t)total;
    }
    auto base_of = [&](int64_t b) { return INLINE ? s_base[b] : block_base[b]; };
    if ((int64_t)blockIdx.x < word_blocks) {
        const int64_t w = (int64_t)blockIdx.x * kCompactThreads + threadIdx.x;
        if (w >= n_words) return;
        const uint2 wi = word_info[w];
        uint32_t bits = wi.x, at = base_of(w / kScanWords) + wi.y;
        while (bits) {
            const int b = __builtin_ctz(bits);
            uslots[at++] = (int32_t)(w * 32 + b);
            bits &= bits - 1;
        }
        return;
    }
    const int64_t bi = (int64_t)blockIdx.x - word_blocks;
    const int32_t r = (int32_t)(bi / chunks), ch = (int32_t)(bi - (int64_t)r * chunks);
    const RowCtx c = row_ctx(p, r);
    const int32_t *lst = p.topk + (int64_t)r * p.topk_row_stride;
    int32_t *out = p.out_idx + (int64_t)r * p.k;
    uint32_t err = 0;                                     // flagged by the marking already
    int32_t j[kEmitPer], pos[kEmitPer];
#pragma unroll
    for (int v = 0; v < kEmitPer; ++v) {
        j[v] = ch * (kEmitPer * kCompactThreads) + v * kCompactThreads + threadIdx.x;
        pos[v] = j[v] < p.k ? lst[j[v]] : -1;
    }
    int64_t sl[kEmitPer];
    uint32_t bits[kEmitPer], base[kEmitPer];
#pragma unroll
    for (int v = 0; v < kEmitPer; ++v) {
        sl[v] = entry_slot(p, c, pos[v], err);
        bits[v] = 0;
        base[v] = 0;
        if (sl[v] >= 0) {
            const int64_t w = sl[v] >> 5;
            const uint2 wi = word_info[w];
            bits[v] = wi.x;
            base[v] = base_of(w / kScanWords) + wi.y;
        }
    }
#pragma unroll
    for (int v = 0; v < kEmitPer; ++v)
        if (j[v] < p.k)
            out[j[v]] = sl[v] >= 0 ? (int32_t)(base[v] + __builtin_popcount(bits[v] & ((1u << (sl[v] & 31)) - 1u)))
                                   : -1;
}

// Small bitmaps (n_words <= kLdsEmitWords): rewrite with the word table in
// LDS, since a gather from a table of a few thousand words touches dozens of
// cache lines per wavefront.  Workgroup b takes rows [b * rows_per_part, ...),
// a wavefront per row as in the marking.
// A word's global base is the sum of the block totals before its block
// (n_words <= kLdsEmitWords: at most two blocks).
__global__ __launch_bounds__(kMarkThreads) void compact_emit_lds_kernel(CompactParams p,
                                                                         const uint2 *__restrict__ word_info,
                                                                         int64_t n_words,
                                                                         const uint32_t *__restrict__ block_sum,
                                                                         int32_t rows_per_part) {
    static_assert(kLdsEmitWords <= 2 * kScanWords, "more than two blocks to sum");
    extern __shared__ uint2 table[];
    for (int i = threadIdx.x; i < n_words; i += kMarkThreads) {
        uint2 wi = word_info[i];
        if (i >= kScanWords) wi.y += block_sum[0];
        table[i] = wi;
    }
    __syncthreads();
    constexpr int kWaves = kMarkThreads / 64;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int32_t r0 = blockIdx.x * rows_per_part, r1 = min(p.n_rows, r0 + rows_per_part);
    uint32_t err = 0;                                     // flagged by the marking already
    for (int32_t r = r0 + wave; r < r1; r += kWaves) {
        const RowCtx c = row_ctx(p, r);
        const int32_t *lst = p.topk + (int64_t)r * p.topk_row_stride;
        int32_t *out = p.out_idx + (int64_t)r * p.k;
        for (int32_t j0 = 0; j0 < p.k; j0 += kMarkPer * 64) {
            int32_t pos[kMarkPer];
#pragma unroll
            for (int v = 0; v < kMarkPer; ++v) {
                const int32_t j = j0 + v * 64 + lane;
                pos[v] = j < p.k ? lst[j] : -1;
            }
#pragma unroll
            for (int v = 0; v < kMarkPer; ++v) {
                const int32_t j = j0 + v * 64 + lane;
                const int64_t sl = entry_slot(p, c, pos[v], err);
                int32_t idx = -1;
                if (sl >= 0) {
                    const uint2 wi = table[sl >> 5];
                    idx = (int32_t)(wi.y + __builtin_popcount(wi.x & ((1u << (sl & 31)) - 1u)));
                }
                if (j < p.k) out[j] = idx;
            }
        }
    }
}

// cpool row i = pool row uslots[i] for i < *count: one 16-byte piece per lane
__global__ __launch_bounds__(kCompactThreads) void compact_copy_kernel(CompactParams p,
                                                                        const int32_t *__restrict__ uslots,
                                                                        const int32_t *__restrict__ count,
                                                                        int64_t max_rows) {
    const int pieces = p.row_bytes / 16;
    const int64_t n = min((int64_t)*count, max_rows) * pieces;
    for (int64_t t = (int64_t)blockIdx.x * kCompactThreads + threadIdx.x; t < n;
         t += (int64_t)gridDim.x * kCompactThreads) {
        const int64_t i = t / pieces;
        const int c = (int)(t - i * pieces);
        const u32x4_t v = *reinterpret_cast<const u32x4_t *>(p.pool + (int64_t)uslots[i] * p.row_bytes + 16 * c);
        *reinterpret_cast<u32x4_t *>(p.cpool + i * p.row_bytes + 16 * c) = v;
    }
}

CompactWorkspace compact_workspace(int64_t n_slots, int32_t n_rows, int32_t k) {
    auto up = [](size_t b) { return (b + 255) / 256 * 256; };
    const int64_t n_entries = (int64_t)n_rows * k;
    CompactWorkspace w;
    w.n_words = ((n_slots + 31) / 32 + 3) / 4 * 4;
    w.n_blocks = (w.n_words + kScanWords - 1) / kScanWords;
    w.max_rows = n_slots < n_entries ? n_slots : n_entries;
    w.n_parts = 0;
    w.rows_per_part = 0;
    if (n_entries > 0 && w.n_words <= kLdsMarkWords) {
        w.rows_per_part = (n_rows + kMarkParts - 1) / kMarkParts;
        w.n_parts = (n_rows + w.rows_per_part - 1) / w.rows_per_part;
    }
    w.bitmap_off = 0;
    w.word_info_off = up((size_t)w.n_words * 4);
    w.block_sum_off = w.word_info_off + up((size_t)w.n_words * 8);
    w.block_base_off = w.block_sum_off + up((size_t)w.n_blocks * 4);
    w.uslots_off = w.block_base_off + up((size_t)w.n_blocks * 4);
    w.parts_off = w.uslots_off + up((size_t)(w.max_rows > 0 ? w.max_rows : 1) * 4);
    w.bytes = w.parts_off + up((size_t)w.n_parts * w.n_words * 4);
    return w;
}

hipError_t launch_global_compact(const CompactParams &p, void *workspace, hipStream_t stream) {
    const CompactWorkspace w = compact_workspace(p.n_slots, p.n_rows, p.k);
    char *ws = static_cast<char *>(workspace);
    uint32_t *bitmap = reinterpret_cast<uint32_t *>(ws + w.bitmap_off);
    uint2 *word_info = reinterpret_cast<uint2 *>(ws + w.word_info_off);
    uint32_t *block_sum = reinterpret_cast<uint32_t *>(ws + w.block_sum_off);
    uint32_t *block_base = reinterpret_cast<uint32_t *>(ws + w.block_base_off);
    int32_t *uslots = reinterpret_cast<int32_t *>(ws + w.uslots_off);
    const int64_t n_entries = (int64_t)p.n_rows * p.k;
    if (w.n_parts > 0) {
        // every bitmap word is written by the reduction: no clearing
        uint32_t *parts = reinterpret_cast<uint32_t *>(ws + w.parts_off);
        hipLaunchKernelGGL(compact_mark_lds_kernel, dim3((unsigned)w.n_parts), dim3(kMarkThreads),
                           (size_t)w.n_words * 4, stream, p, parts, w.n_words, w.rows_per_part);
        hipLaunchKernelGGL(compact_reduce_kernel, dim3((unsigned)((w.n_words / 4 + 15) / 16)), dim3(1024), 0, stream,
                           parts, w.n_parts, w.n_words, bitmap);
    } else {
        const unsigned clear_blocks =
            (unsigned)std::min<int64_t>(2048, (w.n_words / 4 + kCompactThreads - 1) / kCompactThreads);
        if (clear_blocks > 0)
            hipLaunchKernelGGL(compact_clear_kernel, dim3(clear_blocks), dim3(kCompactThreads), 0, stream, bitmap,
                               w.n_words);
        if (n_entries > 0) {
            const int32_t chunks = (p.k + kCompactThreads - 1) / kCompactThreads;
            hipLaunchKernelGGL(compact_mark_global_kernel, dim3((unsigned)((int64_t)p.n_rows * chunks)),
                               dim3(kCompactThreads), 0, stream, p, bitmap, chunks);
        }
    }
    if (w.n_blocks > 0)
        hipLaunchKernelGGL(compact_scan_kernel, dim3((unsigned)w.n_blocks), dim3(kCompactThreads), 0, stream, bitmap,
                           w.n_words, word_info, block_sum);
    // with few blocks the rewriting workgroups scan the block totals themselves
    // (and the first writes |U|); otherwise one workgroup scans them first
    const bool inline_base = w.n_blocks > 0 && w.n_blocks <= kInlineBlocks;
    if (!inline_base)
        hipLaunchKernelGGL(compact_top_kernel, dim3(1), dim3(1024), 0, stream, block_sum, (int32_t)w.n_blocks,
                           block_base, p.out_count);
    const int64_t word_blocks = (w.n_words + kCompactThreads - 1) / kCompactThreads;
    const int32_t chunks = (p.k + kEmitPer * kCompactThreads - 1) / (kEmitPer * kCompactThreads);
    const bool lds_emit = w.n_parts > 0 && w.n_words <= kLdsEmitWords;
    const int64_t entry_blocks = n_entries > 0 && !lds_emit ? (int64_t)p.n_rows * chunks : 0;
    if (lds_emit)
        hipLaunchKernelGGL(compact_emit_lds_kernel, dim3((unsigned)w.n_parts), dim3(kMarkThreads),
                           (size_t)w.n_words * 8, stream, p, word_info, w.n_words, block_sum, w.rows_per_part);
    if (word_blocks + entry_blocks > 0) {
        if (inline_base)
            hipLaunchKernelGGL(compact_emit_kernel<true>, dim3((unsigned)(word_blocks + entry_blocks)),
                               dim3(kCompactThreads), 0, stream, p, word_info, w.n_words, block_sum,
                               (int32_t)w.n_blocks, block_base, word_blocks, chunks, uslots);
        else
            hipLaunchKernelGGL(compact_emit_kernel<false>, dim3((unsigned)(word_blocks + entry_blocks)),
                               dim3(kCompactThreads), 0, stream, p, word_info, w.n_words, block_sum,
                               (int32_t)w.n_blocks, block_base, word_blocks, chunks, uslots);
    }
    if (w.max_rows > 0) {
        const int64_t pieces = w.max_rows * (p.row_bytes / 16);
        const unsigned copy_blocks = (unsigned)std::min<int64_t>(16384, (pieces + kCompactThreads - 1) / kCompactThreads);
        hipLaunchKernelGGL(compact_copy_kernel, dim3(copy_blocks), dim3(kCompactThreads), 0, stream, p, uslots,
                           p.out_count, w.max_rows);
    }
    return hipGetLastError();
}

}  // namespace kv4
