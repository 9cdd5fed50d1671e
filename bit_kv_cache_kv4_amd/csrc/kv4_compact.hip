// Global dedup across lists into a compacted pool (README "60+ inference
// optimizations & kernels", section "4-bit KV cache": dedup compaction, read
// across all lists at once).  Every entry of every list is translated as the
// attention kernels translate it; U = the distinct valid slots in increasing
// order; cpool row i = pool row U[i]; each entry is rewritten as the index of
// its slot in U (-1 when skipped).  Attention over cpool with the rewritten
// lists as physical slots then gathers from |U| contiguous rows instead of
// scattered ones and equals attention over the original, entry for entry.
//
// A bitmap over the pool's slots carries the set: launches clear it, mark the
// entries (through a workgroup-private LDS copy when the bitmap fits in
// 64 KB, so repeated slots cost LDS atomics, not global ones), scan it (per
// word, then per block of 4096 words, then over the blocks), then one launch
// both lists U and rewrites the entries (a slot's index is its block's base
// plus its word's base plus the set bits below it in the word), and a last
// one copies the rows, one 16-byte piece per lane.
#include "kv4_device.h"
#include "kv4_launch.h"

#include <algorithm>

namespace kv4 {

constexpr int kCompactThreads = 256;
constexpr int kScanWords = 4096;                 // bitmap words per scan block
constexpr int kLdsMarkWords = 16384;             // bitmaps up to 64 KB are marked in LDS first
constexpr int kMarkEntries = 8192;               // entries per workgroup of the LDS marking

// entry e = (query row r, list position j) -> slot or -1 (flags into err)
__device__ __forceinline__ int64_t compact_entry_slot(const CompactParams &p, int64_t e, uint32_t &err) {
    const int32_t r = (int32_t)(e / p.k), j = (int32_t)(e - (int64_t)r * p.k);
    const int32_t pos = p.topk[(int64_t)r * p.topk_row_stride + j];
    const int32_t req = p.row_req ? p.row_req[r] : r;
    if (p.page_table && (req < 0 || req >= p.pt_n_rows)) {
        if (pos >= 0) err |= kErrPage;
        return -1;
    }
    const int32_t *pt_row = p.page_table ? p.page_table + (int64_t)req * p.pt_row_stride : nullptr;
    return translate_slot(pos, pt_row, p.pt_n_pages, p.page_shift, p.n_slots, err);
}

__global__ __launch_bounds__(kCompactThreads) void compact_clear_kernel(uint32_t *__restrict__ bitmap,
                                                                         int64_t n_words) {
    // n_words is a multiple of 4 (the workspace rounds it up)
    for (int64_t i = 4 * ((int64_t)blockIdx.x * kCompactThreads + threadIdx.x); i < n_words;
         i += 4 * (int64_t)gridDim.x * kCompactThreads)
        *reinterpret_cast<uint4 *>(bitmap + i) = uint4{0, 0, 0, 0};
}

template <bool LDS>
__global__ __launch_bounds__(kCompactThreads) void compact_mark_kernel(CompactParams p, uint32_t *__restrict__ bitmap,
                                                                        int64_t n_words) {
    __shared__ uint32_t local[LDS ? kLdsMarkWords : 1];
    const int64_t n_entries = (int64_t)p.n_rows * p.k;
    uint32_t err = 0;
    if constexpr (LDS) {
        for (int i = threadIdx.x; i < n_words; i += kCompactThreads) local[i] = 0;
        __syncthreads();
        const int64_t e0 = (int64_t)blockIdx.x * kMarkEntries;
        const int64_t e1 = min(n_entries, e0 + kMarkEntries);
        for (int64_t e = e0 + threadIdx.x; e < e1; e += kCompactThreads) {
            const int64_t s = compact_entry_slot(p, e, err);
            if (s >= 0)
                (void)__hip_atomic_fetch_or(&local[s >> 5], 1u << (s & 31), __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        __syncthreads();
        for (int i = threadIdx.x; i < n_words; i += kCompactThreads)
            if (local[i]) atomicOr(bitmap + i, local[i]);
    } else {
        for (int64_t e = (int64_t)blockIdx.x * kCompactThreads + threadIdx.x; e < n_entries;
             e += (int64_t)gridDim.x * kCompactThreads) {
            const int64_t s = compact_entry_slot(p, e, err);
            if (s >= 0) atomicOr(bitmap + (s >> 5), 1u << (s & 31));
        }
    }
    if (err && p.err_word) atomicOr(p.err_word, err);
}

// per block of kScanWords words: the exclusive prefix of set bits per word
// (within the block) and the block's total
__global__ __launch_bounds__(kCompactThreads) void compact_scan_kernel(const uint32_t *__restrict__ bitmap,
                                                                        int64_t n_words,
                                                                        uint32_t *__restrict__ word_base,
                                                                        uint32_t *__restrict__ block_sum) {
    constexpr int kPer = kScanWords / kCompactThreads;   // 16 consecutive words per lane
    __shared__ uint32_t wave_tot[kCompactThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t w0 = (int64_t)blockIdx.x * kScanWords + (int64_t)tid * kPer;
    uint32_t c[kPer], sum = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        c[i] = w0 + i < n_words ? __builtin_popcount(bitmap[w0 + i]) : 0u;
        sum += c[i];
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
        if (w0 + i < n_words) word_base[w0 + i] = run;
        run += c[i];
    }
    if (tid == 0) block_sum[blockIdx.x] = total;
}

// one workgroup: exclusive prefix over the blocks, and the total |U|
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
// the rest: rewrite the entries (lane per entry)
__global__ __launch_bounds__(kCompactThreads) void compact_emit_kernel(CompactParams p,
                                                                        const uint32_t *__restrict__ bitmap,
                                                                        int64_t n_words,
                                                                        const uint32_t *__restrict__ word_base,
                                                                        const uint32_t *__restrict__ block_base,
                                                                        int64_t word_blocks,
                                                                        int32_t *__restrict__ uslots) {
    if ((int64_t)blockIdx.x < word_blocks) {
        const int64_t w = (int64_t)blockIdx.x * kCompactThreads + threadIdx.x;
        if (w >= n_words) return;
        uint32_t bits = bitmap[w];
        uint32_t at = block_base[w / kScanWords] + word_base[w];
        while (bits) {
            const int b = __builtin_ctz(bits);
            uslots[at++] = (int32_t)(w * 32 + b);
            bits &= bits - 1;
        }
        return;
    }
    const int64_t e = ((int64_t)blockIdx.x - word_blocks) * kCompactThreads + threadIdx.x;
    if (e >= (int64_t)p.n_rows * p.k) return;
    uint32_t err = 0;                                     // flagged by the marking already
    const int64_t s = compact_entry_slot(p, e, err);
    int32_t idx = -1;
    if (s >= 0) {
        const int64_t w = s >> 5;
        idx = (int32_t)(block_base[w / kScanWords] + word_base[w] +
                        __builtin_popcount(bitmap[w] & ((1u << (s & 31)) - 1u)));
    }
    const int32_t r = (int32_t)(e / p.k);
    p.out_idx[(int64_t)r * p.k + (e - (int64_t)r * p.k)] = idx;
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

CompactWorkspace compact_workspace(int64_t n_slots, int64_t n_entries) {
    auto up = [](size_t b) { return (b + 255) / 256 * 256; };
    CompactWorkspace w;
    w.n_words = ((n_slots + 31) / 32 + 3) / 4 * 4;
    w.n_blocks = (w.n_words + kScanWords - 1) / kScanWords;
    w.max_rows = n_slots < n_entries ? n_slots : n_entries;
    w.bitmap_off = 0;
    w.word_base_off = up((size_t)w.n_words * 4);
    w.block_sum_off = w.word_base_off + up((size_t)w.n_words * 4);
    w.block_base_off = w.block_sum_off + up((size_t)w.n_blocks * 4);
    w.uslots_off = w.block_base_off + up((size_t)w.n_blocks * 4);
    w.bytes = w.uslots_off + up((size_t)(w.max_rows > 0 ? w.max_rows : 1) * 4);
    return w;
}

hipError_t launch_global_compact(const CompactParams &p, void *workspace, hipStream_t stream) {
    const CompactWorkspace w = compact_workspace(p.n_slots, (int64_t)p.n_rows * p.k);
    char *ws = static_cast<char *>(workspace);
    uint32_t *bitmap = reinterpret_cast<uint32_t *>(ws + w.bitmap_off);
    uint32_t *word_base = reinterpret_cast<uint32_t *>(ws + w.word_base_off);
    uint32_t *block_sum = reinterpret_cast<uint32_t *>(ws + w.block_sum_off);
    uint32_t *block_base = reinterpret_cast<uint32_t *>(ws + w.block_base_off);
    int32_t *uslots = reinterpret_cast<int32_t *>(ws + w.uslots_off);
    const int64_t n_entries = (int64_t)p.n_rows * p.k;
    const unsigned clear_blocks = (unsigned)std::min<int64_t>(2048, (w.n_words / 4 + kCompactThreads - 1) / kCompactThreads);
    hipLaunchKernelGGL(compact_clear_kernel, dim3(std::max(1u, clear_blocks)), dim3(kCompactThreads), 0, stream,
                       bitmap, w.n_words);
    if (n_entries > 0) {
        if (w.n_words <= kLdsMarkWords) {
            const int64_t blocks = (n_entries + kMarkEntries - 1) / kMarkEntries;
            hipLaunchKernelGGL(compact_mark_kernel<true>, dim3((unsigned)blocks), dim3(kCompactThreads), 0, stream, p,
                               bitmap, w.n_words);
        } else {
            const int64_t blocks = std::min<int64_t>(8192, (n_entries + kCompactThreads - 1) / kCompactThreads);
            hipLaunchKernelGGL(compact_mark_kernel<false>, dim3((unsigned)blocks), dim3(kCompactThreads), 0, stream, p,
                               bitmap, w.n_words);
        }
    }
    if (w.n_blocks > 0)
        hipLaunchKernelGGL(compact_scan_kernel, dim3((unsigned)w.n_blocks), dim3(kCompactThreads), 0, stream, bitmap,
                           w.n_words, word_base, block_sum);
    hipLaunchKernelGGL(compact_top_kernel, dim3(1), dim3(1024), 0, stream, block_sum, (int32_t)w.n_blocks, block_base,
                       p.out_count);
    const int64_t word_blocks = (w.n_words + kCompactThreads - 1) / kCompactThreads;
    const int64_t entry_blocks = (n_entries + kCompactThreads - 1) / kCompactThreads;
    if (word_blocks + entry_blocks > 0)
        hipLaunchKernelGGL(compact_emit_kernel, dim3((unsigned)(word_blocks + entry_blocks)), dim3(kCompactThreads), 0,
                           stream, p, bitmap, w.n_words, word_base, block_base, word_blocks, uslots);
    if (w.max_rows > 0) {
        const int64_t pieces = w.max_rows * (p.row_bytes / 16);
        const unsigned copy_blocks = (unsigned)std::min<int64_t>(16384, (pieces + kCompactThreads - 1) / kCompactThreads);
        hipLaunchKernelGGL(compact_copy_kernel, dim3(copy_blocks), dim3(kCompactThreads), 0, stream, p, uslots,
                           p.out_count, w.max_rows);
    }
    return hipGetLastError();
}

}  // namespace kv4
