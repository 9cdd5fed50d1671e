// Dedup compaction of top-k lists (README "60+ inference optimizations &
// kernels", section "4-bit KV cache": dedup compaction).
//
// One workgroup per list, its width chosen by list length and count: 1024
// lanes when there are too few lists to fill the compute units, else 256 or
// (for lists of 1025..2048) 512, whose two workgroups per compute unit hide
// each other's memory waits best.  The list is staged through LDS with
// coalesced loads; each lane then owns ITEMS consecutive entries.  Every value
// >= 0 is inserted into an LDS open-addressing table (compare-and-swap on the
// key, linear probing) whose slot also keeps the smallest list position seen
// (atomic min), so "first occurrence" does not depend on the order in which
// lanes win the race.  A lane keeps an entry iff its position is that
// minimum.  The kept entries are placed by an exclusive prefix sum of per-lane
// counts (wave scan with cross-lane reads, wave totals through LDS), staged in
// LDS in list order and written out coalesced together with the -1 fill.
#include "kv4_dedup_impl.h"
#include "kv4_launch.h"

namespace kv4 {

template <int THREADS, int ITEMS>
__global__ __launch_bounds__(THREADS) void dedup_kernel(const int32_t *__restrict__ idx, int32_t k,
                                                        int64_t idx_row_stride, int32_t *__restrict__ out_idx,
                                                        int32_t *__restrict__ out_count, int log2_table) {
    extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
    dedup_list<THREADS, ITEMS>(idx, k, idx_row_stride, out_idx, out_count, log2_table, blockIdx.x, lds);
}

template <int THREADS, int ITEMS>
static hipError_t launch_dedup_items(const int32_t *idx, int64_t n_lists, int32_t k, int64_t stride,
                                     int32_t *out_idx, int32_t *out_count, hipStream_t stream) {
    const int log2_table = dedup_log2_table(k, THREADS);
    const size_t lds = dedup_lds_words(THREADS, ITEMS, log2_table) * 4;
    if (lds > 65536) {
        static bool raised = false;   // benign race: every caller sets the same value
        if (!raised) {
            const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&dedup_kernel<THREADS, ITEMS>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
            raised = true;
        }
    }
    hipLaunchKernelGGL((dedup_kernel<THREADS, ITEMS>), dim3((unsigned)n_lists), dim3(THREADS), lds, stream, idx, k,
                       stride, out_idx, out_count, log2_table);
    return hipGetLastError();
}

hipError_t launch_dedup_compact(const int32_t *idx, int64_t n_lists, int32_t k, int64_t idx_row_stride,
                                int32_t *out_idx, int32_t *out_count, hipStream_t stream) {
    if (n_lists == 0) return hipSuccess;
    if (k <= 256) return launch_dedup_items<256, 1>(idx, n_lists, k, idx_row_stride, out_idx, out_count, stream);
    if (k <= 512) return launch_dedup_items<256, 2>(idx, n_lists, k, idx_row_stride, out_idx, out_count, stream);
    if (n_lists < 256) {   // fewer lists than compute units: four times the lanes per list
        if (k <= 1024) return launch_dedup_items<1024, 1>(idx, n_lists, k, idx_row_stride, out_idx, out_count, stream);
        if (k <= 2048) return launch_dedup_items<1024, 2>(idx, n_lists, k, idx_row_stride, out_idx, out_count, stream);
        return launch_dedup_items<1024, 4>(idx, n_lists, k, idx_row_stride, out_idx, out_count, stream);
    }
    if (k <= 1024) return launch_dedup_items<256, 4>(idx, n_lists, k, idx_row_stride, out_idx, out_count, stream);
    if (k <= 2048) return launch_dedup_items<512, 4>(idx, n_lists, k, idx_row_stride, out_idx, out_count, stream);
    return launch_dedup_items<256, 16>(idx, n_lists, k, idx_row_stride, out_idx, out_count, stream);
}

}  // namespace kv4
