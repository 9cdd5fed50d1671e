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
// counts (within a wavefront from one ballot per item, the wavefronts' totals
// through LDS), staged in LDS in list order and written out coalesced
// together with the -1 fill.
// With more lists than workgroups that fit on the chip at once, each
// workgroup walks lists g, g + G, g + 2G, ... (G = the grid): the next
// list's loads are issued before the current list is compacted, so their
// round trip overlaps that work, and only the table slots a list used are
// cleared before the next one.
#include <hip/hip_runtime.h>

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

template <int THREADS, int ITEMS, bool DIRECT>
__global__ __launch_bounds__(THREADS) void dedup_stream_kernel(const int32_t *__restrict__ idx, int32_t k,
                                                               int64_t idx_row_stride, int32_t *__restrict__ out_idx,
                                                               int32_t *__restrict__ out_count, int log2_table,
                                                               int64_t n_lists) {
    extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
    __builtin_assume(k > 0);                       // the launch takes this kernel only for k >= 1
    const DedupLds<THREADS, ITEMS> m(lds, 1 << log2_table);
    int64_t list = blockIdx.x;                     // < n_lists: the grid holds at most n_lists workgroups
    int32_t v[ITEMS], ld[ITEMS];
    if constexpr (DIRECT) {
        // each thread's entries straight into registers: no staging through LDS
        dedup_load_direct<THREADS, ITEMS>(idx + list * idx_row_stride, k, v);
        dedup_clear<THREADS, ITEMS>(m, 1 << log2_table);
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) asm volatile("" : "+v"(v[i]));   // the first list's wait, before the loop
        __syncthreads();                           // table clear
    } else {
        dedup_load<THREADS, ITEMS>(idx + list * idx_row_stride, k, ld);
        dedup_clear<THREADS, ITEMS>(m, 1 << log2_table);
        dedup_stage<THREADS, ITEMS>(m, ld);
        __syncthreads();                           // list staged, table clear
        dedup_read_staged<THREADS, ITEMS>(m, v);
    }
    // Each list's loads go out before the current list is compacted and are
    // waited for at the end of the iteration, after that list's stores (a
    // fixed number per thread): the wait then leaves the stores in flight,
    // which a wait at the loop's top, shared with the first list's, would not.
    for (;;) {
        const int64_t next = list + gridDim.x;
        if (next < n_lists) {                      // uniform
            if constexpr (DIRECT) dedup_load_direct<THREADS, ITEMS>(idx + next * idx_row_stride, k, ld);
            else dedup_load<THREADS, ITEMS>(idx + next * idx_row_stride, k, ld);
        }
        uint32_t slot[ITEMS];
        dedup_core<THREADS, ITEMS>(m, k, log2_table, out_idx + list * (int64_t)k, out_count + list, v, slot);
        if (next >= n_lists) break;
        dedup_undo<THREADS, ITEMS>(m, v, slot);
        if constexpr (DIRECT) {
#pragma unroll
            for (int i = 0; i < ITEMS; ++i) {
                asm volatile("" : "+v"(ld[i]));    // the wait for the next list's loads lands here
                v[i] = ld[i];
            }
            __syncthreads();                       // stage read out and the table cleared
        } else {
            __syncthreads();                       // stage read out before it takes the next list
            dedup_stage<THREADS, ITEMS>(m, ld);
            __syncthreads();                       // next list staged, table cleared
            dedup_read_staged<THREADS, ITEMS>(m, v);
        }
        list = next;
    }
}

// Workgroups of dedup_stream_kernel<THREADS, ITEMS> with `lds` bytes (a
// function of the table size) that fit on the current device at once, 0 if
// the runtime cannot say; looked up once per instance, device and table size.
template <int THREADS, int ITEMS, bool DIRECT>
static int64_t resident_workgroups(int log2_table, size_t lds) {
    constexpr int kMaxDev = 64, kMaxLog2 = 32;
    static int64_t cached[kMaxDev][kMaxLog2] = {};  // benign race: every caller stores the same value
    const auto kernel = dedup_stream_kernel<THREADS, ITEMS, DIRECT>;
    const int threads = THREADS;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    const bool slot = dev >= 0 && dev < kMaxDev && log2_table >= 0 && log2_table < kMaxLog2;
    if (slot && cached[dev][log2_table] > 0) return cached[dev][log2_table];
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(kernel), threads, lds) !=
            hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    const int64_t n = (int64_t)per_cu * cus;
    if (slot) cached[dev][log2_table] = n;
    return n;
}

// The streaming kernel when more lists than fit on the chip at once (and
// k >= 1), else one workgroup per list.
template <int THREADS, int ITEMS, bool DIRECT>
static hipError_t launch_stream(const int32_t *idx, int64_t n_lists, int32_t k, int64_t stride, int32_t *out_idx,
                                int32_t *out_count, int log2_table, size_t lds, hipStream_t stream) {
    auto stream_kernel = dedup_stream_kernel<THREADS, ITEMS, DIRECT>;
    if (lds > 65536) {
        static bool raised = false;   // benign race: every caller sets the same value
        if (!raised) {
            const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(stream_kernel),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
            raised = true;
        }
    }
    const int64_t resident = resident_workgroups<THREADS, ITEMS, DIRECT>(log2_table, lds);
    if (k > 0 && resident > 0 && n_lists > resident) {
        hipLaunchKernelGGL(stream_kernel, dim3((unsigned)resident), dim3(THREADS), lds, stream, idx, k, stride, out_idx,
                           out_count, log2_table, n_lists);
    } else {
        hipLaunchKernelGGL((dedup_kernel<THREADS, ITEMS>), dim3((unsigned)n_lists), dim3(THREADS), lds, stream, idx,
                           k, stride, out_idx, out_count, log2_table);
    }
    return hipGetLastError();
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
    // each thread's entries loaded as vectors when every list row is aligned
    // to them and k is a whole number of them
    constexpr int kVec = ITEMS < 4 ? ITEMS * 4 : 16;   // bytes per vector load
    const bool direct = k % ITEMS == 0 && reinterpret_cast<uintptr_t>(idx) % kVec == 0 && (stride * 4) % kVec == 0;
    if (direct) return launch_stream<THREADS, ITEMS, true>(idx, n_lists, k, stride, out_idx, out_count, log2_table, lds,
                                                          stream);
    return launch_stream<THREADS, ITEMS, false>(idx, n_lists, k, stride, out_idx, out_count, log2_table, lds, stream);
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
