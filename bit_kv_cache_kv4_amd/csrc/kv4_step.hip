// The decode step's row write and list compaction in one launch (README "60+
// inference optimizations & kernels", section "4-bit KV cache": the quantized
// write and the dedup compaction).  The two are independent: as one kernel
// they cost one launch boundary fewer and their memory waits overlap.  A
// workgroup of 1024 lanes either compacts one list (as kv4_dedup.hip's wide
// workgroups do) or writes 16 rows, one per wavefront (as kv4_quant.hip).
#include "kv4_dedup_impl.h"
#include "kv4_quant_impl.h"
#include "kv4_launch.h"

namespace kv4 {

constexpr int kStepThreads = 1024;
constexpr int kStepRowsPerBlock = kStepThreads / 64;

template <int ITEMS, bool DIRECT>
__global__ __launch_bounds__(kStepThreads) void write_dedup_kernel(WriteDedupParams p, int log2_table) {
    extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
    if ((int64_t)blockIdx.x < p.n_lists) {     // uniform per workgroup
        dedup_list<kStepThreads, ITEMS, DIRECT>(p.idx, p.k, p.idx_row_stride, p.out_idx, p.out_count, log2_table, blockIdx.x,
                                        lds);
        return;
    }
    const int64_t b = (int64_t)blockIdx.x - p.n_lists;
    quant_write_row(p.kv, p.kv_row_stride, p.slots, p.n_tokens, p.pool, p.n_slots, p.err_word,
                    b * kStepRowsPerBlock + (threadIdx.x >> 6), threadIdx.x & 63);
}

template <int ITEMS, bool DIRECT>
static hipError_t launch_fused(const WriteDedupParams &p, hipStream_t stream) {
    const int log2_table = dedup_log2_table(p.k, kStepThreads);
    const size_t lds = dedup_lds_words(kStepThreads, ITEMS, log2_table) * 4;
    if (lds > 65536) {
        static bool raised = false;   // benign race: every caller sets the same value
        if (!raised) {
            const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&write_dedup_kernel<ITEMS, DIRECT>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
            raised = true;
        }
    }
    const int64_t blocks = p.n_lists + (p.n_tokens + kStepRowsPerBlock - 1) / kStepRowsPerBlock;
    hipLaunchKernelGGL((write_dedup_kernel<ITEMS, DIRECT>), dim3((unsigned)blocks), dim3(kStepThreads), lds, stream, p,
                       log2_table);
    return hipGetLastError();
}

hipError_t launch_write_dedup(const WriteDedupParams &p, hipStream_t stream) {
    if (p.n_lists == 0 || p.n_lists >= 256) {   // nothing to share a launch with, or enough lists to fill the chip
        hipError_t e = hipSuccess;
        if (p.n_tokens > 0)
            e = launch_quant_write(p.kv, p.kv_row_stride, p.slots, p.n_tokens, p.pool, p.n_slots, p.err_word, stream);
        if (e == hipSuccess)
            e = launch_dedup_compact(p.idx, p.n_lists, p.k, p.idx_row_stride, p.out_idx, p.out_count, stream);
        return e;
    }
    // each thread's entries loaded as one vector when every row is aligned to
    // it and k is a whole number of them (no staging through LDS)
    auto direct = [&](int items) {
        const int vec = items < 4 ? items * 4 : 16;
        return p.k % items == 0 && reinterpret_cast<uintptr_t>(p.idx) % vec == 0 && (p.idx_row_stride * 4) % vec == 0;
    };
    if (p.k <= 1024) return direct(1) ? launch_fused<1, true>(p, stream) : launch_fused<1, false>(p, stream);
    if (p.k <= 2048) return direct(2) ? launch_fused<2, true>(p, stream) : launch_fused<2, false>(p, stream);
    return direct(4) ? launch_fused<4, true>(p, stream) : launch_fused<4, false>(p, stream);
}

}  // namespace kv4
