// Internal host-side launchers of the kv4 kernels; each returns the HIP status
// of its launch.  Arguments were validated by the C-ABI layer (kv4_api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kv4.h"
#include "kv4_attn.h"

namespace kv4 {

// Sets kv4_last_error()'s text (printf-style) and returns st.
kv4_status api_fail(kv4_status st, const char *fmt, ...);

hipError_t launch_quant_write(const float *kv, int64_t kv_row_stride, const int32_t *slots,
                              int64_t n_tokens, uint8_t *pool, int64_t n_slots, uint32_t *err_word,
                              hipStream_t stream);

// the same for the 288-byte rope-free row (kv rows of 512 values)
hipError_t launch_quant_write_rope_free(const float *kv, int64_t kv_row_stride, const int32_t *slots,
                                        int64_t n_tokens, uint8_t *pool, int64_t n_slots, uint32_t *err_word,
                                        hipStream_t stream);

// the same with MSE-searched block scales (kv4_quant_mse.hip); rope: 352-byte
// rows from 576 values, else 288-byte rows from 512
hipError_t launch_quant_write_mse(const float *kv, int64_t kv_row_stride, const int32_t *slots, int64_t n_tokens,
                                  uint8_t *pool, int64_t n_slots, bool rope, uint32_t *err_word,
                                  hipStream_t stream);

hipError_t launch_dedup_compact(const int32_t *idx, int64_t n_lists, int32_t k, int64_t idx_row_stride,
                                int32_t *out_idx, int32_t *out_count, hipStream_t stream);

// The row write and the list compaction in one launch (both as above).
struct WriteDedupParams {
    const float *kv;
    int64_t kv_row_stride;
    const int32_t *slots;
    int64_t n_tokens;
    uint8_t *pool;
    int64_t n_slots;
    uint32_t *err_word;
    const int32_t *idx;
    int64_t n_lists;
    int32_t k;
    int64_t idx_row_stride;
    int32_t *out_idx;
    int32_t *out_count;
};

// One kernel when there are fewer lists than compute units (its workgroups
// hold either a list or 16 rows), else the two launches above.
hipError_t launch_write_dedup(const WriteDedupParams &p, hipStream_t stream);

// Global dedup across lists into a compacted pool (kv4_compact.hip).
struct CompactParams {
    const int32_t *topk;
    int64_t topk_row_stride;
    int32_t n_rows, k;
    const int32_t *page_table;
    int64_t pt_row_stride;
    int32_t pt_n_rows, pt_n_pages, page_shift;
    const int32_t *row_req;
    const uint8_t *pool;
    int64_t n_slots;
    int32_t row_bytes;         // 352 or 288
    uint8_t *cpool;            // [max_rows, row_bytes]
    int32_t *out_idx;          // [n_rows, k]
    int32_t *out_count;        // [1]: |U|
    uint32_t *err_word;
};

// Workspace layout of the compaction: slot bitmap, per-word bits and prefix
// (uint2), per-block sums and bases, the list U of slots and, for bitmaps
// marked in LDS, one partial bitmap per marking workgroup (each part 256-byte
// aligned).
struct CompactWorkspace {
    int64_t n_words, n_blocks, max_rows;
    int32_t n_parts, rows_per_part;   // LDS marking: workgroups and the query rows each takes (0: global marking)
    size_t bitmap_off, word_info_off, block_sum_off, block_base_off, uslots_off, parts_off, bytes;
};
CompactWorkspace compact_workspace(int64_t n_slots, int32_t n_rows, int32_t k);
hipError_t launch_global_compact(const CompactParams &p, void *workspace, hipStream_t stream);

}  // namespace kv4
