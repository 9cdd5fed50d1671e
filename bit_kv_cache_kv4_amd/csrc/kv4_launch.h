// Internal host-side launchers of the kv4 kernels; each returns the HIP status
// of its launch.  Arguments were validated by the C-ABI layer (kv4_api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kv4 {

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

struct AttnParams {
    const void *q;
    int64_t q_row_stride, q_head_stride;
    int32_t n_rows, n_heads;
    const uint8_t *pool;
    int64_t n_slots;
    const int32_t *page_table;
    int64_t pt_row_stride;
    int32_t pt_n_rows, pt_n_pages, page_shift;
    const int32_t *row_req;
    const int32_t *topk;
    int64_t topk_row_stride;
    int32_t k;
    int32_t tiles_per_split;   // tiles of 32 entries per split
    float score_mul;           // sm_scale * log2(e)
    float *out;                // element (s, r, h, d) at s*out_split_stride + r*out_row_stride + h*512 + d
    int64_t out_row_stride, out_split_stride;
    float *lse;                // element (s, r, h) at s*lse_split_stride + r*lse_row_stride + h
    int64_t lse_row_stride, lse_split_stride;
    uint32_t *err_word;
    int32_t rope_dims;         // 64: 352-byte rows, q of 576 dims; 0: 288-byte rope-free rows, q of 512
};

// grid = (n_rows, n_splits, ceil(n_heads / 64))
hipError_t launch_sparse_mla(const AttnParams &p, bool q_f32, int32_t n_splits, hipStream_t stream);

// grid = (n_rows, ceil(k / 32)); out[(r * k + j) * 576 + i] fp16 bits, slots_out nullable
hipError_t launch_gather_dequant(const AttnParams &p, uint16_t *out, int32_t *slots_out, hipStream_t stream);

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

// Workspace layout of the compaction: slot bitmap, per-word and per-block
// prefixes, and the list U of slots (each part 256-byte aligned).
struct CompactWorkspace {
    int64_t n_words, n_blocks, max_rows;
    size_t bitmap_off, word_base_off, block_sum_off, block_base_off, uslots_off, bytes;
};
CompactWorkspace compact_workspace(int64_t n_slots, int64_t n_entries);
hipError_t launch_global_compact(const CompactParams &p, void *workspace, hipStream_t stream);

struct MergeParams {
    const float *part_o;       // (s, t, d) at (s * n_states + t) * dim + d
    const float *part_lse;     // (s, t) at s * n_states + t
    int32_t n_parts;
    int64_t n_states;
    int32_t dim;
    int32_t states_per_row;    // output state t goes to row t / spr, column t % spr
    float *out;                // (t, d) at (t / spr) * out_row_stride + (t % spr) * out_col_stride + d
    int64_t out_row_stride, out_col_stride;
    float *lse;                // (t) at t, nullable
};

hipError_t launch_merge_states(const MergeParams &p, hipStream_t stream);

}  // namespace kv4
