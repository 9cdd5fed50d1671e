// Internal host-side launchers of the attention kernels (kv4_attn.hip):
// the per-split and prefill attention, the dequantizing gather and the
// (o, lse) merge.  Each returns the HIP status of its launch; arguments were
// validated by the C-ABI layer (kv4_api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kv4 {

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
    _Float16 *out_h;           // non-null: o goes here instead, as fp16, at the same element offsets
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

struct MergeParams {
    const float *part_o;       // (s, t, d) at (s * n_states + t) * dim + d
    const _Float16 *part_o_h;  // non-null: the parts' o as fp16 (same offsets), part_o unused
    const float *part_lse;     // (s, t) at s * n_states + t
    int32_t n_parts;
    int64_t n_states;
    int32_t dim;
    int32_t states_per_row;    // output state t goes to row t / spr, column t % spr
    float *out;                // (t, d) at (t / spr) * out_row_stride + (t % spr) * out_col_stride + d
    int64_t out_row_stride, out_col_stride;
    float *lse;                // (t) at t, nullable
    // Placement hint, 0 for none: the states come in groups of this many
    // consecutive ones, group g's parts written by workgroups on XCD g % 8
    // (the split kernel's rows when their count is a multiple of 8).  The
    // merge then takes each group on that XCD, where the parts may still
    // sit in L2.  Only the order of the work depends on it.
    int64_t xcd_group;
};

hipError_t launch_merge_states(const MergeParams &p, hipStream_t stream);

}  // namespace kv4
