// C ABI of libkv4.so (declared in include/kv4.h): argument checks, launch
// shapes, and the thread-local error text.  Nothing here allocates or
// synchronizes; every launch goes to the caller's stream.
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <cmath>

#include "kv4.h"
#include "kv4_launch.h"

namespace {

thread_local char g_err[512] = "";

kv4_status fail(kv4_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

kv4_status ok() {
    g_err[0] = '\0';
    return KV4_OK;
}

}  // namespace

namespace kv4 {
kv4_status api_fail(kv4_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}
}  // namespace kv4

namespace {

kv4_status hip_status(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(KV4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int device_cu_count() {
    // Compute units of the current device; 256 (MI355X) if it cannot be read.
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
    return n;
}

constexpr int kTile = 32;

// Argument checks shared by the entry points that take kv4_attn_args; with
// need_q false (the gather and the compaction) q, its strides and n_heads are
// not used and not checked.
kv4_status check_attn(const kv4_attn_args *a, bool need_out, bool need_q = true) {
    if (!a) return fail(KV4_ERR_NULL, "args is NULL");
    if (a->struct_size != sizeof(kv4_attn_args))
        return fail(KV4_ERR_SHAPE, "args->struct_size = %u, this library expects %zu", a->struct_size,
                    sizeof(kv4_attn_args));
    if (a->q_dtype != KV4_BF16 && a->q_dtype != KV4_F32) return fail(KV4_ERR_SHAPE, "q_dtype must be KV4_BF16 or KV4_F32");
    if (a->row_format != KV4_ROW_ROPE && a->row_format != KV4_ROW_ROPE_FREE)
        return fail(KV4_ERR_SHAPE, "row_format must be KV4_ROW_ROPE or KV4_ROW_ROPE_FREE");
    if (a->n_rows < 0) return fail(KV4_ERR_SHAPE, "n_rows = %d < 0", a->n_rows);
    if (need_q && (a->n_heads < 16 || a->n_heads > 128 || a->n_heads % 16))
        return fail(KV4_ERR_UNSUPPORTED, "n_heads = %d; supported: a multiple of 16 in [16, 128]", a->n_heads);
    if (a->k < 0) return fail(KV4_ERR_SHAPE, "k = %d < 0", a->k);
    if (a->k > KV4_MAX_K) return fail(KV4_ERR_UNSUPPORTED, "k = %d > %d", a->k, KV4_MAX_K);
    if (a->n_slots < 0) return fail(KV4_ERR_SHAPE, "n_slots < 0");
    if (a->n_slots > 0x7FFFFFFF)   // slots are 32-bit inside the kernels
        return fail(KV4_ERR_UNSUPPORTED, "n_slots = %lld; at most 2^31 - 1", (long long)a->n_slots);
    if (need_q && !std::isfinite(a->sm_scale))
        return fail(KV4_ERR_SHAPE, "sm_scale must be finite (got %g)", (double)a->sm_scale);
    if (a->n_rows == 0) return ok();
    if (need_q && !a->q) return fail(KV4_ERR_NULL, "q is NULL");
    if (a->k > 0 && !a->topk) return fail(KV4_ERR_NULL, "topk is NULL");
    if (a->k > 0 && !a->pool && a->n_slots > 0) return fail(KV4_ERR_NULL, "pool is NULL");
    if (need_out && !a->out) return fail(KV4_ERR_NULL, "out is NULL");
    if (need_q) {
        const int64_t vec = a->q_dtype == KV4_BF16 ? 8 : 4;
        if (!aligned(a->q, 16)) return fail(KV4_ERR_ALIGN, "q must be 16-byte aligned");
        const int64_t dim = a->row_format == KV4_ROW_ROPE_FREE ? KV4_LATENT : KV4_DIM;
        if (a->q_head_stride < dim || a->q_head_stride % vec)
            return fail(KV4_ERR_ALIGN, "q_head_stride = %lld; need >= %lld and a multiple of %lld",
                        (long long)a->q_head_stride, (long long)dim, (long long)vec);
        if (a->q_row_stride < 0 || a->q_row_stride % vec ||
            (a->n_rows > 1 && a->q_row_stride < a->q_head_stride * a->n_heads))
            return fail(KV4_ERR_ALIGN, "q_row_stride = %lld; need >= n_heads * q_head_stride and a multiple of %lld",
                        (long long)a->q_row_stride, (long long)vec);
    }
    if (a->pool && !aligned(a->pool, 16)) return fail(KV4_ERR_ALIGN, "pool must be 16-byte aligned");
    if (a->topk_row_stride < a->k) return fail(KV4_ERR_SHAPE, "topk_row_stride < k");
    if (a->page_table) {
        if (a->page_size <= 0 || (a->page_size & (a->page_size - 1)) || a->page_size > (1 << 20))
            return fail(KV4_ERR_SHAPE, "page_size = %d; need a power of two <= 2^20", a->page_size);
        if (a->pt_n_pages < 0 || a->pt_row_stride < 0) return fail(KV4_ERR_SHAPE, "pt_n_pages/pt_row_stride < 0");
        if (a->pt_n_rows < 1) return fail(KV4_ERR_SHAPE, "pt_n_rows = %d; a page table needs at least one row", a->pt_n_rows);
        if (!a->row_req && a->pt_n_rows < a->n_rows)
            return fail(KV4_ERR_SHAPE, "pt_n_rows = %d < n_rows = %d and no row_req", a->pt_n_rows, a->n_rows);
    }
    if (need_out) {
        if (!aligned(a->out, 16)) return fail(KV4_ERR_ALIGN, "out must be 16-byte aligned");
        if (a->out_row_stride % 4 || (a->n_rows > 1 && a->out_row_stride < (int64_t)a->n_heads * KV4_LATENT))
            return fail(KV4_ERR_ALIGN, "out_row_stride = %lld; need >= n_heads * 512 and a multiple of 4",
                        (long long)a->out_row_stride);
    }
    return ok();
}

int32_t page_shift(const kv4_attn_args *a) {
    int s = 0;
    if (a->page_table)
        while ((1 << s) < a->page_size) ++s;
    return s;
}

kv4::AttnParams base_params(const kv4_attn_args *a) {
    kv4::AttnParams p{};
    p.q = a->q;
    p.q_row_stride = a->q_row_stride;
    p.q_head_stride = a->q_head_stride;
    p.n_rows = a->n_rows;
    p.n_heads = a->n_heads;
    p.pool = a->pool;
    p.n_slots = a->pool ? a->n_slots : 0;
    p.page_table = a->page_table;
    p.pt_row_stride = a->pt_row_stride;
    p.pt_n_rows = a->pt_n_rows;
    p.pt_n_pages = a->pt_n_pages;
    p.page_shift = page_shift(a);
    p.row_req = a->row_req;
    p.topk = a->topk;
    p.topk_row_stride = a->topk_row_stride;
    p.k = a->k;
    p.score_mul = a->sm_scale * 1.44269504088896340736f;
    p.err_word = a->err_word;
    p.rope_dims = a->row_format == KV4_ROW_ROPE_FREE ? 0 : KV4_ROPE;
    return p;
}

int32_t n_tiles(const kv4_attn_args *a) { return (a->k + kTile - 1) / kTile; }

int32_t auto_splits(const kv4_attn_args *a) {
    // Enough workgroups for one per compute unit, but at least four tiles of
    // 32 entries per split: a split's fixed cost (list, page table, queries,
    // first gathers, the state written and merged) is worth a few tiles.
    // Measured on 8 rows x 64 heads x 2048 entries: 5 splits 46.4 us, 8 37.0,
    // 16 33.5, 32 40.0; on 64 rows the compute units bound it at 4.  When the
    // merge has fewer states than compute units its cost hardly grows with the
    // split count, and two tiles per split suffice (1 row x 16 heads x 256
    // entries: 2 splits 23.2 us, 4 21.4, 8 22.2).
    const int32_t tiles = n_tiles(a);
    if (tiles <= 1 || a->n_rows == 0) return 1;
    const int64_t base = (int64_t)a->n_rows * ((a->n_heads + 63) / 64);
    const int64_t cus = device_cu_count();
    int64_t s = (cus + base - 1) / base;
    const int32_t min_tiles = (int64_t)a->n_rows * a->n_heads < cus ? 2 : 4;
    s = std::min<int64_t>(s, std::max<int32_t>(1, tiles / min_tiles));
    s = std::min<int64_t>(s, KV4_MAX_SPLITS);
    return (int32_t)std::max<int64_t>(s, 1);
}

kv4_status check_splits(const kv4_attn_args *a, int32_t num_splits, int32_t *out) {
    if (num_splits < 0 || num_splits > KV4_MAX_SPLITS)
        return fail(KV4_ERR_SHAPE, "num_splits = %d; need 0 (auto) or 1..%d", num_splits, KV4_MAX_SPLITS);
    *out = num_splits == 0 ? auto_splits(a) : num_splits;
    return ok();
}

// kv4_sparse_mla_decode_partial and its fp16 form: exactly one of o32, o16 is set
kv4_status decode_partial(const kv4_attn_args *a, int32_t num_splits, float *o32, _Float16 *o16, float *part_lse,
                          void *stream) {
    kv4_status st = check_attn(a, false);
    if (st != KV4_OK) return st;
    if (num_splits < 1 || num_splits > KV4_MAX_SPLITS)
        return fail(KV4_ERR_SHAPE, "num_splits = %d; need 1..%d", num_splits, KV4_MAX_SPLITS);
    if (a->n_rows == 0) return ok();
    if ((!o32 && !o16) || !part_lse) return fail(KV4_ERR_NULL, "part_o or part_lse is NULL");
    if (o32 ? !aligned(o32, 16) : !aligned(o16, 8))
        return fail(KV4_ERR_ALIGN, "part_o must be %d-byte aligned", o32 ? 16 : 8);
    kv4::AttnParams p = base_params(a);
    p.tiles_per_split = (n_tiles(a) + num_splits - 1) / num_splits;
    p.out = o32;
    p.out_h = o16;
    p.out_row_stride = (int64_t)a->n_heads * KV4_LATENT;
    p.out_split_stride = (int64_t)a->n_rows * a->n_heads * KV4_LATENT;
    p.lse = part_lse;
    p.lse_row_stride = a->n_heads;
    p.lse_split_stride = (int64_t)a->n_rows * a->n_heads;
    return hip_status(kv4::launch_sparse_mla(p, a->q_dtype == KV4_F32, num_splits, (hipStream_t)stream),
                      "sparse_mla launch");
}

// kv4_merge_states and its fp16 form: exactly one of o32, o16 is set
kv4_status merge_states(const float *o32, const _Float16 *o16, const float *part_lse, int32_t n_parts,
                        int64_t n_states, int32_t dim, float *out, int64_t out_state_stride, float *lse, void *stream) {
    if (n_parts < 1 || n_parts > 64) return fail(KV4_ERR_SHAPE, "n_parts = %d; need 1..64", n_parts);
    if (n_states < 0 || n_states > 0x7FFFFFFF) return fail(KV4_ERR_SHAPE, "n_states out of range");
    if (dim < 4 || dim > 4096 || dim % 4) return fail(KV4_ERR_SHAPE, "dim = %d; need a multiple of 4 in [4, 4096]", dim);
    if (n_states == 0) return ok();
    if ((!o32 && !o16) || !part_lse || !out) return fail(KV4_ERR_NULL, "part_o, part_lse or out is NULL");
    if ((o32 ? !aligned(o32, 16) : !aligned(o16, 8)) || !aligned(out, 16))
        return fail(KV4_ERR_ALIGN, "part_o must be %d-byte and out 16-byte aligned", o32 ? 16 : 8);
    if (out_state_stride < dim || out_state_stride % 4)
        return fail(KV4_ERR_ALIGN, "out_state_stride = %lld; need >= dim and a multiple of 4", (long long)out_state_stride);
    kv4::MergeParams m{};
    m.part_o = o32;
    m.part_o_h = o16;
    m.part_lse = part_lse;
    m.n_parts = n_parts;
    m.n_states = n_states;
    m.dim = dim;
    m.states_per_row = 1;
    m.out = out;
    m.out_row_stride = out_state_stride;
    m.out_col_stride = 0;
    m.lse = lse;
    return hip_status(kv4::launch_merge_states(m, (hipStream_t)stream), "merge_states launch");
}

}  // namespace

extern "C" {

const char *kv4_version(void) { return "kv4 1.0.0 gfx950"; }

const char *kv4_last_error(void) { return g_err; }

size_t kv4_attn_args_size(void) { return sizeof(kv4_attn_args); }

namespace {

// Argument checks of kv4_quant_write; *work is false when there is nothing to write.
kv4_status check_quant_write(const float *kv, int64_t kv_row_stride, const int32_t *slots, int64_t n_tokens,
                             const uint8_t *pool, int64_t n_slots, bool *work, int64_t dim = KV4_DIM) {
    *work = false;
    if (n_tokens < 0) return fail(KV4_ERR_SHAPE, "n_tokens = %lld < 0", (long long)n_tokens);
    if (n_slots < 0) return fail(KV4_ERR_SHAPE, "n_slots = %lld < 0", (long long)n_slots);
    if (n_tokens > (int64_t)4 * 0x7FFFFFFF) return fail(KV4_ERR_UNSUPPORTED, "n_tokens too large");
    if (n_tokens == 0) return ok();
    if (!kv || !slots) return fail(KV4_ERR_NULL, "kv or slots is NULL");
    if (!pool && n_slots > 0) return fail(KV4_ERR_NULL, "pool is NULL");
    if (kv_row_stride < dim || kv_row_stride % 4)
        return fail(KV4_ERR_ALIGN, "kv_row_stride = %lld; need >= %lld and a multiple of 4", (long long)kv_row_stride,
                    (long long)dim);
    if (!aligned(kv, 16)) return fail(KV4_ERR_ALIGN, "kv must be 16-byte aligned");
    if (pool && !aligned(pool, 16)) return fail(KV4_ERR_ALIGN, "pool must be 16-byte aligned");
    if (!aligned(slots, 4)) return fail(KV4_ERR_ALIGN, "slots must be 4-byte aligned");
    *work = true;
    return ok();
}

// Argument checks of kv4_dedup_compact; *work is false when there is no list.
kv4_status check_dedup(const int32_t *idx, int64_t n_lists, int32_t k, int64_t idx_row_stride, const int32_t *out_idx,
                       const int32_t *out_count, bool *work) {
    *work = false;
    if (n_lists < 0 || k < 0) return fail(KV4_ERR_SHAPE, "n_lists or k < 0");
    if (k > KV4_MAX_DEDUP_K) return fail(KV4_ERR_UNSUPPORTED, "k = %d > %d", k, KV4_MAX_DEDUP_K);
    if (n_lists > 0x7FFFFFFF) return fail(KV4_ERR_UNSUPPORTED, "n_lists too large");
    if (n_lists == 0) return ok();
    if (!out_count || (k > 0 && (!idx || !out_idx))) return fail(KV4_ERR_NULL, "idx, out_idx or out_count is NULL");
    if (idx_row_stride < k) return fail(KV4_ERR_SHAPE, "idx_row_stride < k");
    if (k > 0) {
        const char *a0 = reinterpret_cast<const char *>(idx), *a1 = a0 + 4 * ((n_lists - 1) * idx_row_stride + k);
        const char *b0 = reinterpret_cast<const char *>(out_idx), *b1 = b0 + 4 * (n_lists * (int64_t)k);
        if (a0 < b1 && b0 < a1) return fail(KV4_ERR_SHAPE, "out_idx overlaps idx");
    }
    *work = true;
    return ok();
}

}  // namespace

kv4_status kv4_quant_write(const float *kv, int64_t kv_row_stride, const int32_t *slots, int64_t n_tokens,
                           uint8_t *pool, int64_t n_slots, uint32_t *err_word, void *stream) {
    bool work = false;
    const kv4_status st = check_quant_write(kv, kv_row_stride, slots, n_tokens, pool, n_slots, &work);
    if (st != KV4_OK || !work) return st;
    return hip_status(kv4::launch_quant_write(kv, kv_row_stride, slots, n_tokens, pool, pool ? n_slots : 0, err_word,
                                              (hipStream_t)stream),
                      "quant_write launch");
}

kv4_status kv4_quant_write_rope_free(const float *kv, int64_t kv_row_stride, const int32_t *slots, int64_t n_tokens,
                                     uint8_t *pool, int64_t n_slots, uint32_t *err_word, void *stream) {
    bool work = false;
    const kv4_status st = check_quant_write(kv, kv_row_stride, slots, n_tokens, pool, n_slots, &work, KV4_LATENT);
    if (st != KV4_OK || !work) return st;
    return hip_status(kv4::launch_quant_write_rope_free(kv, kv_row_stride, slots, n_tokens, pool, pool ? n_slots : 0,
                                                        err_word, (hipStream_t)stream),
                      "quant_write_rope_free launch");
}

kv4_status kv4_quant_write_mse(const float *kv, int64_t kv_row_stride, const int32_t *slots, int64_t n_tokens,
                               uint8_t *pool, int64_t n_slots, kv4_row_format row_format, uint32_t *err_word,
                               void *stream) {
    if (row_format != KV4_ROW_ROPE && row_format != KV4_ROW_ROPE_FREE)
        return fail(KV4_ERR_SHAPE, "row_format = %d; need KV4_ROW_ROPE or KV4_ROW_ROPE_FREE", (int)row_format);
    const bool rope = row_format == KV4_ROW_ROPE;
    bool work = false;
    const kv4_status st =
        check_quant_write(kv, kv_row_stride, slots, n_tokens, pool, n_slots, &work, rope ? KV4_DIM : KV4_LATENT);
    if (st != KV4_OK || !work) return st;
    return hip_status(kv4::launch_quant_write_mse(kv, kv_row_stride, slots, n_tokens, pool, pool ? n_slots : 0, rope,
                                                  err_word, (hipStream_t)stream),
                      "quant_write_mse launch");
}

kv4_status kv4_dedup_compact(const int32_t *idx, int64_t n_lists, int32_t k, int64_t idx_row_stride, int32_t *out_idx,
                             int32_t *out_count, void *stream) {
    bool work = false;
    const kv4_status st = check_dedup(idx, n_lists, k, idx_row_stride, out_idx, out_count, &work);
    if (st != KV4_OK || !work) return st;
    return hip_status(kv4::launch_dedup_compact(idx, n_lists, k, idx_row_stride, out_idx, out_count, (hipStream_t)stream),
                      "dedup_compact launch");
}

kv4_status kv4_write_and_dedup(const float *kv, int64_t kv_row_stride, const int32_t *slots, int64_t n_tokens,
                               uint8_t *pool, int64_t n_slots, uint32_t *err_word, const int32_t *idx,
                               int64_t n_lists, int32_t k, int64_t idx_row_stride, int32_t *out_idx,
                               int32_t *out_count, void *stream) {
    bool write = false, dedup = false;
    kv4_status st = check_quant_write(kv, kv_row_stride, slots, n_tokens, pool, n_slots, &write);
    if (st != KV4_OK) return st;
    st = check_dedup(idx, n_lists, k, idx_row_stride, out_idx, out_count, &dedup);
    if (st != KV4_OK) return st;
    if (!write && !dedup) return ok();
    kv4::WriteDedupParams p{};
    if (write) {
        p.kv = kv;
        p.kv_row_stride = kv_row_stride;
        p.slots = slots;
        p.n_tokens = n_tokens;
        p.pool = pool;
        p.n_slots = pool ? n_slots : 0;
        p.err_word = err_word;
    }
    if (dedup) {
        p.idx = idx;
        p.n_lists = n_lists;
        p.k = k;
        p.idx_row_stride = idx_row_stride;
        p.out_idx = out_idx;
        p.out_count = out_count;
    }
    return hip_status(kv4::launch_write_dedup(p, (hipStream_t)stream), "write_and_dedup launch");
}

int32_t kv4_sparse_mla_decode_splits(const kv4_attn_args *a) {
    const kv4_status st = check_attn(a, false);
    if (st != KV4_OK) return -(int32_t)st;
    return auto_splits(a);
}

size_t kv4_sparse_mla_decode_workspace(const kv4_attn_args *a, int32_t num_splits) {
    if (check_attn(a, false) != KV4_OK) return 0;
    int32_t s = 0;
    if (check_splits(a, num_splits, &s) != KV4_OK || s <= 1) return 0;
    // the splits' o as fp16 (256-byte padded), then their lse as fp32
    const size_t states = (size_t)s * a->n_rows * a->n_heads;
    return ((states * KV4_LATENT * 2 + 255) / 256) * 256 + ((states * 4 + 255) / 256) * 256;
}

kv4_status kv4_sparse_mla_decode_partial(const kv4_attn_args *a, int32_t num_splits, float *part_o, float *part_lse,
                                         void *stream) {
    return decode_partial(a, num_splits, part_o, nullptr, part_lse, stream);
}

kv4_status kv4_sparse_mla_decode_partial_f16(const kv4_attn_args *a, int32_t num_splits, void *part_o,
                                             float *part_lse, void *stream) {
    return decode_partial(a, num_splits, nullptr, static_cast<_Float16 *>(part_o), part_lse, stream);
}

kv4_status kv4_sparse_mla_decode(const kv4_attn_args *a, int32_t num_splits, void *workspace, size_t workspace_bytes,
                                 void *stream) {
    kv4_status st = check_attn(a, true);
    if (st != KV4_OK) return st;
    int32_t s = 0;
    st = check_splits(a, num_splits, &s);
    if (st != KV4_OK) return st;
    if (a->n_rows == 0) return ok();
    kv4::AttnParams p = base_params(a);
    if (s == 1) {
        p.tiles_per_split = std::max(1, n_tiles(a));
        p.out = a->out;
        p.out_row_stride = a->out_row_stride;
        p.out_split_stride = 0;
        p.lse = a->lse;
        p.lse_row_stride = a->n_heads;
        p.lse_split_stride = 0;
        return hip_status(kv4::launch_sparse_mla(p, a->q_dtype == KV4_F32, 1, (hipStream_t)stream), "sparse_mla launch");
    }
    const size_t need = kv4_sparse_mla_decode_workspace(a, s);
    if (!workspace || workspace_bytes < need)
        return fail(KV4_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed for %d splits", workspace ? workspace_bytes : 0,
                    need, s);
    if (!aligned(workspace, 256)) return fail(KV4_ERR_ALIGN, "workspace must be 256-byte aligned");
    // The splits' o travel as fp16: each is a convex combination of latent
    // values, so |o| <= 6 * 448 = 2688 (within fp16's range) and the rounding
    // adds at most 2^-11 of |o| relative to the fp32 state.
    const size_t states = (size_t)s * a->n_rows * a->n_heads;
    _Float16 *part_o = static_cast<_Float16 *>(workspace);
    float *part_lse = reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) +
                                                ((states * KV4_LATENT * 2 + 255) / 256) * 256);
    p.tiles_per_split = (n_tiles(a) + s - 1) / s;
    p.out = nullptr;
    p.out_h = part_o;
    p.out_row_stride = (int64_t)a->n_heads * KV4_LATENT;
    p.out_split_stride = (int64_t)a->n_rows * a->n_heads * KV4_LATENT;
    p.lse = part_lse;
    p.lse_row_stride = a->n_heads;
    p.lse_split_stride = (int64_t)a->n_rows * a->n_heads;
    st = hip_status(kv4::launch_sparse_mla(p, a->q_dtype == KV4_F32, s, (hipStream_t)stream), "sparse_mla launch");
    if (st != KV4_OK) return st;
    kv4::MergeParams m{};
    m.part_o_h = part_o;
    m.part_lse = part_lse;
    m.n_parts = s;
    m.n_states = (int64_t)a->n_rows * a->n_heads;
    m.dim = KV4_LATENT;
    m.states_per_row = a->n_heads;
    m.out = a->out;
    m.out_row_stride = a->out_row_stride;
    m.out_col_stride = KV4_LATENT;
    m.lse = a->lse;
    // the split kernel's workgroup (r, s, z) has linear index r + n_rows (s +
    // S z); dealt round-robin over the 8 XCDs, every split of row r then runs
    // on XCD r % 8 when n_rows is a multiple of 8
    m.xcd_group = a->n_rows % 8 == 0 ? a->n_heads : 0;
    return hip_status(kv4::launch_merge_states(m, (hipStream_t)stream), "merge_states launch");
}

kv4_status kv4_merge_states(const float *part_o, const float *part_lse, int32_t n_parts, int64_t n_states, int32_t dim,
                            float *out, int64_t out_state_stride, float *lse, void *stream) {
    return merge_states(part_o, nullptr, part_lse, n_parts, n_states, dim, out, out_state_stride, lse, stream);
}

kv4_status kv4_merge_states_f16(const void *part_o, const float *part_lse, int32_t n_parts, int64_t n_states,
                                int32_t dim, float *out, int64_t out_state_stride, float *lse, void *stream) {
    return merge_states(nullptr, static_cast<const _Float16 *>(part_o), part_lse, n_parts, n_states, dim, out,
                        out_state_stride, lse, stream);
}

size_t kv4_global_compact_workspace(const kv4_attn_args *a) {
    if (check_attn(a, false, false) != KV4_OK) return 0;
    return kv4::compact_workspace(a->pool ? a->n_slots : 0, a->n_rows, a->k).bytes;
}

kv4_status kv4_global_compact(const kv4_attn_args *a, uint8_t *cpool, int64_t cpool_rows, int32_t *out_idx,
                              int32_t *out_count, void *workspace, size_t workspace_bytes, void *stream) {
    const kv4_status st = check_attn(a, false, false);
    if (st != KV4_OK) return st;
    if (!out_count) return fail(KV4_ERR_NULL, "out_count is NULL");
    const int64_t n_slots = a->pool ? a->n_slots : 0;
    if (n_slots > 0x7FFFFFFF) return fail(KV4_ERR_UNSUPPORTED, "n_slots = %lld; at most 2^31 - 1", (long long)n_slots);
    const int64_t n_entries = (int64_t)a->n_rows * a->k;
    if ((int64_t)a->n_rows * ((a->k + 255) / 256) + (n_slots + 8191) / 8192 > 0x7FFFFFFF)
        return fail(KV4_ERR_UNSUPPORTED, "n_rows * ceil(k / 256) too large for one launch");
    const kv4::CompactWorkspace w = kv4::compact_workspace(n_slots, a->n_rows, a->k);
    if (n_entries > 0 && !out_idx) return fail(KV4_ERR_NULL, "out_idx is NULL");
    if (cpool_rows < w.max_rows)
        return fail(KV4_ERR_SHAPE, "cpool has %lld rows; min(n_slots, n_rows * k) = %lld needed", (long long)cpool_rows,
                    (long long)w.max_rows);
    if (w.max_rows > 0 && !cpool) return fail(KV4_ERR_NULL, "cpool is NULL");
    if (cpool && !aligned(cpool, 16)) return fail(KV4_ERR_ALIGN, "cpool must be 16-byte aligned");
    if (!workspace || workspace_bytes < w.bytes)
        return fail(KV4_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace ? workspace_bytes : 0, w.bytes);
    if (!aligned(workspace, 256)) return fail(KV4_ERR_ALIGN, "workspace must be 256-byte aligned");
    kv4::CompactParams p{};
    p.topk = a->topk;
    p.topk_row_stride = a->topk_row_stride;
    p.n_rows = a->n_rows;
    p.k = a->k;
    p.page_table = a->page_table;
    p.pt_row_stride = a->pt_row_stride;
    p.pt_n_rows = a->pt_n_rows;
    p.pt_n_pages = a->pt_n_pages;
    p.page_shift = page_shift(a);
    p.row_req = a->row_req;
    p.pool = a->pool;
    p.n_slots = n_slots;
    p.row_bytes = a->row_format == KV4_ROW_ROPE_FREE ? KV4_ROW_BYTES_ROPE_FREE : KV4_ROW_BYTES;
    p.cpool = cpool;
    p.out_idx = out_idx;
    p.out_count = out_count;
    p.err_word = a->err_word;
    return hip_status(kv4::launch_global_compact(p, workspace, (hipStream_t)stream), "global_compact launch");
}

kv4_status kv4_gather_dequant(const kv4_attn_args *a, uint16_t *out, int32_t *slots_out, void *stream) {
    const kv4_status st = check_attn(a, false, false);
    if (st != KV4_OK) return st;
    if (a->n_rows == 0 || a->k == 0) return ok();
    if (!out) return fail(KV4_ERR_NULL, "out is NULL");
    if (!aligned(out, 16)) return fail(KV4_ERR_ALIGN, "out must be 16-byte aligned");
    if (slots_out && !aligned(slots_out, 4)) return fail(KV4_ERR_ALIGN, "slots_out must be 4-byte aligned");
    if ((int64_t)a->k > 65535LL * kTile) return fail(KV4_ERR_UNSUPPORTED, "k = %d too long for one gather", a->k);
    return hip_status(kv4::launch_gather_dequant(base_params(a), out, slots_out, (hipStream_t)stream),
                      "gather_dequant launch");
}

kv4_status kv4_sparse_mla_prefill(const kv4_attn_args *a, void *stream) {
    const kv4_status st = check_attn(a, true);
    if (st != KV4_OK) return st;
    if (a->n_rows == 0) return ok();
    kv4::AttnParams p = base_params(a);
    p.tiles_per_split = std::max(1, n_tiles(a));
    p.out = a->out;
    p.out_row_stride = a->out_row_stride;
    p.out_split_stride = 0;
    p.lse = a->lse;
    p.lse_row_stride = a->n_heads;
    p.lse_split_stride = 0;
    return hip_status(kv4::launch_sparse_mla(p, a->q_dtype == KV4_F32, 1, (hipStream_t)stream), "sparse_mla launch");
}

}  // extern "C"
