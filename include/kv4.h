/*
 * kv4.h -- C ABI of libkv4.so: sparse MLA attention over a paged pool of
 * 4-bit NVFP4 KV rows, for AMD Instinct MI355X (gfx950).
 *
 * The row format and the operations follow the README "60+ inference
 * optimizations & kernels", section "4-bit KV cache": a 352-byte NVFP4 row
 * (E2M1 values, one E4M3 scale per 16 values) replaces the 576-byte FP8 row of
 * DSA sparse attention, with a quantized write, a dequantizing gather and dedup
 * compaction; section "AMD MI355X" (hand-written HIP sparse MLA decode,
 * split-K decode) and "Parallelism and disaggregation" ((o, lse) merge).  The
 * pool is addressed through a 64-token page table passed with its stride, and
 * each query row brings its own top-k list (sgl-amd-mono GLM-5.3 monokernel
 * PR, "Modifications"; lists may hold request-local positions or pool slots,
 * its "Review fixes").
 *
 * Row layout (352 bytes, every row 16-byte aligned inside the pool):
 *   [  0, 256)  E2M1 codes of latent dims 0..511; dim 2i in the low nibble of
 *               byte i, dim 2i+1 in the high nibble; nibble = s e e m
 *   [256, 288)  E4M3 (OCP "fn") scale of latent block b = dims 16b..16b+15
 *   [288, 352)  E4M3 rope dims 512..575 (no scale)
 * Value of latent dim i = E2M1(code_i) * E4M3(scale_{i/16}); rope = E4M3.
 *
 * Conventions for every entry point:
 *  - Device pointers are caller-owned device memory; the library never
 *    allocates, frees or synchronizes.  Work is enqueued on `stream` (a
 *    hipStream_t passed as void*; NULL = the null stream) and the call
 *    returns without waiting for it.
 *  - Arguments are checked on the host before anything is enqueued.  On a
 *    non-OK status nothing was enqueued and kv4_last_error() names the
 *    argument and what was expected.  KV4_ERR_HIP reports a failed launch.
 *  - Data errors found on the device (a position past the page table, an
 *    unmapped page, a slot past the pool) never fault: the entry is skipped
 *    and a KV4_ERRBIT_* bit is OR-ed into *err_word when err_word != NULL.
 *  - The library is reentrant; calls on different streams may overlap as
 *    long as their outputs do not alias.
 */
#ifndef KV4_H
#define KV4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KV4_LATENT 512
#define KV4_ROPE 64
#define KV4_DIM 576
#define KV4_BLOCK 16
#define KV4_ROW_BYTES 352
#define KV4_SCALE_OFFSET 256
#define KV4_ROPE_OFFSET 288

#define KV4_MAX_DEDUP_K 4096   /* longest list kv4_dedup_compact accepts */
#define KV4_MAX_SPLITS 64      /* most splits kv4_sparse_mla_decode uses */
#define KV4_MAX_K (1 << 30)    /* longest list the attention and compaction entry points accept */

typedef enum {
    KV4_OK = 0,
    KV4_ERR_NULL = 1,        /* a required pointer is NULL */
    KV4_ERR_SHAPE = 2,       /* a size or stride is out of range */
    KV4_ERR_ALIGN = 3,       /* a pointer or stride breaks the alignment rule */
    KV4_ERR_UNSUPPORTED = 4, /* valid but outside what this build implements */
    KV4_ERR_WORKSPACE = 5,   /* workspace missing or too small */
    KV4_ERR_HIP = 6          /* a HIP call failed */
} kv4_status;

typedef enum { KV4_F32 = 0, KV4_BF16 = 1 } kv4_dtype;

/* Row formats of the pool (README, "4-bit KV cache"): the 352-byte row with
 * 64 E4M3 rope values after the codes and scales, and GLM-5.3-Flash's
 * 288-byte rope-free row (codes and scales only, 512 dims). */
typedef enum { KV4_ROW_ROPE = 0, KV4_ROW_ROPE_FREE = 1 } kv4_row_format;
#define KV4_ROW_BYTES_ROPE_FREE 288

#define KV4_ERRBIT_PAGE 1u /* position past the page table, or page entry < 0 */
#define KV4_ERRBIT_SLOT 2u /* slot >= n_slots */

/* Library version string, e.g. "kv4 1.0.0 gfx950". */
const char *kv4_version(void);

/* Text for the last non-OK status returned on the calling thread ("" if none). */
const char *kv4_last_error(void);

/* sizeof(kv4_attn_args) in this build (for binding layout checks). */
size_t kv4_attn_args_size(void);

/*
 * Quantized row write (README, "4-bit KV cache": the quantized write).
 * For every token n in [0, n_tokens) with slots[n] >= 0, quantize the fp32
 * row kv[n * kv_row_stride + 0..575] and store its 352 bytes at
 * pool + slots[n] * 352.  Per latent block: amax = max |x|, scale =
 * E4M3 nearest to the fp32 quotient amax / 6 (saturating at 448); a scale that
 * rounds to 0 writes scale 0 and all-zero codes; otherwise each code = E2M1
 * nearest to the fp32 quotient x / scale, ties to the even code, saturating at
 * +-6, sign kept on zero.  Rope dims: E4M3 nearest of x, same rules.
 *   kv            device, fp32, 16-byte aligned; kv_row_stride (elements) >= 576
 *                 and a multiple of 4.  Finite values expected.
 *   slots         device, int32 [n_tokens]; slot < 0 = pad row, nothing written
 *                 (sgl-amd-mono PR, "pad rows write no cache"); slot >= n_slots
 *                 writes nothing and sets KV4_ERRBIT_SLOT.
 *   pool          device, [n_slots, 352] bytes, 16-byte aligned.  Two tokens
 *                 naming the same slot leave that row unspecified.
 *   err_word      device, nullable.
 * Errors: KV4_ERR_NULL, KV4_ERR_SHAPE (n_tokens < 0, n_slots < 0, stride),
 * KV4_ERR_ALIGN, KV4_ERR_HIP.
 */
kv4_status kv4_quant_write(const float *kv, int64_t kv_row_stride, const int32_t *slots,
                           int64_t n_tokens, uint8_t *pool, int64_t n_slots, uint32_t *err_word,
                           void *stream);

/*
 * kv4_quant_write for the 288-byte rope-free row (README, "4-bit KV cache":
 * GLM-5.3-Flash's rope-free row): kv rows hold the 512 latent values
 * (kv_row_stride >= 512), pool is [n_slots, 288] (codes [0, 256), block
 * scales [256, 288)).  Everything else as kv4_quant_write.
 */
kv4_status kv4_quant_write_rope_free(const float *kv, int64_t kv_row_stride, const int32_t *slots,
                                     int64_t n_tokens, uint8_t *pool, int64_t n_slots, uint32_t *err_word,
                                     void *stream);

/*
 * kv4_quant_write with MSE-searched block scales (README, "4-bit KV cache":
 * the DeepSeek V4 Pro pools quantize with an MSE-searched scale).  Per
 * latent block, every finite non-negative E4M3 scale d is a candidate; its
 * error is the fp32 sum over the 16 values, in index order and one fused
 * multiply-add each, of (x - c d)^2 with c the E2M1 code of the fp32
 * quotient x / d (all codes zero when d = 0).  The amax/6 scale of
 * kv4_quant_write stays unless a candidate is strictly better; ties among
 * better candidates go to the smallest code.  Codes are then those of the
 * chosen scale, and rope bytes are as in kv4_quant_write.  A block holding a
 * NaN or an infinity keeps the amax/6 scale.
 *   row_format    KV4_ROW_ROPE: kv rows of 576 values, pool [n_slots, 352];
 *                 KV4_ROW_ROPE_FREE: kv rows of 512, pool [n_slots, 288].
 * Everything else (slots, pads, flags, alignment, errors) as kv4_quant_write,
 * plus KV4_ERR_SHAPE for an unknown row_format.
 */
kv4_status kv4_quant_write_mse(const float *kv, int64_t kv_row_stride, const int32_t *slots,
                               int64_t n_tokens, uint8_t *pool, int64_t n_slots, kv4_row_format row_format,
                               uint32_t *err_word, void *stream);

/*
 * Dedup compaction of top-k lists (README, "4-bit KV cache": dedup
 * compaction).  For each list l in [0, n_lists), independently: walk
 * idx[l * idx_row_stride + 0..k-1] in order, keep the first occurrence of
 * every value >= 0, drop negative entries and repeats, write the kept values
 * in their original order to out_idx[l * k + 0..count-1], fill
 * out_idx[l * k + count..k-1] with -1 and write out_count[l] = count.
 *   idx           device int32; idx_row_stride >= k.
 *   out_idx       device int32 [n_lists, k]; must not overlap idx.
 *   out_count     device int32 [n_lists].
 *   k             0 <= k <= KV4_MAX_DEDUP_K.
 * Errors: KV4_ERR_NULL, KV4_ERR_SHAPE, KV4_ERR_UNSUPPORTED (k too large),
 * KV4_ERR_HIP.
 */
kv4_status kv4_dedup_compact(const int32_t *idx, int64_t n_lists, int32_t k, int64_t idx_row_stride,
                             int32_t *out_idx, int32_t *out_count, void *stream);

/*
 * kv4_quant_write and kv4_dedup_compact in one call, the decode step's work
 * before attention (README, "4-bit KV cache": the quantized write and the
 * dedup compaction).  The two are independent; with fewer than 256 lists they
 * run as one kernel, so there is one launch boundary instead of two and their
 * memory waits overlap; with more, as the two kernels.  Arguments, results
 * and errors are exactly those of the two calls (n_tokens == 0 or n_lists == 0
 * leaves that part out); out_idx must not overlap the pool or kv either.
 */
kv4_status kv4_write_and_dedup(const float *kv, int64_t kv_row_stride, const int32_t *slots, int64_t n_tokens,
                               uint8_t *pool, int64_t n_slots, uint32_t *err_word, const int32_t *idx,
                               int64_t n_lists, int32_t k, int64_t idx_row_stride, int32_t *out_idx,
                               int32_t *out_count, void *stream);

/*
 * Arguments of the attention entry points.  For query row r and head h the
 * result is, over the valid entries j of row r's list,
 *   s_j = sm_scale * sum_{i<D} q[r, h, i] * K_j[i]     (D = 576, or 512 rope-free)
 *   o[r, h, :] = sum_j exp(s_j - m) V_j / sum_j exp(s_j - m),   m = max_j s_j
 *   lse[r, h]  = m + ln sum_j exp(s_j - m)
 * where K_j is the dequantized row of entry j (D values) and V_j its first
 * 512 (the latent part: the absorbed-MLA attention core, W_UK applied before
 * and W_UV after it, sgl-amd-mono GLM-5.3 PR, "How a decode step runs").
 * Entry j of row r: pos = topk[r * topk_row_stride + j]; pos < 0 is skipped;
 * with a page table, slot = page_table[req * pt_row_stride + pos / page_size]
 * * page_size + pos % page_size (req = row_req ? row_req[r] : r); without
 * one, slot = pos.  Entries naming the same slot count as often as they
 * appear.  A row with no valid entry gives o = 0 and lse = -inf.
 */
typedef struct kv4_attn_args {
    uint32_t struct_size;      /* must equal sizeof(kv4_attn_args) */
    kv4_dtype q_dtype;         /* KV4_BF16 or KV4_F32 */
    const void *q;             /* device [n_rows, n_heads, D]; 16-byte aligned */
    int64_t q_row_stride;      /* elements; multiple of 8 (bf16) or 4 (f32) */
    int64_t q_head_stride;     /* elements; >= D, multiple of 8 (bf16) or 4 (f32) */
    int32_t n_rows;            /* query rows (decode: one per request) */
    int32_t n_heads;           /* multiple of 16, 16..128 */
    const uint8_t *pool;       /* device [n_slots, 352 or 288 (rope-free)]; 16-byte aligned */
    int64_t n_slots;           /* 0 <= n_slots <= 2^31 - 1 (slots are 32-bit inside the
                                  kernels): larger gives KV4_ERR_UNSUPPORTED */
    const int32_t *page_table; /* device, nullable: NULL => list entries are slots */
    int64_t pt_row_stride;     /* elements between page-table rows (0 = shared row) */
    int32_t pt_n_rows;         /* page-table rows; a query row whose request is outside
                                  [0, pt_n_rows) attends to nothing and sets KV4_ERRBIT_PAGE */
    int32_t pt_n_pages;        /* valid entries per page-table row */
    int32_t page_size;         /* tokens per page, a power of two (64 on the pages) */
    const int32_t *row_req;    /* device [n_rows], nullable: page-table row of each query row */
    const int32_t *topk;       /* device [n_rows, >= k] */
    int64_t topk_row_stride;   /* elements, >= k */
    int32_t k;                 /* list length, 0 <= k <= KV4_MAX_K */
    float sm_scale;            /* softmax scale, e.g. 1/sqrt(576); any finite value (a
                                  negative one reverses the order of the scores), NaN or
                                  infinity gives KV4_ERR_SHAPE */
    float *out;                /* device [n_rows, n_heads, 512] fp32; 16-byte aligned */
    int64_t out_row_stride;    /* elements, >= n_heads * 512, multiple of 4 */
    float *lse;                /* device [n_rows, n_heads] fp32, nullable */
    uint32_t *err_word;        /* device, nullable */
    kv4_row_format row_format; /* KV4_ROW_ROPE (0; D = 576) or KV4_ROW_ROPE_FREE (D = 512) */
} kv4_attn_args;

/* Number of splits kv4_sparse_mla_decode uses for num_splits = 0, or a
 * negative kv4_status if the arguments are invalid. */
int32_t kv4_sparse_mla_decode_splits(const kv4_attn_args *a);

/* Workspace bytes kv4_sparse_mla_decode needs for these arguments and
 * num_splits (0 = the automatic choice); 0 if none is needed or the
 * arguments are invalid. */
size_t kv4_sparse_mla_decode_workspace(const kv4_attn_args *a, int32_t num_splits);

/*
 * Sparse MLA decode (README, "AMD MI355X": hand-written HIP sparse MLA decode
 * and split-K DSA decode; "4-bit KV cache": kv4mla dequantizes rows on chip
 * instead of into an FP8 scratch copy).  Splits each row's list into
 * num_splits contiguous parts (0 = automatic, 1..KV4_MAX_SPLITS), computes a
 * normalised (o, lse) per part from 4-bit rows dequantized on chip, and merges
 * the parts into out/lse.  The parts' o are held in the workspace as fp16
 * (round to nearest even; a part's o is a convex combination of latent values,
 * so |o| <= 2688 and the rounding error is at most 2^-11 of |o|), their lse as
 * fp32: the result equals kv4_merge_states over kv4_sparse_mla_decode_partial's
 * parts with each o first rounded to fp16.
 *   workspace     device, >= kv4_sparse_mla_decode_workspace(a, num_splits)
 *                 bytes, 256-byte aligned; may be NULL when that is 0.
 *                 Its contents are scratch; two calls in flight must not share it.
 * Errors: KV4_ERR_NULL, KV4_ERR_SHAPE, KV4_ERR_ALIGN, KV4_ERR_UNSUPPORTED,
 * KV4_ERR_WORKSPACE, KV4_ERR_HIP.
 */
kv4_status kv4_sparse_mla_decode(const kv4_attn_args *a, int32_t num_splits, void *workspace,
                                 size_t workspace_bytes, void *stream);

/*
 * kv4_sparse_mla_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and result, with the split parts held in a
 * scratch array the library keeps on each device it runs on (allocated with
 * the library's code, held until the process ends) instead of a workspace
 * argument.  No allocation happens in the call.
 *   Limit: kv4_sparse_mla_decode_workspace(a, num_splits) must not exceed
 *   kv4_noalloc_scratch_bytes() (32 MiB); larger gives KV4_ERR_WORKSPACE with
 *   nothing enqueued.
 *   Every call on one device shares that device's array: calls that overlap
 *   on one device (different streams, or one still running on the GPU while
 *   another is enqueued on another stream) race.  Calls on one stream are
 *   ordered and safe.
 * Errors: those of kv4_sparse_mla_decode; KV4_ERR_HIP if the array's device
 * address cannot be found.
 */
kv4_status kv4_sparse_mla_decode_noalloc(const kv4_attn_args *a, int32_t num_splits, void *stream);

/* Bytes of the scratch array kv4_sparse_mla_decode_noalloc uses on each device. */
size_t kv4_noalloc_scratch_bytes(void);

/*
 * The first half of kv4_sparse_mla_decode: for each split s in
 * [0, num_splits) (num_splits >= 1), the normalised state of row r, head h
 * over the entries [s * c, min(k, (s + 1) * c)) with c = 32 * ceil(ceil(k / 32)
 * / num_splits):
 *   part_o[((s * n_rows + r) * n_heads + h) * 512 + d]  (fp32, 16-byte aligned)
 *   part_lse[(s * n_rows + r) * n_heads + h]            (fp32; -inf if empty)
 * a->out, a->out_row_stride and a->lse are ignored.  kv4_merge_states turns
 * the parts into the decode result.  Errors as kv4_sparse_mla_decode.
 */
kv4_status kv4_sparse_mla_decode_partial(const kv4_attn_args *a, int32_t num_splits, float *part_o,
                                         float *part_lse, void *stream);

/*
 * kv4_sparse_mla_decode_partial with the parts' o written as fp16 (round to
 * nearest even; |o| <= 2688, so the rounding error is at most 2^-11 of |o|):
 * the form kv4_sparse_mla_decode keeps in its workspace, which halves the
 * bytes the parts cost to write and to merge.
 *   part_o        device fp16 bit patterns at the offsets above, 8-byte aligned.
 * Errors as kv4_sparse_mla_decode.
 */
kv4_status kv4_sparse_mla_decode_partial_f16(const kv4_attn_args *a, int32_t num_splits, void *part_o,
                                             float *part_lse, void *stream);

/*
 * Merge of attention states (README, "Parallelism and disaggregation": each
 * rank returns (o, lse) to a merge).  For each state t in [0, n_states):
 *   M = max_s lse_s, w_s = exp(lse_s - M), W = sum_s w_s
 *   out[t * out_state_stride + d] = sum_s w_s o_s[d] / W,   lse[t] = M + ln W
 * with o_s = part_o[(s * n_states + t) * dim + d], lse_s = part_lse[s * n_states + t].
 * Parts with lse = -inf carry no weight; if every part is -inf the state
 * gets o = 0 and lse = -inf.
 *   dim           multiple of 4, 4..4096; part_o and out 16-byte aligned;
 *                 out_state_stride >= dim, multiple of 4.
 *   lse           nullable.
 * Errors: KV4_ERR_NULL, KV4_ERR_SHAPE, KV4_ERR_ALIGN, KV4_ERR_HIP.
 */
kv4_status kv4_merge_states(const float *part_o, const float *part_lse, int32_t n_parts,
                            int64_t n_states, int32_t dim, float *out, int64_t out_state_stride,
                            float *lse, void *stream);

/*
 * kv4_merge_states over parts whose o are fp16 bit patterns (as
 * kv4_sparse_mla_decode_partial_f16 writes them), 8-byte aligned; each is
 * widened exactly to fp32 and merged as above.  Errors as kv4_merge_states.
 */
kv4_status kv4_merge_states_f16(const void *part_o, const float *part_lse, int32_t n_parts,
                                int64_t n_states, int32_t dim, float *out, int64_t out_state_stride,
                                float *lse, void *stream);

/*
 * Dequantizing gather (README, "4-bit KV cache": the dequantizing gather),
 * through the attention kernels' own front end: each chunk of 2048 list
 * entries of query row r (entries c0 .. c0 + 2047) is translated as above and
 * its valid entries are packed to the chunk's front in list order, exactly as
 * the attention kernels hold them in their K tiles.  Output position
 * r * k + c0 + i receives the chunk's i-th valid entry: its D dequantized
 * values (D = 576, or 512 for rope-free rows) as fp16 bit patterns at
 * out[(r * k + c0 + i) * D + d] and its pool slot at slots_out[r * k + c0 + i];
 * positions past the chunk's valid count get D zeros and slot -1.  Every value
 * is exact in fp16 (an E2M1 x E4M3 product or an E4M3 value).  The attention
 * entry points never build this copy; it serves tests and callers that want
 * the rows themselves.
 *   out           device [n_rows, k, D] uint16 (fp16 bits), 16-byte aligned.
 *   slots_out     device [n_rows, k] int32, nullable.
 * a->q, a->q_dtype, its strides, a->n_heads, a->out and a->lse are ignored (q
 * may be NULL).  Errors: as kv4_sparse_mla_decode.
 */
kv4_status kv4_gather_dequant(const kv4_attn_args *a, uint16_t *out, int32_t *slots_out, void *stream);

/*
 * Global dedup across lists into a compacted pool (README, "4-bit KV cache":
 * dedup compaction, here across all lists at once).  Every entry of every
 * list is translated exactly as the attention entry points translate it (a
 * query row whose request is outside the page table skips its entries and
 * sets KV4_ERRBIT_PAGE).  With U the distinct valid slots in increasing
 * order: cpool row i = pool row U[i] (i < |U|), out_idx[r * k + j] = the
 * index in U of entry (r, j)'s slot or -1, *out_count = |U|.  Attention with
 * pool = cpool, page_table = NULL and topk = out_idx equals attention over
 * the original arguments, entry for entry; the rows it gathers are |U|
 * contiguous ones.
 *   a             the attention arguments; q, q_dtype, its strides, n_heads,
 *                 sm_scale, out and lse are ignored (q may be NULL).
 *   cpool         device [cpool_rows, row bytes of a->row_format], 16-byte
 *                 aligned; cpool_rows >= min(n_slots, n_rows * k).
 *   out_idx       device int32 [n_rows, k]; out_count device int32 [1].
 *   workspace     device, >= kv4_global_compact_workspace(a) bytes, 256-byte
 *                 aligned (a bitmap of n_slots bits, per-word prefixes, U
 *                 and, for pools of at most 2^19 slots, up to 512 partial
 *                 bitmaps); its contents need no initialisation.
 * Errors: those of kv4_sparse_mla_decode, KV4_ERR_WORKSPACE, and
 * KV4_ERR_UNSUPPORTED for n_slots >= 2^31.
 */
size_t kv4_global_compact_workspace(const kv4_attn_args *a);
kv4_status kv4_global_compact(const kv4_attn_args *a, uint8_t *cpool, int64_t cpool_rows, int32_t *out_idx,
                              int32_t *out_count, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Sparse MLA prefill (README, "AMD MI355X": sparse MLA prefill for gfx950).
 * The same result as kv4_sparse_mla_decode for every query row, computed
 * without splitting the list: one workgroup per (query row, 64 heads) walks
 * the whole list and all its heads share each dequantized tile of rows.  Use
 * row_req (or pt_row_stride = 0) to let many query rows share one request's
 * page table.  No workspace.  Errors as kv4_sparse_mla_decode.
 */
kv4_status kv4_sparse_mla_prefill(const kv4_attn_args *a, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KV4_H */
