/*
 * kv4 oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, CPU implementation of what the sparse-MLA-over-NVFP4 hot path
 * computes.  Only the test suite, the smoke check and the benchmark's CPU
 * baseline may load this library.  The product path (the HIP library) never
 * calls it and shares no code, header, table or constant with it.
 *
 * Sources (web pages; sections named, lines not):
 *  [P1-KV4]  "60+ inference optimizations & kernels" (README), section
 *            "4-bit KV cache": a 352-byte NVFP4 row with E2M1 values and one
 *            E4M3 scale per 16 values replaces the 576-byte FP8 row of DSA
 *            sparse attention; kernels perform the quantized write, the
 *            dequantizing gather and dedup compaction.  The rope-free
 *            GLM-5.3-Flash row is 288 bytes.
 *  [P1-PAR]  same page, section "Parallelism and disaggregation": each rank
 *            returns (o, lse) to a merge.
 *  [P4-PT]   sgl-amd-mono PR "GLM-5.3 decode monokernels", section
 *            "Modifications": a 64-token page table, passed with its stride,
 *            maps request positions to pool slots; exact top-2048 per row;
 *            absorbed query (W_UK) before and W_UV after the attention core.
 *  [P4-PAD]  same page: pad rows write no cache.
 *
 * Readings of points the pages leave open (each listed in the design notes):
 *  R1 row byte order: codes [0, L/2) | block scales [L/2, L/2 + L/16) | rope.
 *  R2 nibble order: element 2i in the low nibble of byte i, 2i+1 in the high.
 *  R3 E4M3 is the OCP "fn" variant (bias 7, no infinities, max 448, 0x7F/0xFF
 *     NaN).  E2M1: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa.
 *  R4 block scale = E4M3 nearest to the fp32 quotient amax / 6 (no second
 *     level scale); a scale that rounds to zero zeroes the whole block.
 *  R5 each latent code = E2M1 nearest to the fp32 quotient x / scale;
 *     ties go to the even code; magnitudes above 6 saturate; the sign is kept
 *     for values that round to zero.
 *  R6 rope values are plain E4M3 (scale 1), ties to even, saturate at 448,
 *     sign kept for zero.
 *  R7 scores use all latent+rope dims, values are the latent dims only.
 *  R8 negative list entries are skipped; entries that translate outside the
 *     page table or the pool are skipped and flagged.
 *  R9 duplicates inside an attention list count as given.
 *  R10 an empty list gives o = 0 and lse = -inf; lse is the natural log of
 *     the sum of exp(scaled score).
 *  R11 dedup keeps, per list, the first occurrence of each non-negative value
 *     in list order, then fills with -1, and reports the count.
 *  R20 MSE-searched scale: the candidates are all finite non-negative E4M3
 *     scales; a block's squared error is summed in fp32 in index order with
 *     fused multiply-adds; the amax/6 scale stays unless another is strictly
 *     better, and ties among better ones go to the smallest code.
 *
 * Precision: every decision that turns a float into a code (amax / 6, x / d)
 * is made in fp32, the precision of the kernels; attention arithmetic is fp64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ERR_PAGE 1u
#define ERR_SLOT 2u

int o_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void o_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ---------------------------------------------------------------- codecs */

/* OCP E4M3 ("fn"): s eeee mmm, bias 7.  Subnormals when e == 0.
 * e == 15 and m == 7 is NaN; there are no infinities. */
double o_e4m3_value(uint8_t c)
{
    int s = (c >> 7) & 1, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m / 8.0, 1 - 7);
    else        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/* E2M1: s ee m, bias 1.  Subnormal (0 or 0.5) when e == 0. */
double o_e2m1_value(uint8_t c)
{
    int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
    double v;
    if (e == 0) v = 0.5 * (double)m;
    else        v = ldexp(1.0 + 0.5 * (double)m, e - 1);
    return s ? -v : v;
}

/* Nearest finite non-negative E4M3 code to |x| by exhaustive search; a tie
 * goes to the code whose mantissa LSB is 0 (the even code).  Magnitudes above
 * the largest finite value (448) saturate to it.  The sign bit follows x,
 * also when the magnitude rounds to zero. */
uint8_t o_e4m3_encode(float x)
{
    double a = fabs((double)x);
    uint8_t best = 0;
    double bestd = INFINITY;
    int code;
    if (isnan(x)) return 0x7F;
    if (a > 448.0) a = 448.0;
    for (code = 0; code <= 0x7E; ++code) {
        double d = fabs(a - o_e4m3_value((uint8_t)code));
        if (d < bestd || (d == bestd && (code & 1) == 0 && (best & 1) == 1)) {
            bestd = d;
            best = (uint8_t)code;
        }
    }
    return (uint8_t)(best | (signbit(x) ? 0x80 : 0));
}

/* Nearest E2M1 code to |y| by exhaustive search over the 8 magnitudes; ties
 * go to the even code; magnitudes above 6 saturate; the sign follows y. */
uint8_t o_e2m1_encode(float y)
{
    double a = fabs((double)y);
    uint8_t best = 0;
    double bestd = INFINITY;
    int code;
    if (a > 6.0) a = 6.0;
    for (code = 0; code < 8; ++code) {
        double d = fabs(a - o_e2m1_value((uint8_t)code));
        if (d < bestd || (d == bestd && (code & 1) == 0 && (best & 1) == 1)) {
            bestd = d;
            best = (uint8_t)code;
        }
    }
    return (uint8_t)(best | (signbit(y) ? 0x8 : 0));
}

/* -------------------------------------------------------------- row format */

/* Bytes of one row: n_latent/2 code bytes, n_latent/16 scale bytes and one
 * byte per rope dim ([P1-KV4]: 512 + 64 dims -> 352 B; rope-free 512 -> 288 B). */
int o_row_bytes(int n_latent, int n_rope)
{
    return n_latent / 2 + n_latent / 16 + n_rope;
}

/* ---------------------------------------------------- MSE-searched scale */

/* Squared error of coding the 16 values blk[0..15] with E4M3 scale `code`
 * (R20): each value takes its R5 code (none when the scale is zero), the
 * error x - c*d is formed in fp32 (c*d is exact there) and the squares are
 * summed in index order, one fp32 fused multiply-add per value. */
static float o_block_sq_error(const float *blk, uint8_t code)
{
    double d = o_e4m3_value(code);
    float s = 0.0f;
    int i;
    for (i = 0; i < 16; ++i) {
        float cd = 0.0f, e;
        if (d != 0.0) cd = (float)(o_e2m1_value(o_e2m1_encode(blk[i] / (float)d)) * d);
        e = blk[i] - cd;
        s = fmaf(e, e, s);
    }
    return s;
}

/* MSE-searched block scale ([P1-KV4] DeepSeek V4 Pro pools; R20): every
 * finite non-negative E4M3 code is a candidate.  The amax/6 scale `base`
 * stays unless some candidate has a strictly smaller squared error; then the
 * smallest code among those with the least error wins.  A block whose error
 * is NaN (a NaN value) keeps `base`. */
static uint8_t o_mse_scale(const float *blk, uint8_t base)
{
    uint8_t best = base;
    float best_err = o_block_sq_error(blk, base);
    int code;
    for (code = 0; code <= 0x7E; ++code) {
        float err = o_block_sq_error(blk, (uint8_t)code);
        if (err < best_err) {
            best_err = err;
            best = (uint8_t)code;
        }
    }
    return best;
}

/* Quantize one row with the amax/6 scale (mse = 0) or the MSE-searched one. */
static void o_quantize_row_rule(const float *x, int n_latent, int n_rope, int mse, uint8_t *out)
{
    int nblk = n_latent / 16, b, i;
    uint8_t *codes = out, *scales = out + n_latent / 2, *rope = scales + nblk;
    memset(codes, 0, (size_t)(n_latent / 2));
    for (b = 0; b < nblk; ++b) {
        float amax = 0.0f, scale_f;
        uint8_t s;
        double d;
        for (i = 0; i < 16; ++i) {
            float a = fabsf(x[16 * b + i]);
            if (a > amax) amax = a;
        }
        scale_f = amax / 6.0f;                 /* fp32 division (R4) */
        s = o_e4m3_encode(scale_f);
        if (mse) s = o_mse_scale(x + 16 * b, s);
        d = o_e4m3_value(s);
        scales[b] = s;
        if (d == 0.0) continue;                /* zero block: codes stay 0 */
        for (i = 0; i < 16; ++i) {
            int e = 16 * b + i;
            float q = x[e] / (float)d;         /* fp32 division (R5) */
            uint8_t c = o_e2m1_encode(q);
            if (e & 1) codes[e >> 1] |= (uint8_t)(c << 4);
            else       codes[e >> 1] |= c;
        }
    }
    for (i = 0; i < n_rope; ++i) rope[i] = o_e4m3_encode(x[n_latent + i]);
}

/* Quantize one row x[n_latent + n_rope] into out[o_row_bytes(...)]. */
void o_quantize_row(const float *x, int n_latent, int n_rope, uint8_t *out)
{
    o_quantize_row_rule(x, n_latent, n_rope, 0, out);
}

/* The same with MSE-searched block scales; rope bytes are unchanged. */
void o_quantize_row_mse(const float *x, int n_latent, int n_rope, uint8_t *out)
{
    o_quantize_row_rule(x, n_latent, n_rope, 1, out);
}

/* Dequantize one row: latent value = E2M1 value * its block's E4M3 scale,
 * rope value = E4M3 value.  Every result is exact in double. */
void o_dequantize_row(const uint8_t *row, int n_latent, int n_rope, double *out)
{
    const uint8_t *codes = row, *scales = row + n_latent / 2, *rope = scales + n_latent / 16;
    int e;
    for (e = 0; e < n_latent; ++e) {
        uint8_t c = (e & 1) ? (uint8_t)(codes[e >> 1] >> 4) : (uint8_t)(codes[e >> 1] & 15);
        out[e] = o_e2m1_value(c) * o_e4m3_value(scales[e / 16]);
    }
    for (e = 0; e < n_rope; ++e) out[n_latent + e] = o_e4m3_value(rope[e]);
}

/* ------------------------------------------------------ quantized row write */

/* For each token n with slot[n] >= 0, quantize kv[n] and store the row at
 * pool[slot * row_bytes].  A negative slot is a pad row and writes nothing
 * ([P4-PAD]); a slot >= n_slots writes nothing and sets ERR_SLOT. */
static void o_quant_write_rule(const float *kv, int64_t kv_row_stride, const int32_t *slots, int64_t n_tokens,
                               int n_latent, int n_rope, int mse, uint8_t *pool, int64_t n_slots, uint32_t *err)
{
    int rb = o_row_bytes(n_latent, n_rope);
    uint32_t e = 0;
    int64_t n;
    /* Tokens are independent; two tokens naming the same slot leave that row
     * unspecified, as in the kernel. */
#pragma omp parallel for schedule(static) reduction(| : e)
    for (n = 0; n < n_tokens; ++n) {
        int32_t s = slots[n];
        if (s < 0) continue;
        if ((int64_t)s >= n_slots) { e |= ERR_SLOT; continue; }
        o_quantize_row_rule(kv + n * kv_row_stride, n_latent, n_rope, mse, pool + (int64_t)s * rb);
    }
    if (err) *err |= e;
}

void o_quant_write(const float *kv, int64_t kv_row_stride, const int32_t *slots, int64_t n_tokens,
                   int n_latent, int n_rope, uint8_t *pool, int64_t n_slots, uint32_t *err)
{
    o_quant_write_rule(kv, kv_row_stride, slots, n_tokens, n_latent, n_rope, 0, pool, n_slots, err);
}

/* The quantized write with MSE-searched block scales (R20). */
void o_quant_write_mse(const float *kv, int64_t kv_row_stride, const int32_t *slots, int64_t n_tokens,
                       int n_latent, int n_rope, uint8_t *pool, int64_t n_slots, uint32_t *err)
{
    o_quant_write_rule(kv, kv_row_stride, slots, n_tokens, n_latent, n_rope, 1, pool, n_slots, err);
}

/* ------------------------------------------------------ dedup / compaction */

typedef struct { int32_t v; int32_t pos; } o_pair;

static int o_pair_cmp(const void *a, const void *b)
{
    const o_pair *x = (const o_pair *)a, *y = (const o_pair *)b;
    if (x->v != y->v) return x->v < y->v ? -1 : 1;
    return x->pos < y->pos ? -1 : (x->pos > y->pos);
}

static int o_int_cmp(const void *a, const void *b)
{
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return x < y ? -1 : (x > y);
}

/* Per list (R11): keep the first occurrence of every value >= 0, in list
 * order, pad with -1, report the count.  Done the plain way: sort
 * (value, position) pairs, take the lowest position of each value, sort those
 * positions back into list order. */
void o_dedup_compact(const int32_t *idx, int64_t n_lists, int32_t k, int64_t idx_row_stride,
                     int32_t *out, int32_t *count)
{
    int64_t l;
#pragma omp parallel for schedule(dynamic, 16)
    for (l = 0; l < n_lists; ++l) {
        const int32_t *src = idx + l * idx_row_stride;
        int32_t *dst = out + l * (int64_t)k;
        o_pair *pairs = (o_pair *)malloc(sizeof(o_pair) * (size_t)(k > 0 ? k : 1));
        int32_t *keep = (int32_t *)malloc(sizeof(int32_t) * (size_t)(k > 0 ? k : 1));
        int np = 0, nk = 0, j;
        for (j = 0; j < k; ++j)
            if (src[j] >= 0) { pairs[np].v = src[j]; pairs[np].pos = j; ++np; }
        qsort(pairs, (size_t)np, sizeof(o_pair), o_pair_cmp);
        for (j = 0; j < np; ++j)
            if (j == 0 || pairs[j].v != pairs[j - 1].v) keep[nk++] = pairs[j].pos;
        qsort(keep, (size_t)nk, sizeof(int32_t), o_int_cmp);
        for (j = 0; j < nk; ++j) dst[j] = src[keep[j]];
        for (j = nk; j < k; ++j) dst[j] = -1;
        count[l] = nk;
        free(pairs);
        free(keep);
    }
}

/* ------------------------------------------------------ index -> pool slot */

/* pos -> slot.  With a page table: slot = pt[page] * page_size + pos % page_size
 * where page = pos / page_size ([P4-PT]); without one, slot = pos.  Returns -1
 * for a negative pos (no flag) and for a position whose page is outside the
 * table or unmapped (ERR_PAGE) or whose slot is outside the pool (ERR_SLOT). */
int64_t o_translate(int32_t pos, const int32_t *pt_row, int32_t pt_n_pages, int32_t page_size,
                    int64_t n_slots, uint32_t *err)
{
    int64_t slot;
    if (pos < 0) return -1;
    if (pt_row) {
        int32_t page = pos / page_size, phys;
        if (page >= pt_n_pages) { *err |= ERR_PAGE; return -1; }
        phys = pt_row[page];
        if (phys < 0) { *err |= ERR_PAGE; return -1; }
        slot = (int64_t)phys * page_size + pos % page_size;
    } else {
        slot = pos;
    }
    if (slot >= n_slots) { *err |= ERR_SLOT; return -1; }
    return slot;
}

/* ------------------------------------------------ global dedup across lists */

/* The compacted pool ([P1-KV4] "dedup compaction" read across all lists at
 * once).  Every entry of every list is translated as for attention (entries
 * of a query row whose request is outside [0, pt_n_rows) are skipped and
 * flag ERR_PAGE when >= 0).  U = the distinct valid slots in increasing
 * order; cpool row i = pool row U[i]; out_idx[r * k + j] = the index in U of
 * entry (r, j)'s slot, -1 for a skipped entry.  Returns |U|.  Attention over
 * cpool with out_idx as physical slots equals attention over pool with the
 * original lists, entry for entry. */
int64_t o_global_compact(const int32_t *topk, int32_t n_rows, int32_t k, int64_t topk_row_stride,
                         const int32_t *page_table, int64_t pt_row_stride, int32_t pt_n_rows, int32_t pt_n_pages,
                         int32_t page_size, const int32_t *row_req, const uint8_t *pool, int64_t n_slots,
                         int row_bytes, uint8_t *cpool, int32_t *out_idx, uint32_t *err)
{
    char *seen = (char *)calloc((size_t)(n_slots > 0 ? n_slots : 1), 1);
    int64_t *rank = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n_slots > 0 ? n_slots : 1));
    int64_t count = 0, s;
    int32_t r, j;
    int pass;
    for (pass = 0; pass < 2; ++pass) {        /* 0: mark the slots; 1: rewrite the lists */
        for (r = 0; r < n_rows; ++r) {
            int32_t req = row_req ? row_req[r] : r;
            int bad = page_table && (req < 0 || req >= pt_n_rows);
            const int32_t *pt_row = page_table && !bad ? page_table + (int64_t)req * pt_row_stride : NULL;
            for (j = 0; j < k; ++j) {
                int32_t pos = topk[(int64_t)r * topk_row_stride + j];
                int64_t slot = -1;
                if (bad) {
                    if (pos >= 0) *err |= ERR_PAGE;
                } else {
                    slot = o_translate(pos, pt_row, pt_n_pages, page_size, n_slots, err);
                }
                if (pass == 0) {
                    if (slot >= 0) seen[slot] = 1;
                } else {
                    out_idx[(int64_t)r * k + j] = slot >= 0 ? (int32_t)rank[slot] : -1;
                }
            }
        }
        if (pass == 0) {
            for (s = 0; s < n_slots; ++s) {
                if (!seen[s]) continue;
                rank[s] = count;
                memcpy(cpool + count * row_bytes, pool + s * row_bytes, (size_t)row_bytes);
                ++count;
            }
        }
    }
    free(seen);
    free(rank);
    return count;
}

/* ------------------------------------------------------ sparse MLA attention */

/* One argument block shared by the attention entry points.  q is fp32
 * (a bf16 query is widened exactly by the caller).  Layouts:
 *   q[r * q_row_stride + h * q_head_stride + i], i < n_latent + n_rope
 *   page_table[req * pt_row_stride + page], req = row_req ? row_req[r] : r
 *   topk[r * topk_row_stride + j], j < k
 *   out[(r * n_heads + h) * n_latent + d], lse[r * n_heads + h]            */
typedef struct {
    const float *q; int64_t q_row_stride, q_head_stride;
    int32_t n_rows, n_heads, n_latent, n_rope;
    const uint8_t *pool; int64_t n_slots;
    const int32_t *page_table; int64_t pt_row_stride; int32_t pt_n_pages, page_size;
    const int32_t *row_req;
    const int32_t *topk; int64_t topk_row_stride; int32_t k;
    double sm_scale;
} o_attn_args;

/* For every (row r, head h), over the valid entries of row r's list:
 *   s_j = sm_scale * sum_i q[r,h,i] K_j[i]            (all latent+rope dims)
 *   m = max_j s_j, p_j = exp(s_j - m), l = sum_j p_j
 *   o[r,h,:] = sum_j p_j V_j / l, V_j = K_j[0:n_latent]
 *   lse[r,h] = m + ln l
 * K_j is the dequantized pool row of entry j.  Optionally returns the
 * normalised probabilities p_j / l (probs[(r*n_heads+h)*k + j], 0 for
 * skipped entries). */
void o_sparse_mla(const o_attn_args *a, double *out, double *lse, double *probs, uint32_t *err)
{
    int D = a->n_latent + a->n_rope;
    int32_t r;
    uint32_t err_all = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err_all)
    for (r = 0; r < a->n_rows; ++r) {
        int32_t req = a->row_req ? a->row_req[r] : r;
        const int32_t *pt_row = a->page_table ? a->page_table + (int64_t)req * a->pt_row_stride : NULL;
        const int32_t *list = a->topk + (int64_t)r * a->topk_row_stride;
        double *K = (double *)malloc(sizeof(double) * (size_t)D * (size_t)(a->k > 0 ? a->k : 1));
        double *s = (double *)malloc(sizeof(double) * (size_t)(a->k > 0 ? a->k : 1));
        char *valid = (char *)malloc((size_t)(a->k > 0 ? a->k : 1));
        int rb = o_row_bytes(a->n_latent, a->n_rope);
        uint32_t e = 0;
        int32_t j, h;
        int nvalid = 0;
        for (j = 0; j < a->k; ++j) {
            int64_t slot = o_translate(list[j], pt_row, a->pt_n_pages, a->page_size, a->n_slots, &e);
            valid[j] = slot >= 0;
            if (valid[j]) {
                o_dequantize_row(a->pool + slot * rb, a->n_latent, a->n_rope, K + (int64_t)j * D);
                ++nvalid;
            }
        }
        err_all |= e;
        for (h = 0; h < a->n_heads; ++h) {
            const float *qh = a->q + (int64_t)r * a->q_row_stride + (int64_t)h * a->q_head_stride;
            double *o = out + ((int64_t)r * a->n_heads + h) * a->n_latent;
            double m = -INFINITY, l = 0.0;
            int d, i;
            for (d = 0; d < a->n_latent; ++d) o[d] = 0.0;
            if (nvalid == 0) {
                lse[(int64_t)r * a->n_heads + h] = -INFINITY;
                if (probs)
                    for (j = 0; j < a->k; ++j) probs[((int64_t)r * a->n_heads + h) * a->k + j] = 0.0;
                continue;
            }
            for (j = 0; j < a->k; ++j) {
                double acc = 0.0;
                if (!valid[j]) continue;
                for (i = 0; i < D; ++i) acc += (double)qh[i] * K[(int64_t)j * D + i];
                s[j] = a->sm_scale * acc;
                if (s[j] > m) m = s[j];
            }
            for (j = 0; j < a->k; ++j) {
                double p;
                if (!valid[j]) continue;
                p = exp(s[j] - m);
                l += p;
                for (d = 0; d < a->n_latent; ++d) o[d] += p * K[(int64_t)j * D + d];
            }
            for (d = 0; d < a->n_latent; ++d) o[d] /= l;
            lse[(int64_t)r * a->n_heads + h] = m + log(l);
            if (probs)
                for (j = 0; j < a->k; ++j)
                    probs[((int64_t)r * a->n_heads + h) * a->k + j] = valid[j] ? exp(s[j] - m) / l : 0.0;
        }
        free(K);
        free(s);
        free(valid);
    }
    if (err) *err |= err_all;
}

/* ------------------------------------------------ (o, lse) state merge */

/* Merge n_parts attention states of the same (row, head) into one ([P1-PAR]):
 *   M = max_s lse_s, w_s = exp(lse_s - M), W = sum_s w_s
 *   o = sum_s w_s o_s / W, lse = M + ln W
 * Parts with lse = -inf carry no weight; if all are -inf, o = 0, lse = -inf.
 * part_o[(s * n_states + t) * dim + d], part_lse[s * n_states + t]. */
void o_merge_states(const double *part_o, const double *part_lse, int n_parts, int64_t n_states,
                    int dim, double *out, double *lse)
{
    int64_t t;
#pragma omp parallel for schedule(static)
    for (t = 0; t < n_states; ++t) {
        double M = -INFINITY, W = 0.0;
        int s, d;
        for (s = 0; s < n_parts; ++s)
            if (part_lse[(int64_t)s * n_states + t] > M) M = part_lse[(int64_t)s * n_states + t];
        for (d = 0; d < dim; ++d) out[t * dim + d] = 0.0;
        if (M == -INFINITY) { lse[t] = -INFINITY; continue; }
        for (s = 0; s < n_parts; ++s) {
            double ls = part_lse[(int64_t)s * n_states + t], w;
            if (ls == -INFINITY) continue;
            w = exp(ls - M);
            W += w;
            for (d = 0; d < dim; ++d) out[t * dim + d] += w * part_o[((int64_t)s * n_states + t) * dim + d];
        }
        for (d = 0; d < dim; ++d) out[t * dim + d] /= W;
        lse[t] = M + log(W);
    }
}
