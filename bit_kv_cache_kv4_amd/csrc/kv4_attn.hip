// Sparse MLA attention over the 4-bit pool: decode (split-K) and prefill.
//
// README "60+ inference optimizations & kernels": section "4-bit KV cache"
// (kv4mla dequantizes the 4-bit rows on chip instead of into an FP8 scratch
// copy), section "AMD MI355X" (hand-written HIP sparse MLA decode whose K tile
// in LDS is also the PV operand through a transposing LDS read; split-K
// decode), "Parallelism and disaggregation" (per-part (o, lse) and a merge).
// sgl-amd-mono GLM-5.3 PR, "Modifications": 64-token page table and its stride
// as launch arguments; a split task serves many heads so each key row is
// gathered once per task.
//
// Workgroup = 4 wavefronts = (query row r, split s, chunk of up to 64 heads),
// one per SIMD with the whole register file (queries and accumulators stay in
// registers).  Wavefront w = (head group hg = w / 2 of 32 heads, half h = w %
// 2).  Per tile of 32 list entries:
//   1. the entries' pool slots (translated once per chunk of 2048 entries and
//      kept in LDS) name 32 rows; lane t gathers row t % 32, bytes of part
//      t / 32 (64 latent dims, their 4 scales, 8 rope dims) straight from HBM,
//      two tiles ahead of the math;
//   2. the lanes dequantize with gfx950's FP4/FP8 -> fp16 conversions at scale
//      1 and one packed multiply by the E4M3 block scale (every product is exact
//      in fp16) into a row-major K tile [32 rows][576] in LDS, double-buffered
//      so this overlaps the previous tile's scores;
//   3. wavefront (hg, h) computes the partial scores S^T[32 rows x 32 heads]
//      over dims 288h..288h+287 with v_mfma_f32_32x32x16_f16 (queries in
//      registers, pre-scaled per head by a power of two so they are exact in
//      fp16), swaps partials with its partner through LDS, and accumulates
//      O^T[256 dims x 32 heads] for latent dims 256h..256h+255 with the same
//      MFMA from P = 2^(s - m_ref), where m_ref is the head's largest score in
//      the first tile that has a valid entry (so the accumulators are never
//      rescaled).  If a later score exceeds m_ref + 15 (P could overflow fp16)
//      the workgroup runs the list again with m_ref = the exact maximum seen,
//      which the first pass tracked.  P^T comes
//      straight from the score registers and V^T from the K tile through
//      ds_read_b64_tr_b16, which hands each lane a column of a row-major 4x16
//      block.
// The per-split result is written normalised with its lse; a split count of 1
// writes the final output.
#include "kv4_device.h"
#include "kv4_launch.h"

namespace kv4 {

constexpr int kTile = 32;                              // list entries per tile
constexpr int kKChunks = 80;                           // 16-byte chunks per K-tile row (72 used)
constexpr int kKRowBytes = kKChunks * 16;
constexpr int kKTileBytes = kTile * kKRowBytes;        // 40960
constexpr int kXBytes = 4 * 64 * 16 * 4 + 16;          // partial scores: 4 wavefronts x 64 lanes x 16, + a flag
constexpr int kSlotCap = 2048;                         // entries translated per chunk
constexpr int kLdsBytes = 2 * kKTileBytes + kXBytes + kSlotCap * 4;   // 106496
constexpr float kRefSlack = 15.0f;                     // log2 headroom of fp16 P above its reference

typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef short short4_t __attribute__((ext_vector_type(4)));

// K-tile layout: row r starts at r * 1280 + 16 * krot(r) bytes (chunks of 16
// bytes, 72 used, up to 7 chunks of shift).  krot maps eight consecutive rows
// onto eight distinct 16-byte bank groups, so the score operand reads (one
// chunk of rows r..r+7) are conflict-free, and rows 4g..4g+3 start 32 bytes
// apart modulo 128, so the transposing reads (32 bytes of each of 4 rows) are
// too.  Every address is a per-lane base plus a compile-time offset.
__device__ __forceinline__ int krot(int r) { return (2 * (r & 3)) | ((r >> 2) & 1); }
__device__ __forceinline__ int krow(int r) { return r * kKRowBytes + 16 * krot(r); }

__device__ __forceinline__ floatx16_t mfma32(half8_t a, half8_t b, floatx16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ short4_t lds_read_tr16(const uint8_t *lds_base, int byte_off) {
    typedef __attribute__((address_space(3))) short4_t lds_short4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_short4 *)((__attribute__((address_space(3))) uint8_t *)lds_base + byte_off));
}

// One lane's share of a tile's rows: row t % 32, part t / 32 (latent dims
// 64 part .. +63 as 32 code bytes, their 4 block scales, rope dims 8 part .. +7).
struct RowPart {
    u32x4_t c0, c1;
    uint32_t sc;
    u32x2_t rp;
    bool valid;
};

// A skipped entry reads row 0 (the pool has at least one row whenever a slot
// can be valid) and is zeroed by dequant_part: scale and rope bytes become 0.
__device__ __forceinline__ void gather_part(const uint8_t *__restrict__ pool, int32_t slot, int gp, RowPart &R) {
    R.valid = slot >= 0;
    const uint8_t *row = pool + (int64_t)(R.valid ? slot : 0) * kRowBytes;
    R.c0 = *reinterpret_cast<const u32x4_t *>(row + 32 * gp);
    R.c1 = *reinterpret_cast<const u32x4_t *>(row + 32 * gp + 16);
    R.sc = *reinterpret_cast<const uint32_t *>(row + kScaleOff + 4 * gp);
    R.rp = *reinterpret_cast<const u32x2_t *>(row + kRopeOff + 8 * gp);
}

__device__ __forceinline__ void dequant_part(uint8_t *ktile, int gr, int gp, const RowPart &R) {
    const uint32_t sc = R.valid ? R.sc : 0u;
    const u32x2_t rp = R.valid ? R.rp : u32x2_t{0, 0};
    const half2_t d0 = block_scale_half(sc & 0xFFu), d1 = block_scale_half((sc >> 8) & 0xFFu);
    const half2_t d2 = block_scale_half((sc >> 16) & 0xFFu), d3 = block_scale_half(sc >> 24);
    uint8_t *kr = ktile + krow(gr) + 128 * gp;
    uint32_t v[4];
    e2m1x8_to_half_cvt(R.c0[0], d0, v);
    *reinterpret_cast<u32x4_t *>(kr + 0) = u32x4_t{v[0], v[1], v[2], v[3]};
    e2m1x8_to_half_cvt(R.c0[1], d0, v);
    *reinterpret_cast<u32x4_t *>(kr + 16) = u32x4_t{v[0], v[1], v[2], v[3]};
    e2m1x8_to_half_cvt(R.c0[2], d1, v);
    *reinterpret_cast<u32x4_t *>(kr + 32) = u32x4_t{v[0], v[1], v[2], v[3]};
    e2m1x8_to_half_cvt(R.c0[3], d1, v);
    *reinterpret_cast<u32x4_t *>(kr + 48) = u32x4_t{v[0], v[1], v[2], v[3]};
    e2m1x8_to_half_cvt(R.c1[0], d2, v);
    *reinterpret_cast<u32x4_t *>(kr + 64) = u32x4_t{v[0], v[1], v[2], v[3]};
    e2m1x8_to_half_cvt(R.c1[1], d2, v);
    *reinterpret_cast<u32x4_t *>(kr + 80) = u32x4_t{v[0], v[1], v[2], v[3]};
    e2m1x8_to_half_cvt(R.c1[2], d3, v);
    *reinterpret_cast<u32x4_t *>(kr + 96) = u32x4_t{v[0], v[1], v[2], v[3]};
    e2m1x8_to_half_cvt(R.c1[3], d3, v);
    *reinterpret_cast<u32x4_t *>(kr + 112) = u32x4_t{v[0], v[1], v[2], v[3]};
    uint32_t h[4];
    e4m3x4_to_half_cvt(rp[0], h);
    e4m3x4_to_half_cvt(rp[1], h + 2);
    *reinterpret_cast<u32x4_t *>(ktile + krow(gr) + 16 * (64 + gp)) = u32x4_t{h[0], h[1], h[2], h[3]};
}

constexpr int kPosPerLane = kSlotCap / 256;

template <bool QF32>
__global__ __launch_bounds__(256, 1) void sparse_mla_kernel(AttnParams p) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
    floatx4_t *xbuf = reinterpret_cast<floatx4_t *>(lds + 2 * kKTileBytes);
    int32_t *redo = reinterpret_cast<int32_t *>(lds + 2 * kKTileBytes + kXBytes - 16);
    int32_t *slots = reinterpret_cast<int32_t *>(lds + 2 * kKTileBytes + kXBytes);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = blockIdx.x, split = blockIdx.y;
    const int hg = blockIdx.z * 2 + (wave >> 1);
    const int half = wave & 1;
    const int l32 = lane & 31, g = lane >> 5;
    const int head = hg * 32 + l32;
    const bool group_live = hg * 32 < p.n_heads;
    const bool head_live = head < p.n_heads;

    const int n_tiles = (p.k + kTile - 1) / kTile;
    const int t_lo = split * p.tiles_per_split;
    const int t_hi = min(n_tiles, t_lo + p.tiles_per_split);
    const int e_lo = t_lo * kTile;
    const int e_hi = min(p.k, t_hi * kTile);

    const int32_t req = p.row_req ? p.row_req[r] : r;
    const bool bad_req = p.page_table && (req < 0 || req >= p.pt_n_rows);
    const int32_t *pt_row = p.page_table && !bad_req ? p.page_table + (int64_t)req * p.pt_row_stride : nullptr;
    const int32_t *list = p.topk + (int64_t)r * p.topk_row_stride;
    uint32_t err = 0;

    // Translation of a chunk of at most kSlotCap entries into slots[]: the
    // list entries first, then their page-table entries, each batch issued
    // before any of it is used.
    int32_t pos[kPosPerLane], phys[kPosPerLane];
    auto load_positions = [&](int c_lo, int c_hi) {
#pragma unroll
        for (int i = 0; i < kPosPerLane; ++i) {
            const int e = tid + 256 * i;
            pos[i] = c_lo + e < c_hi ? list[c_lo + e] : -1;
        }
    };
    auto load_pages = [&]() {
#pragma unroll
        for (int i = 0; i < kPosPerLane; ++i) {
            phys[i] = -1;
            if (pt_row && pos[i] >= 0 && (pos[i] >> p.page_shift) < p.pt_n_pages) phys[i] = pt_row[pos[i] >> p.page_shift];
        }
    };
    auto write_slots = [&](int n_entries) {
#pragma unroll
        for (int i = 0; i < kPosPerLane; ++i) {
            const int e = tid + 256 * i;
            if (e >= n_entries) break;
            int64_t s = -1;
            if (bad_req) err |= pos[i] >= 0 ? kErrPage : 0u;
            else s = slot_of(pos[i], phys[i], pt_row != nullptr, p.pt_n_pages, p.page_shift, p.n_slots, err);
            slots[e] = (int32_t)s;
        }
    };

    // first chunk's list entries are in flight while the queries load
    const int first_hi = min(e_hi, e_lo + kSlotCap);
    if (e_lo < e_hi) load_positions(e_lo, first_hi);

    // ---- queries: B operand of S^T = K Q^T.  Lane (l32, g) holds head l32,
    // dims 288*half + 16ks + 8g .. +7 for ks = 0..17.  The power-of-two scale
    // qs puts the head's largest |q| in [2^13, 2^14): exact in fp16.  All of
    // the head's loads are issued before any is used.
    half8_t qb[18];
    half8_t ql[QF32 ? 18 : 1];
    float score_mul = 0.0f;
    {
        const int64_t hoff = (int64_t)r * p.q_row_stride + (int64_t)head * p.q_head_stride + 8 * g;
        float qmax = 0.0f;
        if constexpr (QF32) {
            const float *qp = reinterpret_cast<const float *>(p.q) + hoff;
            float4 own[36];
            float4 other[36];
#pragma unroll
            for (int ks = 0; ks < 18; ++ks) {
                const int mine = 288 * half + 16 * ks, theirs = 288 * (half ^ 1) + 16 * ks;
                own[2 * ks] = own[2 * ks + 1] = other[2 * ks] = other[2 * ks + 1] = float4{0, 0, 0, 0};
                if (head_live) {
                    own[2 * ks] = *reinterpret_cast<const float4 *>(qp + mine);
                    own[2 * ks + 1] = *reinterpret_cast<const float4 *>(qp + mine + 4);
                    other[2 * ks] = *reinterpret_cast<const float4 *>(qp + theirs);
                    other[2 * ks + 1] = *reinterpret_cast<const float4 *>(qp + theirs + 4);
                }
            }
            if (e_lo < e_hi) load_pages();
#pragma unroll
            for (int i = 0; i < 36; ++i) {
                const float4 a = own[i], b = other[i];
                qmax = __builtin_fmaxf(qmax, __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(a.x), __builtin_fabsf(a.y)),
                                                             __builtin_fmaxf(__builtin_fabsf(a.z), __builtin_fabsf(a.w))));
                qmax = __builtin_fmaxf(qmax, __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(b.x), __builtin_fabsf(b.y)),
                                                             __builtin_fmaxf(__builtin_fabsf(b.z), __builtin_fabsf(b.w))));
            }
            qmax = __builtin_fmaxf(qmax, __shfl_xor(qmax, 32));
            int ex = 0;
            if (qmax > 0.0f) (void)__builtin_frexpf(qmax, &ex);
            const float qs = __builtin_ldexpf(1.0f, 14 - ex);     // qmax * qs < 2^14
            score_mul = p.score_mul / qs;
#pragma unroll
            for (int ks = 0; ks < 18; ++ks) {
                const float v[8] = {own[2 * ks].x, own[2 * ks].y, own[2 * ks].z, own[2 * ks].w,
                                    own[2 * ks + 1].x, own[2 * ks + 1].y, own[2 * ks + 1].z, own[2 * ks + 1].w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = v[e] * qs;
                    const _Float16 hi = (_Float16)x;
                    qb[ks][e] = hi;
                    ql[ks][e] = (_Float16)(x - (float)hi);
                }
            }
        } else {
            const uint16_t *qp = reinterpret_cast<const uint16_t *>(p.q) + hoff;
            u32x4_t own[18], other[18];
#pragma unroll
            for (int ks = 0; ks < 18; ++ks) {
                own[ks] = other[ks] = u32x4_t{0, 0, 0, 0};
                if (head_live) {
                    own[ks] = *reinterpret_cast<const u32x4_t *>(qp + 288 * half + 16 * ks);
                    other[ks] = *reinterpret_cast<const u32x4_t *>(qp + 288 * (half ^ 1) + 16 * ks);
                }
            }
            if (e_lo < e_hi) load_pages();
#pragma unroll
            for (int ks = 0; ks < 18; ++ks)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    qmax = __builtin_fmaxf(qmax, __builtin_fmaxf(__builtin_fabsf(__uint_as_float(own[ks][c] << 16)),
                                                                 __builtin_fabsf(__uint_as_float(own[ks][c] & 0xFFFF0000u))));
                    qmax = __builtin_fmaxf(qmax, __builtin_fmaxf(__builtin_fabsf(__uint_as_float(other[ks][c] << 16)),
                                                                 __builtin_fabsf(__uint_as_float(other[ks][c] & 0xFFFF0000u))));
                }
            qmax = __builtin_fmaxf(qmax, __shfl_xor(qmax, 32));
            int ex = 0;
            if (qmax > 0.0f) (void)__builtin_frexpf(qmax, &ex);
            const float qs = __builtin_ldexpf(1.0f, 14 - ex);     // qmax * qs < 2^14
            score_mul = p.score_mul / qs;
#pragma unroll
            for (int ks = 0; ks < 18; ++ks)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    qb[ks][2 * c] = (_Float16)(__uint_as_float(own[ks][c] << 16) * qs);
                    qb[ks][2 * c + 1] = (_Float16)(__uint_as_float(own[ks][c] & 0xFFFF0000u) * qs);
                }
        }
    }
    // pad to whole tiles: entries past the chunk's end get slot -1
    if (e_lo < e_hi) write_slots((first_hi - e_lo + kTile - 1) / kTile * kTile);
    if (tid == 0) *redo = 0;                       // set only in pass 0; read after its last barrier
    __syncthreads();

    floatx16_t o[8];
    float m_ref = -__builtin_inff();   // reference of P = 2^(s - m_ref) for this lane's head
    float m_max = -__builtin_inff();   // largest score seen (the exact maximum after a pass)
    float l_run = 0.0f;

    const int gr = tid & 31, gp = tid >> 5;        // gather role: row gr, part gp
    // score operand: row l32, chunk 36*half + 2ks + g
    const int qk_off = krow(l32) + 16 * (36 * half + g);
    // transposing reads: this lane supplies row 4g + (lane&15)/4 (+8 for the
    // second read of a k-half, +16 for the second k-half), 8 bytes at latent
    // dims 256*half + 32*md + 16*((lane>>4)&1) + 4*(lane&3)
    const int tr_off = krow(4 * g + ((lane >> 2) & 3)) + 2 * (256 * half + 16 * ((lane >> 4) & 1) + 4 * (lane & 3));

    // One tile: scores from buffer tt&1 while rows of tile tt+1 (held in nxt)
    // are dequantized into the other buffer and rows of tile tt+3 are
    // requested into nxt; then softmax and P.V.
    auto tile_step = [&](int tt, int n_t, RowPart &nxt) {
        const uint8_t *kcur = lds + (tt & 1) * kKTileBytes;
        const uint64_t vmask = __ballot(lane < kTile && slots[tt * kTile + lane] >= 0);
        floatx16_t sacc = {};
        if (group_live) {
            if constexpr (QF32) {
#pragma unroll
                for (int ks = 0; ks < 18; ++ks) {
                    const half8_t a = *reinterpret_cast<const half8_t *>(kcur + qk_off + 32 * ks);
                    sacc = mfma32(a, qb[ks], sacc);
                    sacc = mfma32(a, ql[ks], sacc);
                    if (ks % 3 == 2) __builtin_amdgcn_sched_barrier(0);   // bound the read-ahead window
                }
            } else {
                floatx16_t s2 = {};
#pragma unroll
                for (int ks = 0; ks < 18; ++ks) {
                    const half8_t a = *reinterpret_cast<const half8_t *>(kcur + qk_off + 32 * ks);
                    if (ks & 1) s2 = mfma32(a, qb[ks], s2);
                    else sacc = mfma32(a, qb[ks], sacc);
                }
                sacc += s2;
            }
        }
        if (tt + 1 < n_t) dequant_part(lds + ((tt + 1) & 1) * kKTileBytes, gr, gp, nxt);
        if (tt + 3 < n_t) gather_part(p.pool, slots[(tt + 3) * kTile + gr], gp, nxt);
        if (group_live) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
                xbuf[(wave * 4 + q4) * 64 + lane] = floatx4_t{sacc[4 * q4], sacc[4 * q4 + 1], sacc[4 * q4 + 2], sacc[4 * q4 + 3]};
        }
        __syncthreads();                           // partial scores and the next tile visible
        if (group_live) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const floatx4_t o4 = xbuf[((wave ^ 1) * 4 + q4) * 64 + lane];
                sacc[4 * q4] += o4[0];
                sacc[4 * q4 + 1] += o4[1];
                sacc[4 * q4 + 2] += o4[2];
                sacc[4 * q4 + 3] += o4[3];
            }
            // ---- softmax numerators.  Register v holds row 8(v/4) + 4g + v%4.
            float sc16[16];
#pragma unroll
            for (int v = 0; v < 16; ++v) sc16[v] = sacc[v] * score_mul;
            if ((uint32_t)vmask != 0xFFFFFFFFu) {      // a tile with skipped entries
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int row = 8 * (v >> 2) + 4 * g + (v & 3);
                    if (!((vmask >> row) & 1)) sc16[v] = -__builtin_inff();
                }
            }
            float tmax = sc16[0];
#pragma unroll
            for (int v = 1; v < 16; ++v) tmax = __builtin_fmaxf(tmax, sc16[v]);
            tmax = __builtin_fmaxf(tmax, __shfl_xor(tmax, 32));
            m_max = __builtin_fmaxf(m_max, tmax);
            if (m_ref == -__builtin_inff()) m_ref = tmax;    // first tile with a valid entry
            if (tmax > m_ref + kRefSlack) *redo = 1;         // P could overflow fp16 (pass 0 only)
            half8_t pb0, pb1;
            float lsum = 0.0f;
            const float mr = m_ref == -__builtin_inff() ? 0.0f : m_ref;   // nothing valid so far
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float pv = __builtin_amdgcn_exp2f(sc16[v] - mr);   // exp2(-inf) = 0
                lsum += pv;
                if (v < 8) pb0[v] = (_Float16)pv;
                else pb1[v - 8] = (_Float16)pv;
            }
            l_run += lsum;
            // ---- O^T[256 x 32] += V^T P^T, V^T through transposing reads
#pragma unroll
            for (int md = 0; md < 8; ++md) {
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const short4_t lo = lds_read_tr16(kcur, tr_off + kKRowBytes * (16 * kk) + 64 * md);
                    const short4_t hi = lds_read_tr16(kcur, tr_off + kKRowBytes * (16 * kk + 8) + 64 * md);
                    const half8_t a = __builtin_bit_cast(half8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                    o[md] = mfma32(a, kk ? pb1 : pb0, o[md]);
                }
                if constexpr (QF32) __builtin_amdgcn_sched_barrier(0);
            }
        }
        __syncthreads();                           // this tile's buffer and the partial scores are free
    };

    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = floatx16_t{};
        l_run = 0.0f;
        if (pass == 1) m_ref = m_max;              // the exact maximum: no P can exceed 1
        for (int c_lo = e_lo; c_lo < e_hi; c_lo += kSlotCap) {
            const int c_hi = min(e_hi, c_lo + kSlotCap);
            const int n_t = (c_hi - c_lo + kTile - 1) / kTile;
            if (c_lo != e_lo || (pass == 1 && e_hi - e_lo > kSlotCap)) {
                __syncthreads();                   // slots of the previous chunk are no longer read
                load_positions(c_lo, c_hi);
                load_pages();
                write_slots(n_t * kTile);
                __syncthreads();
            }
            RowPart ra, rb;
            gather_part(p.pool, slots[gr], gp, ra);
            if (n_t > 1) gather_part(p.pool, slots[kTile + gr], gp, rb);
            dequant_part(lds, gr, gp, ra);
            if (n_t > 2) gather_part(p.pool, slots[2 * kTile + gr], gp, ra);
            __syncthreads();                       // tile 0 in buffer 0
            for (int tt = 0; tt < n_t; tt += 2) {
                tile_step(tt, n_t, rb);            // rb: tile tt+1 -> buffer, then tile tt+3
                if (tt + 1 < n_t) tile_step(tt + 1, n_t, ra);   // ra: tile tt+2 -> buffer, then tile tt+4
            }
        }
        if (pass == 1 || *redo == 0) break;        // uniform: read after the last barrier
    }

    if (err && p.err_word) atomicOr(p.err_word, err);
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float m_fin = m_ref == -__builtin_inff() ? 0.0f : m_ref;
    if (!head_live) return;
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    float *orow = p.out + (int64_t)split * p.out_split_stride + (int64_t)r * p.out_row_stride + (int64_t)head * kLatent;
#pragma unroll
    for (int md = 0; md < 8; ++md)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int d = 256 * half + 32 * md + 8 * j + 4 * g;
            *reinterpret_cast<floatx4_t *>(orow + d) =
                floatx4_t{o[md][4 * j], o[md][4 * j + 1], o[md][4 * j + 2], o[md][4 * j + 3]} * inv;
        }
    if (half == 0 && g == 0 && p.lse) {
        const float lse = l_tot > 0.0f ? (m_fin + __builtin_log2f(l_tot)) * 0.69314718055994530942f : -__builtin_inff();
        p.lse[(int64_t)split * p.lse_split_stride + (int64_t)r * p.lse_row_stride + head] = lse;
    }
}

hipError_t launch_sparse_mla(const AttnParams &p, bool q_f32, int32_t n_splits, hipStream_t stream) {
    if (p.n_rows == 0) return hipSuccess;
    const dim3 grid((unsigned)p.n_rows, (unsigned)n_splits, (unsigned)((p.n_heads + 63) / 64));
    if (q_f32) hipLaunchKernelGGL(sparse_mla_kernel<true>, grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL(sparse_mla_kernel<false>, grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

// --------------------------------------------------- dequantizing gather

// One workgroup per (query row, tile of 32 entries): translate, then the same
// lane roles and decoding as the attention kernel, written row-major to HBM.
__global__ __launch_bounds__(256) void gather_dequant_kernel(AttnParams p, uint16_t *__restrict__ out,
                                                             int32_t *__restrict__ slots_out) {
    __shared__ int32_t slots[kTile];
    const int tid = threadIdx.x, r = blockIdx.x, tile = blockIdx.y;
    const int32_t req = p.row_req ? p.row_req[r] : r;
    const bool bad_req = p.page_table && (req < 0 || req >= p.pt_n_rows);
    const int32_t *pt_row = p.page_table && !bad_req ? p.page_table + (int64_t)req * p.pt_row_stride : nullptr;
    uint32_t err = 0;
    if (tid < kTile) {
        const int e = tile * kTile + tid;
        int64_t s = -1;
        if (e < p.k) {
            const int32_t pos = p.topk[(int64_t)r * p.topk_row_stride + e];
            if (bad_req) err |= pos >= 0 ? kErrPage : 0u;
            else s = translate_slot(pos, pt_row, p.pt_n_pages, p.page_shift, p.n_slots, err);
            if (slots_out) slots_out[(int64_t)r * p.k + e] = (int32_t)s;
        }
        slots[tid] = (int32_t)s;
        if (err && p.err_word) atomicOr(p.err_word, err);
    }
    __syncthreads();
    const int pp = tid & 15, qc = tid >> 4;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int row = 2 * pp + h, e = tile * kTile + row;
        if (e >= p.k) continue;
        const int32_t s = slots[row];
        u32x4_t codes = {0, 0, 0, 0};
        uint32_t sc = 0;
        if (s >= 0) {
            const uint8_t *src = p.pool + (int64_t)s * kRowBytes;
            codes = *reinterpret_cast<const u32x4_t *>(src + 16 * qc);
            sc = *reinterpret_cast<const uint16_t *>(src + kScaleOff + 2 * qc);
        }
        uint32_t v[16];
        dequant_chunk(codes, sc, v);
        uint32_t *dst = reinterpret_cast<uint32_t *>(out + ((int64_t)r * p.k + e) * kDim) + 16 * qc;
#pragma unroll
        for (int c = 0; c < 4; ++c)
            *reinterpret_cast<u32x4_t *>(dst + 4 * c) = u32x4_t{v[4 * c], v[4 * c + 1], v[4 * c + 2], v[4 * c + 3]};
    }
    if (tid < 128) {
        const int row = tid >> 2, e = tile * kTile + row;
        if (e < p.k) {
            const int32_t s = slots[row];
            u32x4_t b = {0, 0, 0, 0};
            if (s >= 0) b = *reinterpret_cast<const u32x4_t *>(p.pool + (int64_t)s * kRowBytes + kRopeOff + 16 * (tid & 3));
            uint32_t h[8];
            dequant_rope16(b, h);
            uint32_t *dst = reinterpret_cast<uint32_t *>(out + ((int64_t)r * p.k + e) * kDim) + kLatent / 2 + 8 * (tid & 3);
            *reinterpret_cast<u32x4_t *>(dst) = u32x4_t{h[0], h[1], h[2], h[3]};
            *reinterpret_cast<u32x4_t *>(dst + 4) = u32x4_t{h[4], h[5], h[6], h[7]};
        }
    }
}

hipError_t launch_gather_dequant(const AttnParams &p, uint16_t *out, int32_t *slots_out, hipStream_t stream) {
    if (p.n_rows == 0 || p.k == 0) return hipSuccess;
    const dim3 grid((unsigned)p.n_rows, (unsigned)((p.k + kTile - 1) / kTile));
    hipLaunchKernelGGL(gather_dequant_kernel, grid, dim3(256), 0, stream, p, out, slots_out);
    return hipGetLastError();
}

// ----------------------------------------------------------------- merge

__global__ __launch_bounds__(128) void merge_states_kernel(MergeParams p) {
    __shared__ float w[64];
    __shared__ float stat[2];
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x;
    if (tid == 0) {
        float M = -__builtin_inff();
        for (int s = 0; s < p.n_parts; ++s) M = __builtin_fmaxf(M, p.part_lse[(int64_t)s * p.n_states + t]);
        stat[0] = M;
    }
    __syncthreads();
    const float M = stat[0];
    if (M != -__builtin_inff() && tid < p.n_parts) {
        const float ls = p.part_lse[(int64_t)tid * p.n_states + t];
        w[tid] = ls == -__builtin_inff() ? 0.0f : expf(ls - M);
    }
    __syncthreads();
    if (tid == 0) {
        float W = 0.0f;
        if (M != -__builtin_inff())
            for (int s = 0; s < p.n_parts; ++s) W += w[s];
        stat[1] = W;
        if (p.lse) p.lse[t] = M == -__builtin_inff() ? M : M + logf(W);
    }
    __syncthreads();
    const float W = stat[1];
    const float inv = W > 0.0f ? 1.0f / W : 0.0f;
    float *orow = p.out + (t / p.states_per_row) * p.out_row_stride + (t % p.states_per_row) * p.out_col_stride;
    for (int d = 4 * tid; d < p.dim; d += 512) {
        floatx4_t acc = {0, 0, 0, 0};
        if (W > 0.0f)
            for (int s = 0; s < p.n_parts; ++s) {
                const float ws = w[s];
                if (ws != 0.0f)
                    acc += ws * *reinterpret_cast<const floatx4_t *>(p.part_o + ((int64_t)s * p.n_states + t) * p.dim + d);
            }
        *reinterpret_cast<floatx4_t *>(orow + d) = acc * inv;
    }
}

hipError_t launch_merge_states(const MergeParams &p, hipStream_t stream) {
    if (p.n_states == 0) return hipSuccess;
    hipLaunchKernelGGL(merge_states_kernel, dim3((unsigned)p.n_states), dim3(128), 0, stream, p);
    return hipGetLastError();
}

}  // namespace kv4
