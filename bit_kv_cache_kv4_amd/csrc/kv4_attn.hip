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

#include <type_traits>

namespace kv4 {

constexpr int kTile = 32;                              // list entries per tile
constexpr int kKChunks = 76;                           // 16-byte chunks per K-tile row: 72 + shift
constexpr int kKRowBytes = kKChunks * 16;              // 1216
constexpr int kKTileBytes = kTile * kKRowBytes;        // 38912
constexpr int kXBytes = 4 * 64 * 16 * 4;               // partial scores: 4 wavefronts x 64 lanes x 16
constexpr int kSlotCap = 1024;                         // entries translated per chunk
constexpr int kKBufs = 3;                              // K tiles in flight: P.V(t), scores(t+1), dequant(t+2)
constexpr int kSlotOff = kKBufs * kKTileBytes + 2 * kXBytes + 16;
constexpr int kCountOff = kSlotOff + kSlotCap * 4;   // valid entries per (batch, wavefront) of a chunk
constexpr int kLdsBytes = kCountOff + 64;             // 153680
constexpr float kRefSlack = 15.0f;                     // log2 headroom of fp16 P above its reference

typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef short short4_t __attribute__((ext_vector_type(4)));

// K-tile layout for gfx950's LDS (64 banks of 4 bytes, 256 bytes a clock):
// row r starts at r * 1216 + 16 * ((r >> 2) & 3).  In 16-byte slots modulo
// 256 bytes that is 12r + (r >> 2) mod 16, so rows 0..15 (and 16..31) sit in
// 16 distinct slots: the score reads and the dequantizing writes (16 rows per
// 16 lanes) are conflict-free.  Rows 4m..4m+3 sit in slots congruent modulo
// 4, so their 64-byte spans in a transposing read (4 rows x 64 bytes per 32
// lanes) tile the 256 bytes.  Every address is a per-lane base plus a
// compile-time offset.
__host__ __device__ constexpr int krow(int r) { return r * kKRowBytes + 16 * ((r >> 2) & 3); }
static_assert(krow(kTile - 1) + 2 * kDim <= kKTileBytes, "K-tile rows overlap");

__device__ __forceinline__ floatx16_t mfma32(half8_t a, half8_t b, floatx16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// LDS accesses by 32-bit byte address.  Each step pins (makes opaque to the
// optimiser) one per-lane base per access pattern, so every access of the step
// is that base plus a constant the instruction's offset field holds.
typedef __attribute__((address_space(3))) uint8_t lds_u8_t;
__device__ __forceinline__ uint32_t lds_addr(uint8_t *p) { return (uint32_t)(size_t)(lds_u8_t *)p; }
__device__ __forceinline__ uint32_t pin(uint32_t v) {
    asm("" : "+v"(v));
    return v;
}
template <typename T>
__device__ __forceinline__ T lds_ld(uint32_t a) {
    return *(const __attribute__((address_space(3))) T *)(size_t)a;
}
template <typename T>
__device__ __forceinline__ void lds_st(uint32_t a, T v) {
    *(__attribute__((address_space(3))) T *)(size_t)a = v;
}
__device__ __forceinline__ short4_t lds_read_tr16(uint32_t a) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t *)(size_t)a);
}

// One lane's share of a tile's rows: row t % 32, part t / 32 (latent dims
// 64 part .. +63 as 32 code bytes, their 4 block scales, rope dims 8 part .. +7).
struct RowPart {
    u32x4_t c0, c1;
    uint32_t sc;
    u32x2_t rp;
    bool valid;
};

// A skipped entry reads 352 readable bytes elsewhere (`stand_in`: the query
// row, at least 1152 bytes, so an empty pool is never touched) and is zeroed by
// dequant_part: scale and rope bytes become 0, so every value is 0.
__device__ __forceinline__ void gather_part(const uint8_t *__restrict__ pool, const uint8_t *stand_in, int32_t slot,
                                            int gp, RowPart &R) {
    R.valid = slot >= 0;
    const uint8_t *row = R.valid ? pool + (int64_t)slot * kRowBytes : stand_in;
    R.c0 = *reinterpret_cast<const u32x4_t *>(row + 32 * gp);
    R.c1 = *reinterpret_cast<const u32x4_t *>(row + 32 * gp + 16);
    R.sc = *reinterpret_cast<const uint32_t *>(row + kScaleOff + 4 * gp);
    R.rp = *reinterpret_cast<const u32x2_t *>(row + kRopeOff + 8 * gp);
}

// dq = K-tile row base + 128 * part (latent chunks), rq = row base + 16 * (64 + part)
__device__ __forceinline__ void dequant_part(uint32_t dq, uint32_t rq, const RowPart &R) {
    const uint32_t sc = R.valid ? R.sc : 0u;
    const u32x2_t rp = R.valid ? R.rp : u32x2_t{0, 0};
    half2_t d[4];
    block_scales_half_cvt(sc, d);
    const uint32_t c[8] = {R.c0[0], R.c0[1], R.c0[2], R.c0[3], R.c1[0], R.c1[1], R.c1[2], R.c1[3]};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t v[4];
        e2m1x8_to_half_cvt(c[i], d[i >> 1], v);
        lds_st<u32x4_t>(dq + 16 * i, u32x4_t{v[0], v[1], v[2], v[3]});
    }
    uint32_t h[4];
    e4m3x4_to_half_cvt(rp[0], h);
    e4m3x4_to_half_cvt(rp[1], h + 2);
    lds_st<u32x4_t>(rq, u32x4_t{h[0], h[1], h[2], h[3]});
}

constexpr int kPosPerLane = kSlotCap / 256;

template <bool QF32>
__global__ __launch_bounds__(256, 1) void sparse_mla_kernel(AttnParams p) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
    int32_t *redo = reinterpret_cast<int32_t *>(lds + kKBufs * kKTileBytes + 2 * kXBytes);
    int32_t *slots = reinterpret_cast<int32_t *>(lds + kSlotOff);
    int32_t *counts = reinterpret_cast<int32_t *>(lds + kCountOff);

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

    // Translation of a chunk of at most kSlotCap entries: the list entries
    // first, then their page-table entries, each batch issued before any of it
    // is used.  write_slots packs the valid entries' slots, in list order, to
    // the front of slots[] and pads the last tile with -1, so every tile but
    // the last is full; it returns the number of valid entries (the same in
    // every thread) and holds a barrier, so all threads call it.
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
    auto write_slots = [&]() -> int {
        int32_t sl[kPosPerLane];
        uint64_t bal[kPosPerLane];
#pragma unroll
        for (int i = 0; i < kPosPerLane; ++i) {       // entry e = tid + 256 i: list order is (i, wave, lane)
            int64_t s = -1;
            if (bad_req) err |= pos[i] >= 0 ? kErrPage : 0u;
            else s = slot_of(pos[i], phys[i], pt_row != nullptr, p.pt_n_pages, p.page_shift, p.n_slots, err);
            sl[i] = (int32_t)s;
            bal[i] = __ballot(s >= 0);
            if (lane == 0) counts[4 * i + wave] = (int32_t)__popcll(bal[i]);
        }
        __syncthreads();
        int nv = 0, base[kPosPerLane];
#pragma unroll
        for (int i = 0; i < kPosPerLane; ++i) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                if (w == wave) base[i] = nv;
                nv += counts[4 * i + w];
            }
        }
#pragma unroll
        for (int i = 0; i < kPosPerLane; ++i) {
            const int below = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal[i] >> 32),
                                                             __builtin_amdgcn_mbcnt_lo((uint32_t)bal[i], 0u));
            if (sl[i] >= 0) slots[base[i] + below] = sl[i];
            const int e = tid + 256 * i;
            if (e >= nv && e < ((nv + kTile - 1) & ~(kTile - 1))) slots[e] = -1;
        }
        return nv;
    };

    // first chunk's list entries are in flight while the queries load
    const int first_hi = min(e_hi, e_lo + kSlotCap);
    if (e_lo < e_hi) load_positions(e_lo, first_hi);
    else load_positions(0, 0);

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
    int nv = e_lo < e_hi ? write_slots() : 0;      // valid entries of the current chunk
    if (tid == 0) *redo = 0;                       // set only in pass 0; read after its last barrier
    __syncthreads();

    floatx16_t o[8];
    float m_ref = -__builtin_inff();   // reference of P = 2^(s - m_ref) for this lane's head
    float m_max = -__builtin_inff();   // largest score seen (the exact maximum after a pass)
    float l_run = 0.0f;

    const int gr = tid & 31, gp = tid >> 5;        // gather role: row gr, part gp
    const uint8_t *stand_in = reinterpret_cast<const uint8_t *>(p.q);
    // per-lane offsets inside a K tile:
    //  score operand: row l32, chunk 36*half + 2ks + g
    const uint32_t qk_off = krow(l32) + 16 * (36 * half + g);
    //  transposing reads: this lane supplies row 4g + (lane&15)/4 (+8 for the
    //  second read of a k-half, +16 for the second k-half), 8 bytes at latent
    //  dims 256*half + 32*md + 16*((lane>>4)&1) + 4*(lane&3)
    const uint32_t tr_off = krow(4 * g + ((lane >> 2) & 3)) + 2 * (256 * half + 16 * ((lane >> 4) & 1) + 4 * (lane & 3));
    //  dequantized row gr, part gp: 8 latent chunks and one rope chunk
    const uint32_t dq_off = krow(gr) + 128 * gp;
    const uint32_t rope_off = krow(gr) + 16 * (64 + gp);
    const uint32_t kb0 = lds_addr(lds);
    // exchange buffers: wavefront w's partial of register group q4 for lane l
    // at (w*4 + q4)*64 + l (16 bytes each); buffer xb at xb * kXBytes
    const uint32_t x_own = pin(kb0 + kKBufs * kKTileBytes + wave * 4096 + 16 * lane);
    const uint32_t x_partner = pin(kb0 + kKBufs * kKTileBytes + (wave ^ 1) * 4096 + 16 * lane);

    // partial scores S^T over this half's 288 dims for the K tile at sb (=
    // tile + qk_off), written to exchange buffer xb (one accumulator chain;
    // fp32 queries add their lo parts into the same chain)
    auto scores_to_x = [&](uint32_t sb, int xb) {
        floatx16_t sacc = {};
#pragma unroll
        for (int ks = 0; ks < 18; ++ks) {
            const half8_t a = lds_ld<half8_t>(sb + 32 * ks);
            sacc = mfma32(a, qb[ks], sacc);
            if constexpr (QF32) sacc = mfma32(a, ql[ks], sacc);
        }
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
            lds_st<floatx4_t>(x_own + xb * kXBytes + 1024 * q4,
                              floatx4_t{sacc[4 * q4], sacc[4 * q4 + 1], sacc[4 * q4 + 2], sacc[4 * q4 + 3]});
    };

    // P of tile t from exchange buffer xb: own + partner partial scores,
    // P = 2^(s - m_ref) as the two fp16 B operands of P.V; updates l_run (the
    // sum of the fp16 P that P.V uses), m_ref, m_max.  The chunk's last tile
    // takes the masked form, where the padding rows' scores become -inf.
    half8_t pb0 = {}, pb1 = {};
    bool need_redo = false;
    int last_rows = kTile;                             // valid rows of the chunk's last tile
    // O^T[256 x 32] += V^T P^T for the K tile at tb (= tile + tr_off), V^T
    // through transposing reads.  The lane's base row is 0..7 (shift 0 or 1),
    // so row base + d (d = 0, 8, 16, 24) starts krow(d) bytes further on.
    auto pv = [&](uint32_t tb) {
#pragma unroll
        for (int md = 0; md < 8; ++md) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const short4_t lo = lds_read_tr16(tb + krow(16 * kk) + 64 * md);
                const short4_t hi = lds_read_tr16(tb + krow(16 * kk + 8) + 64 * md);
                const half8_t a = __builtin_bit_cast(half8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                o[md] = mfma32(a, kk ? pb1 : pb0, o[md]);
            }
        }
    };

    // Steady state, iteration t (one barrier), laid out by hand: the
    // scheduler is fenced (sched_barrier) after every MFMA slot so that
    // operand reads stay a few MFMAs ahead and the VALU work sits between the
    // MFMAs.  Slots 0..17 (36 for fp32 queries): the scores of tile t+1 (K
    // tile at bB, into exchange buffer xb^1) with the softmax of tile t
    // (buffer xb) spread over them.  Slots 0..15 of the second loop: P.V of
    // tile t (bA) with the dequantization of tile t+2 (rows held in cur, into
    // bC) and then the gather of tile t+4 into cur.  Past the chunk's end the
    // scores, dequant and gather work on stale buffers nobody reads (the
    // gather index is clamped to a real tile).
    auto iteration = [&](auto masked, int t, int n_t, RowPart &cur, uint32_t bA, uint32_t bB, uint32_t bC, int xb) {
        constexpr int kAhead = 4;                     // score operand reads in flight
        constexpr int kTrAhead = 3;                   // P.V operand pairs in flight
        const uint32_t sb = pin(bB + qk_off), tb = pin(bA + tr_off);
        const uint32_t dq = pin(bC + dq_off), rq = pin(bC + rope_off);
        const int32_t next_slot = slots[min(t + 4, n_t - 1) * kTile + gr];
        floatx4_t xo[4], xq[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            xo[q4] = lds_ld<floatx4_t>(x_own + xb * kXBytes + 1024 * q4);
            xq[q4] = lds_ld<floatx4_t>(x_partner + xb * kXBytes + 1024 * q4);
        }
        half8_t ka[kAhead];
#pragma unroll
        for (int i = 0; i < kAhead; ++i) ka[i] = lds_ld<half8_t>(sb + 32 * i);
        __builtin_amdgcn_sched_barrier(0);

        float raw[16];
        float rmax = 0.0f, nmr = 0.0f, l0 = 0.0f, l1 = 0.0f;
        const half2_t one2 = {(_Float16)1.0f, (_Float16)1.0f};
        floatx16_t sacc = {};
#pragma unroll
        for (int ks = 0; ks < 18; ++ks) {
            sacc = mfma32(ka[ks % kAhead], qb[ks], sacc);
            if constexpr (QF32) sacc = mfma32(ka[ks % kAhead], ql[ks], sacc);
            if (ks + kAhead < 18) ka[ks % kAhead] = lds_ld<half8_t>(sb + 32 * (ks + kAhead));
            // softmax of tile t, a piece per slot
            if (ks == 1 || ks == 2) {                 // own + partner partial scores
#pragma unroll
                for (int q4 = 2 * (ks - 1); q4 < 2 * ks; ++q4)
#pragma unroll
                    for (int i = 0; i < 4; ++i) raw[4 * q4 + i] = xo[q4][i] + xq[q4][i];
            }
            if (ks == 3) {
                if constexpr (decltype(masked)::value) {   // the chunk's last tile: rows >= last_rows are padding
                    const int lim = last_rows - 4 * g;      // register v holds row 8(v/4) + 4g + v%4
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        if (8 * (v >> 2) + (v & 3) >= lim) raw[v] = -__builtin_inff();
                }
                rmax = __builtin_fmaxf(__builtin_fmaxf(raw[0], raw[1]), raw[2]);
#pragma unroll
                for (int v = 3; v < 15; v += 2) rmax = __builtin_fmaxf(__builtin_fmaxf(rmax, raw[v]), raw[v + 1]);
                rmax = __builtin_fmaxf(rmax, raw[15]);
            }
            if (ks == 4) {
                // lanes l and l ^ 32 hold the same head
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(rmax), __float_as_uint(rmax), false, false);
                const float tmax = __builtin_fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * score_mul;
                m_max = __builtin_fmaxf(m_max, tmax);
                if (m_ref == -__builtin_inff()) m_ref = tmax;    // first tile with a valid entry
                need_redo |= tmax > m_ref + kRefSlack;           // P could overflow fp16 (pass 0 only)
                nmr = m_ref == -__builtin_inff() ? 0.0f : -m_ref;   // nothing valid so far
            }
            if (ks >= 5 && ks < 13) {                 // P = 2^(s - m_ref), two per slot; exp2(-inf) = 0
#pragma unroll
                for (int v = 2 * (ks - 5); v < 2 * (ks - 4); ++v) {
                    const _Float16 ph = (_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf(raw[v], score_mul, nmr));
                    if (v < 8) pb0[v] = ph;
                    else pb1[v - 8] = ph;
                }
            }
            if (ks == 13 || ks == 14) {               // l += the fp16 P that P.V uses
                const int i0 = 2 * (ks - 13);
#pragma unroll
                for (int i = i0; i < i0 + 2; ++i) {
                    l0 = __builtin_amdgcn_fdot2(half2_t{pb0[2 * i], pb0[2 * i + 1]}, one2, l0, false);
                    l1 = __builtin_amdgcn_fdot2(half2_t{pb1[2 * i], pb1[2 * i + 1]}, one2, l1, false);
                }
            }
            if (ks == 15) l_run += l0 + l1;
            __builtin_amdgcn_sched_barrier(0);
        }

        // P.V of tile t with the dequantization of tile t+2
        short4_t tlo[kTrAhead], thi[kTrAhead];
        auto tr_issue = [&](int j, int slot) {
            const int md = j >> 1, kk = j & 1;
            tlo[slot] = lds_read_tr16(tb + krow(16 * kk) + 64 * md);
            thi[slot] = lds_read_tr16(tb + krow(16 * kk + 8) + 64 * md);
        };
#pragma unroll
        for (int j = 0; j < kTrAhead; ++j) tr_issue(j, j);
        __builtin_amdgcn_sched_barrier(0);
        half2_t d[4];
        const uint32_t cw[8] = {cur.c0[0], cur.c0[1], cur.c0[2], cur.c0[3], cur.c1[0], cur.c1[1], cur.c1[2], cur.c1[3]};
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int md = j >> 1, kk = j & 1;
            const half8_t a = __builtin_bit_cast(
                half8_t, __builtin_shufflevector(tlo[j % kTrAhead], thi[j % kTrAhead], 0, 1, 2, 3, 4, 5, 6, 7));
            o[md] = mfma32(a, kk ? pb1 : pb0, o[md]);
            if (j + kTrAhead < 16) tr_issue(j + kTrAhead, j % kTrAhead);
            if (j == 0) block_scales_half_cvt(cur.valid ? cur.sc : 0u, d);
            if (j >= 1 && j <= 8) {                   // latent chunk j-1 of this lane's part
                uint32_t v[4];
                e2m1x8_to_half_cvt(cw[j - 1], d[(j - 1) >> 1], v);
                lds_st<u32x4_t>(dq + 16 * (j - 1), u32x4_t{v[0], v[1], v[2], v[3]});
            }
            if (j == 3) {                             // the scores of tile t+1 to the exchange buffer
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                    lds_st<floatx4_t>(x_own + (xb ^ 1) * kXBytes + 1024 * q4,
                                      floatx4_t{sacc[4 * q4], sacc[4 * q4 + 1], sacc[4 * q4 + 2], sacc[4 * q4 + 3]});
            }
            if (j == 9) {                             // rope chunk
                const u32x2_t rp = cur.valid ? cur.rp : u32x2_t{0, 0};
                uint32_t h[4];
                e4m3x4_to_half_cvt(rp[0], h);
                e4m3x4_to_half_cvt(rp[1], h + 2);
                lds_st<u32x4_t>(rq, u32x4_t{h[0], h[1], h[2], h[3]});
            }
            if (j == 10) gather_part(p.pool, stand_in, next_slot, gp, cur);
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
    };

    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = floatx16_t{};
        l_run = 0.0f;
        if (pass == 1) m_ref = m_max;              // the exact maximum: no P can exceed 1
        for (int c_lo = e_lo; c_lo < e_hi; c_lo += kSlotCap) {
            const int c_hi = min(e_hi, c_lo + kSlotCap);
            if (c_lo != e_lo || (pass == 1 && e_hi - e_lo > kSlotCap)) {
                __syncthreads();                   // slots of the previous chunk are no longer read
                load_positions(c_lo, c_hi);
                load_pages();
                nv = write_slots();
                __syncthreads();
            }
            const int n_t = (nv + kTile - 1) / kTile;
            if (n_t == 0) continue;                // nothing valid in this chunk (uniform)
            last_rows = nv - kTile * (n_t - 1);
            // prologue: tiles 0 and 1 into buffers 0 and 1, tiles 2 and 3 in
            // flight in registers, scores of tile 0
            uint32_t bA = kb0, bB = kb0 + kKTileBytes, bC = kb0 + 2 * kKTileBytes;
            RowPart r0, r1;
            gather_part(p.pool, stand_in, slots[gr], gp, r0);
            gather_part(p.pool, stand_in, slots[min(1, n_t - 1) * kTile + gr], gp, r1);
            dequant_part(pin(bA + dq_off), pin(bA + rope_off), r0);
            gather_part(p.pool, stand_in, slots[min(2, n_t - 1) * kTile + gr], gp, r0);
            dequant_part(pin(bB + dq_off), pin(bB + rope_off), r1);
            gather_part(p.pool, stand_in, slots[min(3, n_t - 1) * kTile + gr], gp, r1);
            __syncthreads();                       // tiles 0 and 1 in LDS
            scores_to_x(pin(bA + qk_off), 0);
            __syncthreads();
            // full tiles two at a time, then the last one or two with the
            // last tile masked
            int t = 0;
            for (; t + 2 < n_t; t += 2) {
                iteration(std::false_type{}, t, n_t, r0, bA, bB, bC, 0);       // r0: tile t+2 -> LDS, then t+4
                iteration(std::false_type{}, t + 1, n_t, r1, bB, bC, bA, 1);   // r1: tile t+3 -> LDS, then t+5
                const uint32_t a0 = bA;            // tiles t+2, t+3, t+4 go to bC, bA, bB
                bA = bC;
                bC = bB;
                bB = a0;
            }
            if (t + 1 < n_t) {
                iteration(std::false_type{}, t, n_t, r0, bA, bB, bC, 0);
                iteration(std::true_type{}, t + 1, n_t, r1, bB, bC, bA, 1);
            } else {
                iteration(std::true_type{}, t, n_t, r0, bA, bB, bC, 0);
            }
            if (need_redo) *redo = 1;
            __syncthreads();                       // buffers free for the next chunk or pass
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
