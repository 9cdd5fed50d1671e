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
//
// Rows are either the 352-byte format (576 dims: 512 latent + 64 rope) or the
// 288-byte rope-free format (512 latent dims; README, "4-bit KV cache": the
// rope-free row of GLM-5.3-Flash).  The rope-free kernel is the same with 16
// score k-steps per half instead of 18 and no rope to gather or decode; it
// keeps the same slot schedule and LDS layout (the last 8 chunks of each K
// tile unused).
#include "kv4_attn.h"
#include "kv4_device.h"

#include <type_traits>

namespace kv4 {

constexpr int kTile = 32;                              // list entries per tile
constexpr int kKChunkBytes = 576;                      // one 16-byte chunk of the 32 rows + 4 slots
constexpr int kKTileBytes = 72 * kKChunkBytes;         // 41472
constexpr int kXBytes = 4 * 64 * 16 * 4;               // partial scores: 4 wavefronts x 64 lanes x 16
constexpr int kSlotCap = 1024;                         // entries translated per chunk
constexpr int kKBufs = 3;                              // K tiles in flight: P.V(t), scores(t+1), dequant(t+2)
constexpr int kSlotOff = kKBufs * kKTileBytes + 2 * kXBytes + 16;
constexpr int kCountOff = kSlotOff + kSlotCap * 4;   // valid entries per (batch, wavefront) of a chunk
constexpr int kQmaxOff = kCountOff + 64;              // per-head query maxima of each wavefront
constexpr int kLdsBytes = kQmaxOff + 4 * 32 * 4;      // 161872
constexpr float kRefSlack = 15.0f;                     // log2 headroom of fp16 P above its reference

typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));

// K-tile layout, chunk-major: element (row r, dim d) is at
// (d / 8) * 576 + 16 r + 2 (d % 8), i.e. the 32 rows' copies of one 16-byte
// chunk are contiguous, padded to 36 slots.  A score operand read (one chunk of
// 32 rows per 32 lanes) and a dequantizing write (one chunk per 32 lanes) each
// touch 512 contiguous bytes; a transposing read (4 rows x 4 chunks per 32
// lanes) touches four 64-byte pieces whose 16-byte slots modulo 256 bytes are
// 4q + 4g + j, all distinct because 36 = 4 mod 16.  gfx950's LDS serves each
// at its full rate (256 bytes a clock for reads, 128 for writes) with no bank
// conflict, and every address is a per-lane base plus a compile-time offset.
constexpr int kcb(int chunk) { return chunk * kKChunkBytes; }

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
// Row layout: 352 bytes with the 64 rope values, or the 288-byte rope-free
// row (codes and scales only, README "60+ inference optimizations & kernels",
// section "4-bit KV cache": GLM-5.3-Flash's rope-free row).
template <bool ROPE>
constexpr int row_bytes() { return ROPE ? kRowBytes : kScaleOff + kLatent / 16; }

template <bool ROPE>
__device__ __forceinline__ void gather_part(const uint8_t *__restrict__ pool, const uint8_t *stand_in, int32_t slot,
                                            int gp, RowPart &R) {
    R.valid = slot >= 0;
    const uint8_t *row = R.valid ? pool + (int64_t)slot * row_bytes<ROPE>() : stand_in;
    R.c0 = *reinterpret_cast<const u32x4_t *>(row + 32 * gp);
    R.c1 = *reinterpret_cast<const u32x4_t *>(row + 32 * gp + 16);
    R.sc = *reinterpret_cast<const uint32_t *>(row + kScaleOff + 4 * gp);
    if constexpr (ROPE) R.rp = *reinterpret_cast<const u32x2_t *>(row + kRopeOff + 8 * gp);
    else R.rp = u32x2_t{0, 0};
}

// dq = the lane's row in its part's first latent chunk (chunk 8 * part), rq =
// the lane's row in its rope chunk (chunk 64 + part)
template <bool ROPE>
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
        lds_st<u32x4_t>(dq + kcb(i), u32x4_t{v[0], v[1], v[2], v[3]});
    }
    if constexpr (ROPE) {
        uint32_t h[4];
        e4m3x4_to_half_cvt(rp[0], h);
        e4m3x4_to_half_cvt(rp[1], h + 2);
        lds_st<u32x4_t>(rq, u32x4_t{h[0], h[1], h[2], h[3]});
    }
}

constexpr int kPosPerLane = kSlotCap / 256;

// f(integral_constant<int, I>) for I = B .. E-1, each with its index known at
// compile time (a plain loop this large is not unrolled by the compiler)
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

template <bool QF32, bool ROPE>
__global__ __launch_bounds__(256, 1) void sparse_mla_kernel(AttnParams p) {
    // row format: K has kD dims (latent + rope, or latent only); each half of
    // the scores covers kD / 2 of them in kSteps MFMA k-steps of 16
    constexpr int kD = ROPE ? kDim : kLatent;
    constexpr int kSteps = kD / 32;
    constexpr int kHalfChunks = kD / 16;
    constexpr int kRowB = row_bytes<ROPE>();
    __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
    int32_t *redo = reinterpret_cast<int32_t *>(lds + kKBufs * kKTileBytes + 2 * kXBytes);
    int32_t *slots = reinterpret_cast<int32_t *>(lds + kSlotOff);
    int32_t *counts = reinterpret_cast<int32_t *>(lds + kCountOff);
    float *qmx = reinterpret_cast<float *>(lds + kQmaxOff);
    const uint32_t kb0 = lds_addr(lds);

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

    // ---- Prologue, arranged so its memory round trips overlap: the first
    // chunk's list entries, then this workgroup's queries (coalesced:
    // consecutive lanes take consecutive 16-byte chunks of a head's row), the
    // page-table entries once the list is back, the queries staged in LDS (the
    // K-tile buffers are not in use yet; rows padded so the fragment reads
    // below are conflict-free), and the slots.  The query fragments are read,
    // scaled and converted in the first chunk's prologue, while its first
    // tiles are being gathered.
    constexpr int kQElem = QF32 ? 4 : 2;
    constexpr int kQChunks = kD * kQElem / 16;             // 16-byte chunks per head row
    constexpr int kQRow = kD * kQElem + 16;                // staged head row (at most 2320 bytes)
    constexpr int kQPer = 64 * kQChunks / 256;             // chunks per thread
    static_assert(64 * kQRow <= kSlotOff - 16, "staged queries overlap the slot list");
    const int first_hi = min(e_hi, e_lo + kSlotCap);
    if (e_lo < e_hi) load_positions(e_lo, first_hi);       // issued first: loads complete in order
    else load_positions(0, 0);
    {
        const int h0 = blockIdx.z * 64;
        const uint8_t *qr = reinterpret_cast<const uint8_t *>(p.q) + (int64_t)r * p.q_row_stride * kQElem;
        u32x4_t qc[kQPer];
#pragma unroll
        for (int i = 0; i < kQPer; ++i) {
            const int c = tid + 256 * i, hh = c / kQChunks, part = c % kQChunks;
            qc[i] = u32x4_t{0, 0, 0, 0};
            if (h0 + hh < p.n_heads)
                qc[i] = *reinterpret_cast<const u32x4_t *>(qr + (int64_t)(h0 + hh) * p.q_head_stride * kQElem + 16 * part);
        }
        if (e_lo < e_hi) load_pages();
#pragma unroll
        for (int i = 0; i < kQPer; ++i) {
            const int c = tid + 256 * i, hh = c / kQChunks, part = c % kQChunks;
            lds_st<u32x4_t>(kb0 + hh * kQRow + 16 * part, qc[i]);
        }
    }
    int nv = e_lo < e_hi ? write_slots() : 0;      // valid entries of the current chunk (holds a barrier)
    if (tid == 0) *redo = 0;                       // set only in pass 0; read after its last barrier
    __syncthreads();

    // ---- queries: B operand of S^T = K Q^T.  Lane (l32, g) holds head l32,
    // dims 288*half + 16ks + 8g .. +7 for ks = 0..17.  The power-of-two scale
    // qs puts the head's largest |q| in [2^13, 2^14): exact in fp16 (fp32
    // queries: a hi and a lo fp16 part).  Run once, with a barrier, by every
    // thread (the largest |q| of the head's other half comes from the partner
    // wavefront through LDS).
    half8_t qb[kSteps];
    half8_t ql[QF32 ? kSteps : 1];
    float score_mul = 0.0f;
    auto convert_queries = [&]() {
        const uint32_t qf = kb0 + ((wave >> 1) * 32 + l32) * kQRow + (kD / 2 * half + 8 * g) * kQElem;
        float qmax = 0.0f;
        if constexpr (QF32) {
            floatx4_t v[2 * kSteps];
#pragma unroll
            for (int ks = 0; ks < kSteps; ++ks) {
                v[2 * ks] = lds_ld<floatx4_t>(qf + 64 * ks);
                v[2 * ks + 1] = lds_ld<floatx4_t>(qf + 64 * ks + 16);
            }
#pragma unroll
            for (int i = 0; i < 2 * kSteps; ++i)
                qmax = __builtin_fmaxf(qmax, __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(v[i][0]), __builtin_fabsf(v[i][1])),
                                                             __builtin_fmaxf(__builtin_fabsf(v[i][2]), __builtin_fabsf(v[i][3]))));
            qmax = __builtin_fmaxf(qmax, __shfl_xor(qmax, 32));
            if (g == 0) qmx[wave * 32 + l32] = qmax;
            __syncthreads();
            qmax = __builtin_fmaxf(qmax, qmx[(wave ^ 1) * 32 + l32]);
            int ex = 0;
            if (qmax > 0.0f) (void)__builtin_frexpf(qmax, &ex);
            const float qs = __builtin_ldexpf(1.0f, 14 - ex);     // qmax * qs < 2^14
            score_mul = p.score_mul / qs;
#pragma unroll
            for (int ks = 0; ks < kSteps; ++ks)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = v[2 * ks + (e >> 2)][e & 3] * qs;
                    const _Float16 hi = (_Float16)x;
                    qb[ks][e] = hi;
                    ql[ks][e] = (_Float16)(x - (float)hi);
                }
        } else {
            u32x4_t v[kSteps];
#pragma unroll
            for (int ks = 0; ks < kSteps; ++ks) v[ks] = lds_ld<u32x4_t>(qf + 32 * ks);
#pragma unroll
            for (int ks = 0; ks < kSteps; ++ks)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    qmax = __builtin_fmaxf(qmax, __builtin_fmaxf(__builtin_fabsf(__uint_as_float(v[ks][c] << 16)),
                                                                 __builtin_fabsf(__uint_as_float(v[ks][c] & 0xFFFF0000u))));
            qmax = __builtin_fmaxf(qmax, __shfl_xor(qmax, 32));
            if (g == 0) qmx[wave * 32 + l32] = qmax;
            __syncthreads();
            qmax = __builtin_fmaxf(qmax, qmx[(wave ^ 1) * 32 + l32]);
            int ex = 0;
            if (qmax > 0.0f) (void)__builtin_frexpf(qmax, &ex);
            const float qs = __builtin_ldexpf(1.0f, 14 - ex);     // qmax * qs < 2^14
            score_mul = p.score_mul / qs;
#pragma unroll
            for (int ks = 0; ks < kSteps; ++ks)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    qb[ks][2 * c] = (_Float16)(__uint_as_float(v[ks][c] << 16) * qs);
                    qb[ks][2 * c + 1] = (_Float16)(__uint_as_float(v[ks][c] & 0xFFFF0000u) * qs);
                }
        }
    };

    floatx16_t o[8];
    float m_ref = -__builtin_inff();   // reference of P = 2^(s - m_ref) for this lane's head
    float m_max = -__builtin_inff();   // largest score seen (the exact maximum after a pass)
    float l_run = 0.0f;

    const int gr = tid & 31, gp = tid >> 5;        // gather role: row gr, part gp
    const uint8_t *stand_in = reinterpret_cast<const uint8_t *>(p.q);
    // per-lane offsets inside a K tile:
    //  score operand: row l32 of chunk 36*half + 2ks + g
    const uint32_t qk_off = kcb(kHalfChunks * half + g) + 16 * l32;
    //  transposing reads: this lane supplies row 4g + (lane&15)/4 (+8 for the
    //  second read of a k-half, +16 for the second k-half), 8 bytes at latent
    //  dims 256*half + 32*md + 16*((lane>>4)&1) + 4*(lane&3)
    const uint32_t tr_off = kcb(32 * half + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)) +
                            16 * (4 * g + ((lane >> 2) & 3)) + 8 * (lane & 1);
    //  dequantized row gr, part gp: latent chunks 8gp..8gp+7 and rope chunk 64+gp
    const uint32_t dq_off = kcb(8 * gp) + 16 * gr;
    const uint32_t rope_off = kcb(64 + gp) + 16 * gr;
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
        for (int ks = 0; ks < kSteps; ++ks) {
            const half8_t a = lds_ld<half8_t>(sb + kcb(2 * ks));
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
    // Steady state, iteration t (one barrier), laid out by hand as 34 MFMA
    // slots: 18 score MFMAs of tile t+1 (K tile at bB, into exchange buffer
    // xb^1; 36 for fp32 queries) then 16 P.V MFMAs of tile t (bA), the first
    // half of P first.  The scheduler is fenced (sched_barrier) after every
    // slot, so operand reads stay a few MFMAs ahead and each slot's other
    // work sits beside its MFMA.  That work is spread evenly because a
    // wavefront issues in order (a value that is not ready stalls it) and
    // gfx950's LDS takes writes at about 64 bytes a clock per CU:
    //  - the softmax of tile t (exchange buffer xb): sums, a max tree, then
    //    fma -> exp -> fp16 -> row sums, one step per slot;
    //  - the dequantization of tile t+2 (rows held in cur, into bC): chunk i
    //    converted in one slot, scaled and stored a slot later, a store every
    //    four slots, interleaved with the four stores of the new scores;
    //  - the gather of tile t+4 into cur, each piece as soon as its
    //    registers are free.
    // Past the chunk's end the scores, dequant and gather work on stale
    // buffers nobody reads (the gather index is clamped to a real tile).
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
        for (int i = 0; i < kAhead; ++i) ka[i] = lds_ld<half8_t>(sb + kcb(2 * i));
        __builtin_amdgcn_sched_barrier(0);

        short4_t tlo[kTrAhead], thi[kTrAhead];
        auto tr_issue = [&](int j) {                  // P.V MFMA j: k-half kk = j / 8, dims block md = j % 8
            const int md = j & 7, kk = j >> 3;
            tlo[j % kTrAhead] = lds_read_tr16(tb + kcb(4 * md) + 16 * (16 * kk));
            thi[j % kTrAhead] = lds_read_tr16(tb + kcb(4 * md) + 16 * (16 * kk + 8));
        };
        float raw[16], mx[7], e[16], ls[4];
        float tmax = 0.0f, nmr = 0.0f;
        uint32_t sw0 = 0, sw1 = 0, sc_sel = 0, cv[2][4], rh[4];
        u32x2_t rp_sel = {0, 0};
        half2_t d[4];
        const uint8_t *nrow = stand_in;
        bool nvalid = false;
        const half2_t one2 = {(_Float16)1.0f, (_Float16)1.0f};
        auto cvt_chunk = [&](int i) {                 // E2M1 codes of latent chunk i -> fp16 at scale 1
            const uint32_t w = i < 4 ? cur.c0[i] : cur.c1[i - 4];
            cv[i & 1][0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0));
            cv[i & 1][1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1));
            cv[i & 1][2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2));
            cv[i & 1][3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3));
        };
        auto scale_store = [&](int i) {               // times the block scale, to the K tile
            const half2_t di = d[i >> 1];
            lds_st<u32x4_t>(dq + kcb(i), u32x4_t{__builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, cv[i & 1][0]) * di),
                                                 __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, cv[i & 1][1]) * di),
                                                 __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, cv[i & 1][2]) * di),
                                                 __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, cv[i & 1][3]) * di)});
        };
        auto x_store = [&](const floatx16_t &sacc, int q4) {   // new scores for the partner
            lds_st<floatx4_t>(x_own + (xb ^ 1) * kXBytes + 1024 * q4,
                              floatx4_t{sacc[4 * q4], sacc[4 * q4 + 1], sacc[4 * q4 + 2], sacc[4 * q4 + 3]});
        };
        floatx16_t sacc = {};
        // The softmax of tile t delivers P in slots 16 and 17, so P.V starts at
        // slot 18 in both row formats; the rope-free scores take slots 0..15
        // and leave 16 and 17 without an MFMA.
        static_for<0, 34>([&](auto slot) {
            constexpr int s = decltype(slot)::value;
            // ---- the MFMA of the slot and the operand reads ahead of it
            if constexpr (s < kSteps) {
                sacc = mfma32(ka[s % kAhead], qb[s], sacc);
                if constexpr (QF32) sacc = mfma32(ka[s % kAhead], ql[s], sacc);
                if constexpr (s + kAhead < kSteps) ka[s % kAhead] = lds_ld<half8_t>(sb + kcb(2 * (s + kAhead)));
            } else if constexpr (s >= 18) {
                constexpr int j = s - 18, md = j & 7, kk = j >> 3;
                const half8_t a = __builtin_bit_cast(
                    half8_t, __builtin_shufflevector(tlo[j % kTrAhead], thi[j % kTrAhead], 0, 1, 2, 3, 4, 5, 6, 7));
                o[md] = mfma32(a, kk ? pb1 : pb0, o[md]);
                if constexpr (j + kTrAhead < 16) tr_issue(j + kTrAhead);
            }
            if constexpr (s >= 18 - kTrAhead && s < 18) tr_issue(s - (18 - kTrAhead));
            // ---- softmax of tile t
            if constexpr (s == 1 || s == 2) {                   // own + partner partial scores
#pragma unroll
                for (int q4 = 2 * (s - 1); q4 < 2 * s; ++q4)
#pragma unroll
                    for (int i = 0; i < 4; ++i) raw[4 * q4 + i] = xo[q4][i] + xq[q4][i];
            }
            if constexpr (s == 2) {
                if constexpr (decltype(masked)::value) {   // the chunk's last tile: rows >= last_rows are padding
                    const int lim = last_rows - 4 * g;      // register v holds row 8(v/4) + 4g + v%4
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        if (8 * (v >> 2) + (v & 3) >= lim) raw[v] = -__builtin_inff();
                }
            }
            if constexpr (s == 3) {                             // row maximum as a tree
#pragma unroll
                for (int i = 0; i < 5; ++i)
                    mx[i] = __builtin_fmaxf(__builtin_fmaxf(raw[3 * i], raw[3 * i + 1]), raw[3 * i + 2]);
            }
            if constexpr (s == 4) {
                mx[5] = __builtin_fmaxf(__builtin_fmaxf(mx[0], mx[1]), mx[2]);
                mx[6] = __builtin_fmaxf(__builtin_fmaxf(mx[3], mx[4]), raw[15]);
            }
            if constexpr (s == 5) {                             // lanes l and l ^ 32 hold the same head
                const float rm = __builtin_fmaxf(mx[5], mx[6]);
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(rm), __float_as_uint(rm), false, false);
                sw0 = sw[0];
                sw1 = sw[1];
            }
            if constexpr (s == 6) tmax = __builtin_fmaxf(__uint_as_float(sw0), __uint_as_float(sw1)) * score_mul;   // score_mul > 0
            if constexpr (s == 7) {
                m_max = __builtin_fmaxf(m_max, tmax);
                if (m_ref == -__builtin_inff()) m_ref = tmax;    // first tile with a valid entry
                need_redo |= tmax > m_ref + kRefSlack;           // P could overflow fp16 (pass 0 only)
                nmr = m_ref == -__builtin_inff() ? 0.0f : -m_ref;   // nothing valid so far
            }
            if constexpr (s >= 8 && s < 16) {                   // exponent of two values, 2^ of the previous two
                constexpr int u = s - 8;
                if constexpr (u > 0) {
                    e[2 * u - 2] = __builtin_amdgcn_exp2f(e[2 * u - 2]);   // exp2(-inf) = 0
                    e[2 * u - 1] = __builtin_amdgcn_exp2f(e[2 * u - 1]);
                }
                e[2 * u] = __builtin_fmaf(raw[2 * u], score_mul, nmr);
                e[2 * u + 1] = __builtin_fmaf(raw[2 * u + 1], score_mul, nmr);
            }
            if constexpr (s == 16) {
                e[14] = __builtin_amdgcn_exp2f(e[14]);
                e[15] = __builtin_amdgcn_exp2f(e[15]);
#pragma unroll
                for (int v = 0; v < 8; ++v) pb0[v] = (_Float16)e[v];
            }
            if constexpr (s == 17) {
#pragma unroll
                for (int v = 0; v < 8; ++v) pb1[v] = (_Float16)e[8 + v];
            }
            if constexpr (s == 18 || s == 19) {                 // l += the fp16 P that P.V uses: four partial sums
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const half2_t pp = s == 18 ? half2_t{pb0[2 * i], pb0[2 * i + 1]} : half2_t{pb1[2 * i], pb1[2 * i + 1]};
                    ls[i] = __builtin_amdgcn_fdot2(pp, one2, s == 18 ? 0.0f : ls[i], false);
                }
            }
            if constexpr (s == 20) {
                ls[0] += ls[1];
                ls[2] += ls[3];
            }
            if constexpr (s == 21) ls[0] += ls[2];
            if constexpr (s == 22) l_run += ls[0];
            // ---- dequantization of tile t+2
            if constexpr (s == 0) {                             // a skipped entry dequantizes to zeros
                sc_sel = cur.valid ? cur.sc : 0u;
                rp_sel = cur.valid ? cur.rp : u32x2_t{0, 0};
                block_scales_half_cvt(sc_sel, d);
            }
            constexpr int ci = s >= 1 && (s - 1) % 4 == 0 && (s - 1) / 4 < 8 ? (s - 1) / 4 : -1;
            constexpr int si = s >= 2 && (s - 2) % 4 == 0 && (s - 2) / 4 < 8 ? (s - 2) / 4 : -1;
            if constexpr (ci >= 0) cvt_chunk(ci);    // chunk i converted in slot 1 + 4i
            if constexpr (si >= 0) scale_store(si);  // and stored a slot later
            if constexpr (ROPE && s == 31) {
                e4m3x4_to_half_cvt(rp_sel[0], rh);
                e4m3x4_to_half_cvt(rp_sel[1], rh + 2);
            }
            if constexpr (ROPE && s == 32) lds_st<u32x4_t>(rq, u32x4_t{rh[0], rh[1], rh[2], rh[3]});
            // ---- the new scores to the exchange buffer, between the dequant stores
            if constexpr (s == 20 || s == 24 || s == 28 || s == 33) x_store(sacc, s == 33 ? 3 : (s - 20) / 4);
            // ---- gather of tile t+4 into cur, piece by piece
            if constexpr (s == 3) {
                nvalid = next_slot >= 0;
                nrow = nvalid ? p.pool + (int64_t)next_slot * kRowB : stand_in;
            }
            if constexpr (s == 7) {
                cur.valid = nvalid;
                cur.sc = *reinterpret_cast<const uint32_t *>(nrow + kScaleOff + 4 * gp);
            }
            if constexpr (s == 14) cur.c0 = *reinterpret_cast<const u32x4_t *>(nrow + 32 * gp);
            if constexpr (s == 30) cur.c1 = *reinterpret_cast<const u32x4_t *>(nrow + 32 * gp + 16);
            if constexpr (ROPE && s == 32) cur.rp = *reinterpret_cast<const u32x2_t *>(nrow + kRopeOff + 8 * gp);
            __builtin_amdgcn_sched_barrier(0);
        });
        __syncthreads();
    };

    // the first chunk's first two tiles are on their way while the queries
    // are converted (the staged queries are read before its barrier, so the
    // tiles may then overwrite them)
    RowPart r0, r1;
    {
        const int n_t0 = (nv + kTile - 1) / kTile;
        if (n_t0 > 0) {
            gather_part<ROPE>(p.pool, stand_in, slots[gr], gp, r0);
            gather_part<ROPE>(p.pool, stand_in, slots[min(1, n_t0 - 1) * kTile + gr], gp, r1);
        }
        convert_queries();
    }

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
            if (pass == 1 || c_lo != e_lo) {       // the first chunk's were gathered before the passes
                gather_part<ROPE>(p.pool, stand_in, slots[gr], gp, r0);
                gather_part<ROPE>(p.pool, stand_in, slots[min(1, n_t - 1) * kTile + gr], gp, r1);
            }
            dequant_part<ROPE>(pin(bA + dq_off), pin(bA + rope_off), r0);
            gather_part<ROPE>(p.pool, stand_in, slots[min(2, n_t - 1) * kTile + gr], gp, r0);
            dequant_part<ROPE>(pin(bB + dq_off), pin(bB + rope_off), r1);
            gather_part<ROPE>(p.pool, stand_in, slots[min(3, n_t - 1) * kTile + gr], gp, r1);
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
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    // O^T of this wavefront (256 dims x 32 heads) leaves through LDS, free
    // since the passes' last barrier: stored straight from the accumulators
    // every store instruction would touch 32 heads' rows 2 KB apart; from LDS
    // each one writes 1 KB of one head's row.  Wavefront w's region holds
    // [32 heads][256 dims + 4 pad] floats (the padding keeps the transposed
    // writes conflict-free).
    constexpr int kORow = 256 + 4;
    const uint32_t oreg = kb0 + wave * (32 * kORow * 4);
    static_assert(4 * 32 * kORow * 4 <= kSlotOff - 16, "output staging overlaps the slot list");
    {
        const uint32_t ow = pin(oreg + (l32 * kORow + 4 * g) * 4);
#pragma unroll
        for (int md = 0; md < 8; ++md)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                lds_st<floatx4_t>(ow + (32 * md + 8 * j) * 4,
                                  floatx4_t{o[md][4 * j], o[md][4 * j + 1], o[md][4 * j + 2], o[md][4 * j + 3]} * inv);
    }
    __syncthreads();
    {
        const uint32_t orr = pin(oreg + 16 * lane);
        const int64_t ob = (int64_t)split * p.out_split_stride + (int64_t)r * p.out_row_stride + 256 * half + 4 * lane;
        if (p.out_h) {                             // fp16 split partials (|o| <= 2688): half the bytes to store
#pragma unroll
            for (int h = 0; h < 32; ++h) {
                const floatx4_t v = lds_ld<floatx4_t>(orr + h * kORow * 4);
                if (hg * 32 + h < p.n_heads)
                    *reinterpret_cast<half4_t *>(p.out_h + ob + (int64_t)(hg * 32 + h) * kLatent) =
                        __builtin_convertvector(v, half4_t);
            }
        } else {
#pragma unroll
            for (int h = 0; h < 32; ++h) {
                const floatx4_t v = lds_ld<floatx4_t>(orr + h * kORow * 4);
                if (hg * 32 + h < p.n_heads)
                    *reinterpret_cast<floatx4_t *>(p.out + ob + (int64_t)(hg * 32 + h) * kLatent) = v;
            }
        }
    }
    if (head_live && half == 0 && g == 0 && p.lse) {
        const float lse = l_tot > 0.0f ? (m_fin + __builtin_log2f(l_tot)) * 0.69314718055994530942f : -__builtin_inff();
        p.lse[(int64_t)split * p.lse_split_stride + (int64_t)r * p.lse_row_stride + head] = lse;
    }
}

hipError_t launch_sparse_mla(const AttnParams &p, bool q_f32, int32_t n_splits, hipStream_t stream) {
    if (p.n_rows == 0) return hipSuccess;
    const dim3 grid((unsigned)p.n_rows, (unsigned)n_splits, (unsigned)((p.n_heads + 63) / 64));
    if (p.rope_dims == kRope) {
        if (q_f32) hipLaunchKernelGGL((sparse_mla_kernel<true, true>), grid, dim3(256), 0, stream, p);
        else hipLaunchKernelGGL((sparse_mla_kernel<false, true>), grid, dim3(256), 0, stream, p);
    } else {
        if (q_f32) hipLaunchKernelGGL((sparse_mla_kernel<true, false>), grid, dim3(256), 0, stream, p);
        else hipLaunchKernelGGL((sparse_mla_kernel<false, false>), grid, dim3(256), 0, stream, p);
    }
    return hipGetLastError();
}

// --------------------------------------------------- dequantizing gather

// One workgroup per (query row, tile of 32 entries): translate, then the same
// lane roles and decoding as the attention kernel, written row-major to HBM
// (576 fp16 values per entry, or 512 for rope-free rows).
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
    const bool rope = p.rope_dims == kRope;
    const int row_b = rope ? kRowBytes : kScaleOff + kLatent / 16, dim = rope ? kDim : kLatent;
    const int pp = tid & 15, qc = tid >> 4;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int row = 2 * pp + h, e = tile * kTile + row;
        if (e >= p.k) continue;
        const int32_t s = slots[row];
        u32x4_t codes = {0, 0, 0, 0};
        uint32_t sc = 0;
        if (s >= 0) {
            const uint8_t *src = p.pool + (int64_t)s * row_b;
            codes = *reinterpret_cast<const u32x4_t *>(src + 16 * qc);
            sc = *reinterpret_cast<const uint16_t *>(src + kScaleOff + 2 * qc);
        }
        uint32_t v[16];
        dequant_chunk(codes, sc, v);
        uint32_t *dst = reinterpret_cast<uint32_t *>(out + ((int64_t)r * p.k + e) * dim) + 16 * qc;
#pragma unroll
        for (int c = 0; c < 4; ++c)
            *reinterpret_cast<u32x4_t *>(dst + 4 * c) = u32x4_t{v[4 * c], v[4 * c + 1], v[4 * c + 2], v[4 * c + 3]};
    }
    if (rope && tid < 128) {
        const int row = tid >> 2, e = tile * kTile + row;
        if (e < p.k) {
            const int32_t s = slots[row];
            u32x4_t b = {0, 0, 0, 0};
            if (s >= 0) b = *reinterpret_cast<const u32x4_t *>(p.pool + (int64_t)s * kRowBytes + kRopeOff + 16 * (tid & 3));
            uint32_t h[8];
            dequant_rope16(b, h);
            uint32_t *dst = reinterpret_cast<uint32_t *>(out + ((int64_t)r * p.k + e) * dim) + kLatent / 2 + 8 * (tid & 3);
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

// One 128-thread workgroup per state t; a thread owns 4 dims per 512.  With
// at most kMergeBatch parts of at most 512 dims (decode's case), the parts' o
// are loaded before the weights are formed, so their round trip overlaps that
// of the lse.  With M the largest lse: w_s = exp(lse_s - M) (an empty part
// weighs 0), W = the w_s summed in part order, o = (the w_s o_s summed in part
// order) / W, lse = M + ln W; all parts empty gives o = 0, lse = -inf.
constexpr int kMergeBatch = 8;

// four consecutive dims of one part's o, widened to fp32 (exact) from fp16 parts
template <bool F16>
__device__ __forceinline__ floatx4_t load_part4(const MergeParams &p, int64_t off) {
    if constexpr (F16) return __builtin_convertvector(*reinterpret_cast<const half4_t *>(p.part_o_h + off), floatx4_t);
    else return *reinterpret_cast<const floatx4_t *>(p.part_o + off);
}

template <bool F16>
__global__ __launch_bounds__(128) void merge_states_kernel(MergeParams p) {
    __shared__ float w[64];
    __shared__ float stat[2];
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x;
    const int S = p.n_parts;
    const int64_t o_t = t * p.dim;                                // part s at s * n_states * dim
    const int64_t o_stride = p.n_states * (int64_t)p.dim;
    const bool early = S <= kMergeBatch && p.dim <= 512;          // uniform
    floatx4_t v[kMergeBatch];
    if (early && 4 * tid < p.dim) {
#pragma unroll
        for (int s = 0; s < kMergeBatch; ++s)
            if (s < S) v[s] = load_part4<F16>(p, o_t + s * o_stride + 4 * tid);
    }
    if (tid == 0) {
        float M = -__builtin_inff();
        for (int s = 0; s < S; ++s) M = __builtin_fmaxf(M, p.part_lse[(int64_t)s * p.n_states + t]);
        stat[0] = M;
    }
    __syncthreads();
    const float M = stat[0];
    if (M != -__builtin_inff() && tid < S) {
        const float ls = p.part_lse[(int64_t)tid * p.n_states + t];
        w[tid] = ls == -__builtin_inff() ? 0.0f : expf(ls - M);
    }
    __syncthreads();
    if (tid == 0) {
        float W = 0.0f;
        if (M != -__builtin_inff())
            for (int s = 0; s < S; ++s) W += w[s];
        stat[1] = W;
        if (p.lse) p.lse[t] = M == -__builtin_inff() ? M : M + logf(W);
    }
    __syncthreads();
    const float W = stat[1];
    const float inv = W > 0.0f ? 1.0f / W : 0.0f;
    float *orow = p.out + (t / p.states_per_row) * p.out_row_stride + (t % p.states_per_row) * p.out_col_stride;
    if (early) {
        if (4 * tid < p.dim) {
            floatx4_t acc = {0, 0, 0, 0};
            if (W > 0.0f) {
#pragma unroll
                for (int s = 0; s < kMergeBatch; ++s) {
                    if (s < S) {
                        const float ws = w[s];
                        if (ws != 0.0f) acc += ws * v[s];
                    }
                }
            }
            *reinterpret_cast<floatx4_t *>(orow + 4 * tid) = acc * inv;
        }
        return;
    }
    for (int d = 4 * tid; d < p.dim; d += 512) {
        floatx4_t acc = {0, 0, 0, 0};
        if (W > 0.0f)
            for (int s = 0; s < S; ++s) {
                const float ws = w[s];
                if (ws != 0.0f) acc += ws * load_part4<F16>(p, o_t + s * o_stride + d);
            }
        *reinterpret_cast<floatx4_t *>(orow + d) = acc * inv;
    }
}

hipError_t launch_merge_states(const MergeParams &p, hipStream_t stream) {
    if (p.n_states == 0) return hipSuccess;
    if (p.part_o_h) hipLaunchKernelGGL(merge_states_kernel<true>, dim3((unsigned)p.n_states), dim3(128), 0, stream, p);
    else hipLaunchKernelGGL(merge_states_kernel<false>, dim3((unsigned)p.n_states), dim3(128), 0, stream, p);
    return hipGetLastError();
}

}  // namespace kv4
