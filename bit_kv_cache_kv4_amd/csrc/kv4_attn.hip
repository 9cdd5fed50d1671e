// Sparse MLA attention over the 4-bit pool: decode (split-K) and prefill.
//
// README "60+ inference optimizations & kernels": section "4-bit KV cache"
// (the 4-bit rows are dequantized on chip, not into an FP8 scratch copy),
// section "AMD MI355X" (hand-written HIP sparse MLA decode whose K tile in LDS
// is also the P.V operand through a transposing LDS read; split-K decode),
// "Parallelism and disaggregation" (per-part (o, lse) and their merge).
// sgl-amd-mono GLM-5.3 PR, "Modifications": 64-token page table and its stride
// as launch arguments; one task serves many heads, so each key row is
// gathered once per task.
//
// Workgroup = 8 wavefronts, two per SIMD, for one task (query row r, split s,
// chunk of up to 64 heads), in two roles that run their own loops (so each
// wavefront's registers hold only its role's state) and meet at the same
// barriers: score wavefronts 0..3 (queries in registers, scores, softmax, P
// into LDS) and P.V wavefronts 4..7 (quarter dq of the 512 latent dims:
// O^T[128 dims x 64 heads] accumulated from V^T, read from the K tile itself
// through ds_read_b64_tr_b16, and the P of all 64 heads).  A SIMD holds one
// wavefront of each role, and the roles let each V^T and P element be read
// once per tile.  At the LDS rates measured on gfx950 (stores about 78 B/clk
// per CU, plain reads about 195, transposing reads about 92) the loops are
// bound by the roles' instruction chains and the shared matrix pipe rather
// than by LDS bandwidth.
//
// bf16 queries (sparse_mla_bf16_kernel): score wavefront = (head group hg =
// w % 2 of 32 heads, row half rh = w / 2 of each tile) holds its heads' queries
// over all dims and computes whole scores S^T[16 rows x 32 heads]
// (v_mfma_f32_16x16x32_f16), so no partial scores are swapped and a tile takes
// one barrier: scores and softmax of t + 1 beside the P.V of t, the score
// wavefronts dequantizing their share of t + 2 between their MFMAs and the
// P.V wavefronts theirs after their MFMAs.  fp32 queries (split into hi and lo
// fp16 parts: twice the registers, sparse_mla_f32q_kernel): score wavefront =
// (head group, half of the dims), partial scores S^T[32 rows x 32 heads]
// (v_mfma_f32_32x32x16_f16) swapped with the partner half through LDS so each
// owns 16 rows; two phases per tile (softmax of t and scores of t + 1, then
// the swap beside the P.V of t), the P.V wavefronts dequantizing whole rows.
//
// Gathering: the entries' pool slots (translated once per chunk of 2048
// entries, valid ones packed to the front, kept in LDS) name 32 rows; thread
// t loads row t % 32, part t / 32 (32 latent dims, their 2 block scales, 8
// rope dims) four tiles ahead of its use, and dequantizes with gfx950's
// FP4/FP8 -> fp16 conversions at scale 1 and one packed multiply by the E4M3
// block scale (every product is exact in fp16; the conversions' own scale
// operand applies only its power of two).  Three K tiles rotate.
// The softmax uses P = 2^(s - m_ref) with m_ref the head's largest score in
// the first tile (agreed across the wavefronts sharing the head); if a later
// score exceeds m_ref + 15 (P could overflow fp16) the workgroup runs the list
// again with m_ref = the exact maximum, which the first pass tracked.  The
// per-split result is written normalised with its lse; a split count of 1
// writes the final output.
//
// Rows are either the 352-byte format (576 dims: 512 latent + 64 rope) or the
// 288-byte rope-free format (512 latent dims; README, "4-bit KV cache": the
// rope-free row of GLM-5.3-Flash).
#include "kv4_attn.h"
#include "kv4_device.h"

#include <algorithm>
#include <type_traits>


namespace kv4 {

namespace {

constexpr int kThreads = 512;                          // 8 wavefronts: 4 score, 4 P.V
constexpr int kTile = 32;                              // list entries per tile
constexpr int kChunkB = 512;                           // one 8-dim chunk of a tile's 32 rows in fp16
constexpr int kKTileB = 72 * kChunkB;                  // 36864: a K tile of 576 dims
constexpr int kNBuf = 3;                               // K tiles in flight
constexpr int kXB = 2 * 2 * 64 * 32;                   // partial scores: [hg][receiving half][lane] x 32 B
constexpr int kPXHead = 80;                            // P of one head: 32 rows fp16 + 16 B pad
constexpr int kPXB = 64 * kPXHead;
constexpr int kSlotCap = 2048;                         // entries translated per chunk
constexpr int kPosPerLane = kSlotCap / kThreads;
// LDS: the small fixed areas first, at addresses below 64 KB that every LDS
// instruction reaches through its immediate offset (no address register held
// for them); then the K tiles and what shares their space; the slot list last.
constexpr int kOffCounts = 0;                          // per-wavefront counts of valid entries
constexpr int kOffRed = kOffCounts + kPosPerLane * 8 * 4;
constexpr int kOffRowSum = kOffRed + 2 * 2 * 32 * 4;
constexpr int kOffRowRef = kOffRowSum + 2 * 2 * 32 * 4;
constexpr int kOffFlag = kOffRowRef + 2 * 32 * 4;
constexpr int kOffK = 1536;                            // K tiles; offsets below are relative to it
static_assert(kOffFlag + 16 <= kOffK, "small areas overlap the K tiles");
constexpr int kOffX = kNBuf * kKTileB;                 // 110592
constexpr int kOffPX = kOffX + kXB;                    // 118784
constexpr int kStageBytes = 64 * (kDim * 4 + 16);      // 148480: all 64 fp32 query rows (K tiles, X, P and spare)
constexpr int kOffSlots = kOffK + kStageBytes;         // 150016 (absolute)
constexpr int kLdsBytes = kOffSlots + kSlotCap * 4;    // 158208
// the output staged for its coalesced store: 64 head rows of 512 fp32 (row
// stride 2064 bytes) or fp16 (1032 bytes) values; the strides put the 16- or
// 8-byte stores of 32 consecutive heads on distinct banks
constexpr int kORowF = kLatent * 4 + 16, kORowH = kLatent * 2 + 8;
static_assert(64 * kORowF <= kStageBytes, "output staging overlaps the slot list");
static_assert(kOffPX + kPXB <= kStageBytes, "P overlaps the slot list");
constexpr float kRefSlack = 15.0f;                     // log2 headroom of fp16 P above its reference

typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef unsigned short ushort2_t __attribute__((ext_vector_type(2)));

// K-tile layout: element (row r, chunk c of 8 dims) at c * 512 + 16 * (r ^ 4 (c & 3)),
// i.e. the 32 rows' copies of a 16-byte chunk are contiguous, their order
// permuted by the chunk index.  A score operand read and a dequantizing write
// (one chunk of 32 rows per 32 lanes) touch 512 contiguous bytes; a
// transposing read (4 rows x 4 consecutive chunks per 32 lanes) touches 16
// distinct 16-byte bank groups, because the XOR spreads the 4 chunks' copies of
// a row over the 4 row groups.  No access pattern has a bank conflict and no
// padding is needed.
__device__ __forceinline__ uint32_t kswz(int r, int c) { return c * kChunkB + 16 * (r ^ (4 * (c & 3))); }

__device__ __forceinline__ floatx16_t mfma32(half8_t a, half8_t b, floatx16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// LDS accesses by 32-bit byte address.
typedef __attribute__((address_space(3))) uint8_t lds_u8_t;
__device__ __forceinline__ uint32_t lds_addr(uint8_t *p) { return (uint32_t)(size_t)(lds_u8_t *)p; }
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

template <bool ROPE>
constexpr int row_bytes() { return ROPE ? kRowBytes : kScaleOff + kLatent / 16; }

// f(integral_constant<int, I>) for I = B .. E-1, each index known at compile time
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// ------------------------------------------------ translation of a list chunk
// Shared by the attention kernel and the gather test entry point, which must
// run the same code.  Thread t holds list entries c_lo + t + 512 i.

struct ListCtx {
    const int32_t *list;      // this query row's list
    const int32_t *pt_row;    // its page-table row; null without a page table or for a bad request
    bool bad_req;             // a page table is given but the row's request is outside it
};

__device__ __forceinline__ ListCtx list_ctx(const AttnParams &p, int r) {
    ListCtx c;
    const int32_t req = p.row_req ? p.row_req[r] : r;
    c.bad_req = p.page_table && (req < 0 || req >= p.pt_n_rows);
    c.pt_row = p.page_table && !c.bad_req ? p.page_table + (int64_t)req * p.pt_row_stride : nullptr;
    c.list = p.topk + (int64_t)r * p.topk_row_stride;
    return c;
}

__device__ __forceinline__ void load_positions(const ListCtx &c, int c_lo, int c_hi, int tid, int32_t (&pos)[kPosPerLane]) {
#pragma unroll
    for (int i = 0; i < kPosPerLane; ++i) {
        const int e = c_lo + tid + kThreads * i;
        pos[i] = e < c_hi ? c.list[e] : -1;
    }
}

__device__ __forceinline__ void load_pages(const AttnParams &p, const ListCtx &c, const int32_t (&pos)[kPosPerLane],
                                           int32_t (&phys)[kPosPerLane]) {
#pragma unroll
    for (int i = 0; i < kPosPerLane; ++i) {
        phys[i] = -1;
        if (c.pt_row && pos[i] >= 0 && (pos[i] >> p.page_shift) < p.pt_n_pages) phys[i] = c.pt_row[pos[i] >> p.page_shift];
    }
}

// Packs the valid entries' slots, in list order, to the front of slots[] and
// pads with -1 up to a whole number of tile pairs (64 entries, at least one
// pair, so the first two tiles' entries are defined even for an empty list);
// returns the number of valid entries (the same in every thread).  Holds a barrier, so every thread calls it; the caller
// synchronizes before slots[] is read.
__device__ __forceinline__ int pack_slots(const AttnParams &p, const ListCtx &c, const int32_t (&pos)[kPosPerLane],
                                          const int32_t (&phys)[kPosPerLane], int tid, int32_t *slots,
                                          int32_t *counts, uint32_t &err) {
    const int lane = tid & 63, w = tid >> 6;
    int32_t sl[kPosPerLane];
    uint64_t bal[kPosPerLane];
#pragma unroll
    for (int i = 0; i < kPosPerLane; ++i) {   // entry tid + 512 i: list order is (i, wavefront, lane)
        int64_t s = -1;
        if (c.bad_req) err |= pos[i] >= 0 ? kErrPage : 0u;
        else s = slot_of(pos[i], phys[i], c.pt_row != nullptr, p.pt_n_pages, p.page_shift, p.n_slots, err);
        sl[i] = (int32_t)s;                   // s < n_slots <= 2^31 - 1
        bal[i] = __ballot(s >= 0);
        if (lane == 0) counts[8 * i + w] = (int32_t)__popcll(bal[i]);
    }
    __syncthreads();
    int nv = 0, base[kPosPerLane];
#pragma unroll
    for (int i = 0; i < kPosPerLane; ++i) {
#pragma unroll
        for (int ww = 0; ww < 8; ++ww) {
            if (ww == w) base[i] = nv;
            nv += counts[8 * i + ww];
        }
    }
#pragma unroll
    for (int i = 0; i < kPosPerLane; ++i) {
        const int below = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal[i] >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((uint32_t)bal[i], 0u));
        if (sl[i] >= 0) slots[base[i] + below] = sl[i];
        const int e = tid + kThreads * i;
        if (e >= nv && e < max(2 * kTile, (nv + 2 * kTile - 1) & ~(2 * kTile - 1))) slots[e] = -1;
    }
    return nv;
}

// ------------------------------------------------ gather and dequantization
// Thread t takes row gr = t % 32 of a tile and part gp = t / 32: code bytes
// 16gp .. 16gp + 15 (latent dims 32gp .. 32gp + 31, K-tile chunks 4gp .. 4gp +
// 3), block scales 2gp and 2gp + 1 (from the aligned word of scales 4(gp/2) ..
// + 3), and (parts 0..7, the score wavefronts' threads, when WITH_ROPE) rope
// bytes 8gp .. 8gp + 7 (chunk 64 + gp).  A skipped
// entry (slot < 0) reads 352 readable bytes elsewhere (`stand_in`) and
// dequantizes to zeros: its scale and rope bytes become 0.  The loads take no
// branch, so the compiler can count them and wait for exactly the set it needs.

template <bool ROPE>
struct GSet {
    u32x4_t c;
    uint32_t sc;
    u32x2_t rp;
    bool valid;
};

template <bool ROPE, bool WITH_ROPE = ROPE>
__device__ __forceinline__ void gather_set(const uint8_t *__restrict__ pool, const uint8_t *stand_in, int32_t slot,
                                           int gp, GSet<ROPE> &G) {
    G.valid = slot >= 0;
    const uint8_t *row = pool + (int64_t)max(slot, 0) * row_bytes<ROPE>();
    row = G.valid ? row : stand_in;
    G.c = *reinterpret_cast<const u32x4_t *>(row + 16 * gp);
    G.sc = *reinterpret_cast<const uint32_t *>(row + kScaleOff + 4 * (gp >> 1));   // scales 4(gp/2) .. +3
    if constexpr (WITH_ROPE) G.rp = *reinterpret_cast<const u32x2_t *>(row + kRopeOff + 8 * (gp & 7));
    else G.rp = u32x2_t{0, 0};
}

// The dequantization in pieces, so a caller can spread them between its
// MFMAs: the part's two block scales (E4M3 -> fp16, exact; 0 for a skipped
// entry), one 8-dim chunk (the conversion at scale 1 is exact, and so is the
// product with the block scale), and the rope chunk.
template <bool ROPE>
__device__ __forceinline__ half2_t dq_scales(const GSet<ROPE> &G, int gp) {
    const uint32_t sc = G.valid ? G.sc >> (16 * (gp & 1)) : 0u;                     // this part's two scales
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sc, 1.0f, false);
}
// chunk 4gp + i: dims 32gp + 8i .. +7, block 2gp + i / 2
template <bool ROPE>
__device__ __forceinline__ void dq_chunk(uint32_t kb, int gr, int gp, int i, half2_t dd, const GSet<ROPE> &G) {
    const half2_t d = i < 2 ? __builtin_shufflevector(dd, dd, 0, 0) : __builtin_shufflevector(dd, dd, 1, 1);
    const uint32_t wv = G.c[i];
    u32x4_t v;
    v[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wv, 1.0f, 0) * d);
    v[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wv, 1.0f, 1) * d);
    v[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wv, 1.0f, 2) * d);
    v[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wv, 1.0f, 3) * d);
    lds_st<u32x4_t>(kb + kswz(gr, 4 * gp + i), v);
}
template <bool ROPE>
__device__ __forceinline__ void dq_rope(uint32_t kb, int gr, int gp, const GSet<ROPE> &G) {
    const u32x2_t rp = G.valid ? G.rp : u32x2_t{0, 0};
    u32x4_t h;
    h[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(rp[0], 1.0f, false));
    h[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(rp[0], 1.0f, true));
    h[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(rp[1], 1.0f, false));
    h[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(rp[1], 1.0f, true));
    lds_st<u32x4_t>(kb + kswz(gr, 64 + gp), h);
}

// rope_part: this wavefront stores the rope chunk (wave-uniform: wavefronts 0..3)
template <bool ROPE>
__device__ __forceinline__ void dequant_set(uint32_t kb, int gr, int gp, bool rope_part, const GSet<ROPE> &G) {
    const half2_t dd = dq_scales<ROPE>(G, gp);
#pragma unroll
    for (int i = 0; i < 4; ++i) dq_chunk<ROPE>(kb, gr, gp, i, dd, G);
    if constexpr (ROPE) {
        if (rope_part) dq_rope<ROPE>(kb, gr, gp, G);
    }
}

}  // namespace

template <bool ROPE>
__global__ __launch_bounds__(kThreads) void sparse_mla_f32q_kernel(AttnParams p) {
    // K has kD dims (latent + rope, or latent only); a score wavefront's half
    // of them is kHd dims = kKs MFMA k-steps of 16 = kHc chunks of 8
    constexpr int kD = ROPE ? kDim : kLatent;
    constexpr int kHd = kD / 2;
    constexpr int kKs = kHd / 16;
    constexpr int kHc = kHd / 8;
    constexpr int kAhead = 2;                  // score operands read ahead of their MFMA
    constexpr int kTrAhead = 4;                // P.V operand pairs read ahead
    __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
    int32_t *slots = reinterpret_cast<int32_t *>(lds + kOffSlots);
    int32_t *counts = reinterpret_cast<int32_t *>(lds + kOffCounts);
    float *red = reinterpret_cast<float *>(lds + kOffRed);
    float *row_sum = reinterpret_cast<float *>(lds + kOffRowSum);   // [head group][half][head]: the halves' l
    float *row_ref = reinterpret_cast<float *>(lds + kOffRowRef);   // [head group][head]: the reference m_ref
    int32_t *flag = reinterpret_cast<int32_t *>(lds + kOffFlag);
    const uint32_t L = lds_addr(lds) + kOffK;      // base of the K tiles and the areas sharing their space

    // wavefront-uniform values live in scalar registers, so the branches on
    // them are scalar and no lane mask is ever saved and restored
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, g = lane >> 5;
    const int gr = tid & 31, gp = tid >> 5;
    const int r = blockIdx.x, split = blockIdx.y, h0 = blockIdx.z * 64;

    const int n_tiles = (p.k + kTile - 1) / kTile;
    const int t_lo = split * p.tiles_per_split;
    const int t_hi = min(n_tiles, t_lo + p.tiles_per_split);
    const int e_lo = t_lo * kTile;
    const int e_hi = min(p.k, t_hi * kTile);

    const ListCtx lc = list_ctx(p, r);
    const uint8_t *stand_in = reinterpret_cast<const uint8_t *>(p.q);
    uint32_t err = 0;

    // ---- Prologue.  Three dependent round trips (list entries, page-table
    // entries, the first rows) come before the first tile.  The list goes out
    // first, then this row's queries (coalesced: consecutive threads take
    // consecutive 16-byte chunks of a head's row; 147 KB), then the page-table
    // entries once the list is back; while those are in flight the queries are
    // converted and staged in LDS (rows padded so the fragment reads are
    // conflict-free), and the slot packing's barrier orders them before their
    // readers.  All 64 head rows are staged at once; they fill most of the LDS
    // (the slot list lies beyond), and a barrier separates their last read
    // from the first K-tile store.
    constexpr int kQE = 4;                                 // bytes per query element
    constexpr int kQRow = kD * kQE + 16;                   // staged head row
    constexpr int kQH = 64;                                // heads staged
    const uint32_t Lq = L;                                 // staging base
    constexpr int kQChunks = kD * kQE / 16;                // 16-byte chunks per head row
    constexpr int kQPer = kQH * kQChunks / kThreads;       // chunks per thread
    static_assert(kQH * kQChunks % kThreads == 0, "query chunks do not divide");
    static_assert(kQH * kQRow <= kStageBytes, "staged queries overlap the slot list");
    // thread t loads head t / kTPH, 16-byte chunks t % kTPH +
    // kTPH i: one base address per thread, consecutive threads on consecutive
    // chunks of a head row
    constexpr int kTPH = kThreads / kQH;                   // threads per head row
    static_assert(kQChunks == kTPH * kQPer, "query chunks do not divide");
    const uint8_t *qr = reinterpret_cast<const uint8_t *>(p.q) + (int64_t)r * p.q_row_stride * kQE;
    const int q_hh = tid / kTPH, q_part = tid % kTPH;
    auto load_q = [&](u32x4_t (&qc)[kQPer]) {   // heads past the last re-read the last one (zeroed when staged)
        const uint8_t *src = qr + (int64_t)min(h0 + q_hh, p.n_heads - 1) * p.q_head_stride * kQE + 16 * q_part;
#pragma unroll
        for (int i = 0; i < kQPer; ++i) qc[i] = *reinterpret_cast<const u32x4_t *>(src + 16 * kTPH * i);
    };
    // The queries as the score MFMAs take them, made by every thread from the
    // 72 values it loaded (chunk q_part + 8 i holds dims 4 (q_part + 8 i) ..
    // +3; chunks i < kHalfI lie in the first half of the dims): per head and
    // half, the head's 8 threads (consecutive lanes) agree on the largest |q|,
    // whose power-of-two scale qs puts it in [2^13, 2^14); each q qs becomes a
    // hi and a lo fp16 part, hi at byte 2d of the head's staging row and lo at
    // 2 kD + 2d, and qs goes to q_scale[2 head + half].  Wavefronts whose heads
    // are all past the last only store zeros.
    constexpr int kHalfI = kHd / (4 * kTPH);
    static_assert(kHd % (4 * kTPH) == 0, "a thread's chunks do not split at the half");
    float *q_scale = red;                          // [head][half]; red is next written after the first tile
    auto stage_q = [&](const u32x4_t (&qc)[kQPer]) {
        const uint32_t dst = Lq + q_hh * kQRow + 8 * q_part;
        if (__builtin_amdgcn_readfirstlane(h0 + 8 * w) >= p.n_heads) {   // the wavefront's 8 heads are all dead
#pragma unroll
            for (int i = 0; i < kQPer; ++i) {
                lds_st<u32x2_t>(dst + 8 * kTPH * i, u32x2_t{0, 0});
                lds_st<u32x2_t>(dst + 2 * kD + 8 * kTPH * i, u32x2_t{0, 0});
            }
            if (q_part == 0) q_scale[2 * q_hh] = q_scale[2 * q_hh + 1] = 1.0f;
            return;
        }
        const bool live = h0 + q_hh < p.n_heads;
        float m[2] = {0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < kQPer; ++i) {
            const floatx4_t v = __builtin_bit_cast(floatx4_t, qc[i]);
            m[i >= kHalfI] = __builtin_fmaxf(m[i >= kHalfI],
                                             __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(v[0]), __builtin_fabsf(v[1])),
                                                             __builtin_fmaxf(__builtin_fabsf(v[2]), __builtin_fabsf(v[3]))));
        }
        float qs[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            float mm = live ? m[h] : 0.0f;
            mm = __builtin_fmaxf(mm, __shfl_xor(mm, 1));
            mm = __builtin_fmaxf(mm, __shfl_xor(mm, 2));
            mm = __builtin_fmaxf(mm, __shfl_xor(mm, 4));
            int ex = 0;
            if (mm > 0.0f) (void)__builtin_frexpf(mm, &ex);
            qs[h] = __builtin_ldexpf(1.0f, 14 - ex);     // the largest |q| times qs < 2^14
        }
        if (q_part == 0) {
            q_scale[2 * q_hh] = qs[0];
            q_scale[2 * q_hh + 1] = qs[1];
        }
#pragma unroll
        for (int i = 0; i < kQPer; ++i) {
            const floatx4_t v = __builtin_bit_cast(floatx4_t, qc[i]);
            half4_t hi, lo;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float x = live ? v[e] * qs[i >= kHalfI] : 0.0f;
                hi[e] = (_Float16)x;
                lo[e] = (_Float16)(x - (float)hi[e]);
            }
            lds_st<half4_t>(dst + 8 * kTPH * i, hi);
            lds_st<half4_t>(dst + 2 * kD + 8 * kTPH * i, lo);
        }
    };

    int32_t pos[kPosPerLane], phys[kPosPerLane];
    const int first_hi = min(e_hi, e_lo + kSlotCap);
    load_positions(lc, e_lo, e_lo < e_hi ? first_hi : e_lo, tid, pos);
    u32x4_t qc[kQPer];
    // the rows (147 KB) are staged before the roles split: their 72 registers
    // per thread must not stay live into the roles
    load_q(qc);
    load_pages(p, lc, pos, phys);
    stage_q(qc);
    int nv = __builtin_amdgcn_readfirstlane(pack_slots(p, lc, pos, phys, tid, slots, counts, err));
    if (tid == 0) *flag = 0;
    __syncthreads();                               // slots[] complete, queries staged

    const uint32_t K0 = L, K1 = L + kKTileB, K2 = L + 2 * kKTileB;
    int n_t = 0, n_real = 0, last_rows = kTile;   // tiles (even), tiles holding entries, rows of the last
    bool have_ref = false;                         // uniform: the softmax reference is set
    // the chunk's tile counts after its slots are packed (the same in every thread)
    auto chunk_tiles = [&]() {
        n_real = (nv + kTile - 1) / kTile;
        n_t = (n_real + 1) & ~1;
        last_rows = nv - kTile * (n_real - 1);
    };
    // rows of tile t below this are entries, the rest padding
    auto tile_lim = [&](int t) { return t < n_real - 1 ? kTile : t == n_real - 1 ? last_rows : 0; };
    // a fresh chunk: translate and pack its slots (every thread, three barriers)
    auto fresh_chunk = [&](int c_lo, int c_hi) {
        __syncthreads();                           // slots of the previous chunk are no longer read
        load_positions(lc, c_lo, c_hi, tid, pos);
        load_pages(p, lc, pos, phys);
        nv = __builtin_amdgcn_readfirstlane(pack_slots(p, lc, pos, phys, tid, slots, counts, err));
        __syncthreads();
    };
    // the output of this task's live heads from its staging rows: 16-byte
    // (fp32) or 8-byte (fp16) pieces, consecutive threads on consecutive
    // pieces of a head row; the head of piece i is the same in a wavefront
    auto store_out = [&]() {
        const int n_live = min(64, p.n_heads - h0);
        const int64_t base = (int64_t)split * p.out_split_stride + (int64_t)r * p.out_row_stride + (int64_t)h0 * kLatent;
        const int pc = tid & 127;
        if (p.out_h) {
            _Float16 *ob = p.out_h + base;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int hh = 4 * i + (tid >> 7);
                if (hh < n_live)
                    *reinterpret_cast<half4_t *>(ob + (hh * kLatent + 4 * pc)) = lds_ld<half4_t>(L + hh * kORowH + 8 * pc);
            }
        } else {
            float *ob = p.out + base;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int hh = 8 * i + (tid >> 6);
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int pj = 64 * j + (tid & 63);
                    if (hh < n_live)   // the final fp32 output, non-temporal (prefill 1% faster)
                        __builtin_nontemporal_store(lds_ld<floatx4_t>(L + hh * kORowF + 16 * pj),
                                                    reinterpret_cast<floatx4_t *>(ob + (hh * kLatent + 4 * pj)));
                }
            }
        }
    };

    if (w < 4) {
        // ================================================ score wavefronts
        const int hg = w & 1, half = w >> 1;
        // (the queries' registers leave no room for gathers here: the P.V
        // wavefronts gather and dequantize whole rows)

        // queries: B operand of S^T = K Q^T.  Lane (l32, g) holds head h0 +
        // 32hg + l32, dims kHd half + 16 ks + 8 g .. +7 for ks < kKs, as
        // staged: a hi and a lo fp16 part (two MFMAs per k-step) at the scale
        // of the head's half.  Each half's partial scores are multiplied by
        // score_mul = sm_scale log2(e) / qs before the two halves are added,
        // so no exchange between them is needed here.
        half8_t qb[kKs];
        half8_t ql[kKs];
        float score_mul;
        {
            const uint32_t qrow = Lq + (32 * hg + l32) * kQRow + 2 * (kHd * half + 8 * g);
#pragma unroll
            for (int ks = 0; ks < kKs; ++ks) {
                qb[ks] = lds_ld<half8_t>(qrow + 32 * ks);
                ql[ks] = lds_ld<half8_t>(qrow + 2 * kD + 32 * ks);
            }
            score_mul = p.score_mul / q_scale[2 * (32 * hg + l32) + half];
            __syncthreads();                   // the first K tiles overwrite the staged queries
        }

        // score operand (A of S^T = K Q^T): row l32, chunk kHc half + 2 ks + g;
        // even and odd k-steps differ in the row permutation (kHc is a
        // multiple of 4)
        const uint32_t sc_off0 = (kHc * half + g) * kChunkB + 16 * (l32 ^ (4 * g));
        const uint32_t sc_off1 = (kHc * half + g) * kChunkB + 16 * (l32 ^ (4 * (g + 2)));
        // partial scores for the partner's rows go to X[hg][1 - half], ours
        // come from X[hg][half] (32 bytes per lane)
        const uint32_t x_w = L + kOffX + ((hg * 2 + 1 - half) * 64 + lane) * 32;
        const uint32_t x_r = L + kOffX + ((hg * 2 + half) * 64 + lane) * 32;
        // P of this lane's head, rows 16 half + 8 (v / 4) + 4 g + v % 4 for v <
        // 8, stored in the order that puts the B operand of P.V k-step kk
        // (rows 16kk + 4g + 0..3, 16kk + 8 + 4g + 0..3) in 16 contiguous bytes
        // (row bits 2 and 3 swapped): here 16 bytes at 16 half + 8 g
        const uint32_t px_w = L + kOffPX + (32 * hg + l32) * kPXHead + 2 * (16 * half + 8 * g);

        float m_ref = -__builtin_inff();   // reference of P = 2^(s - m_ref) for this lane's head
        float m_max = -__builtin_inff();   // largest score this lane has seen
        float l_run = 0.0f;                // sum of this lane's fp16 P
        bool need_redo = false;
        floatx4_t own0 = {0, 0, 0, 0}, own1 = {0, 0, 0, 0};   // this half's partial of its own 16 rows
        floatx16_t sacc;

        // partial S^T of the K tile at kb over this half's dims; the operand
        // reads go out kAhead MFMAs ahead
        auto scores = [&](uint32_t kb) {
            const uint32_t a0 = kb + sc_off0, a1 = kb + sc_off1;
            half8_t a[kAhead];
#pragma unroll
            for (int i = 0; i < kAhead; ++i) a[i] = lds_ld<half8_t>((i & 1 ? a1 : a0) + 2 * kChunkB * i);
            __builtin_amdgcn_sched_barrier(0);     // keep the reads ahead of their MFMAs
            floatx16_t acc = {};
#pragma unroll
            for (int ks = 0; ks < kKs; ++ks) {
                const half8_t cur = a[ks % kAhead];
                acc = mfma32(cur, qb[ks], acc);
                acc = mfma32(cur, ql[ks], acc);
                if (ks + kAhead < kKs) {
                    const int n = ks + kAhead;
                    a[ks % kAhead] = lds_ld<half8_t>((n & 1 ? a1 : a0) + 2 * kChunkB * n);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            sacc = acc;
        };
        // the partner's 16 rows to it, ours kept, both in log2 units (times
        // this half's score_mul; half is scalar: no lane mask)
        auto exchange = [&]() {
            const float sm = score_mul;
            if (half == 0) {
                lds_st<floatx4_t>(x_w, floatx4_t{sacc[8], sacc[9], sacc[10], sacc[11]} * sm);
                lds_st<floatx4_t>(x_w + 16, floatx4_t{sacc[12], sacc[13], sacc[14], sacc[15]} * sm);
                own0 = floatx4_t{sacc[0], sacc[1], sacc[2], sacc[3]} * sm;
                own1 = floatx4_t{sacc[4], sacc[5], sacc[6], sacc[7]} * sm;
            } else {
                lds_st<floatx4_t>(x_w, floatx4_t{sacc[0], sacc[1], sacc[2], sacc[3]} * sm);
                lds_st<floatx4_t>(x_w + 16, floatx4_t{sacc[4], sacc[5], sacc[6], sacc[7]} * sm);
                own0 = floatx4_t{sacc[8], sacc[9], sacc[10], sacc[11]} * sm;
                own1 = floatx4_t{sacc[12], sacc[13], sacc[14], sacc[15]} * sm;
            }
        };
        // scores of this lane's rows 16 half + 8 (v / 4) + 4 g + v % 4: our
        // half's partial plus the partner's
        auto row_raw = [&](floatx4_t x0, floatx4_t x1, float (&raw)[8]) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                raw[j] = own0[j] + x0[j];
                raw[4 + j] = own1[j] + x1[j];
            }
        };
        auto row_of = [&](int v) { return 16 * half + 8 * (v >> 2) + 4 * g + (v & 3); };
        // P = 2^(s - m_ref) of this lane's rows to LDS; rows >= lim are padding
        // (lim < 32 only on the chunk's last two tiles)
        auto softmax = [&](int lim, floatx4_t x0, floatx4_t x1) {
            float raw[8], e[8];
            row_raw(x0, x1, raw);
#pragma unroll
            for (int v = 0; v < 8; ++v) e[v] = raw[v] - m_ref;
            if (lim < kTile) {                     // scalar
#pragma unroll
                for (int v = 0; v < 8; ++v)
                    if (row_of(v) >= lim) e[v] = -__builtin_inff();
            }
            const float emax = __builtin_fmaxf(__builtin_fmaxf(__builtin_fmaxf(e[0], e[1]), __builtin_fmaxf(e[2], e[3])),
                                               __builtin_fmaxf(__builtin_fmaxf(e[4], e[5]), __builtin_fmaxf(e[6], e[7])));
            m_max = __builtin_fmaxf(m_max, emax + m_ref);
            need_redo |= emax > kRefSlack;         // P could overflow fp16
            half8_t ph;
#pragma unroll
            for (int v = 0; v < 8; ++v) ph[v] = (_Float16)__builtin_amdgcn_exp2f(e[v]);   // exp2(-inf) = 0
            const half2_t one2 = {(_Float16)1.0f, (_Float16)1.0f};
            float ls0 = __builtin_amdgcn_fdot2(half2_t{ph[0], ph[1]}, one2, 0.0f, false);
            float ls1 = __builtin_amdgcn_fdot2(half2_t{ph[4], ph[5]}, one2, 0.0f, false);
            ls0 = __builtin_amdgcn_fdot2(half2_t{ph[2], ph[3]}, one2, ls0, false);
            ls1 = __builtin_amdgcn_fdot2(half2_t{ph[6], ph[7]}, one2, ls1, false);
            l_run += ls0 + ls1;
            lds_st<half8_t>(px_w, ph);
        };
        // Phase 1 of a tile, laid out by hand: the MFMAs of the scores of t + 1
        // (one per slot, operands read kAhead slots ahead) with the softmax of
        // t spread between them, so the in-order wavefront issues its VALU work
        // while the MFMA chain runs instead of after it.
        auto scores_softmax = [&](uint32_t kb, int lim) {
            const floatx4_t x0 = lds_ld<floatx4_t>(x_r), x1 = lds_ld<floatx4_t>(x_r + 16);
            const uint32_t a0 = kb + sc_off0, a1 = kb + sc_off1;
            half8_t a[kAhead];
#pragma unroll
            for (int i = 0; i < kAhead; ++i) a[i] = lds_ld<half8_t>((i & 1 ? a1 : a0) + 2 * kChunkB * i);
            __builtin_amdgcn_sched_barrier(0);
            floatx16_t acc = {};
            float raw[8], e[8], emax = 0.0f, ls0 = 0.0f, ls1 = 0.0f;
            half8_t ph;
            const half2_t one2 = {(_Float16)1.0f, (_Float16)1.0f};
            static_for<0, kKs>([&](auto slot) {
                constexpr int ks = decltype(slot)::value;
                const half8_t cur = a[ks % kAhead];
                acc = mfma32(cur, qb[ks], acc);
                acc = mfma32(cur, ql[ks], acc);
                if constexpr (ks + kAhead < kKs)
                    a[ks % kAhead] = lds_ld<half8_t>(((ks + kAhead) & 1 ? a1 : a0) + 2 * kChunkB * (ks + kAhead));
                if constexpr (ks == 2)
#pragma unroll
                    for (int j = 0; j < 4; ++j) raw[j] = own0[j] + x0[j];
                if constexpr (ks == 3)
#pragma unroll
                    for (int j = 0; j < 4; ++j) raw[4 + j] = own1[j] + x1[j];
                if constexpr (ks == 4)
#pragma unroll
                    for (int v = 0; v < 4; ++v) e[v] = raw[v] - m_ref;
                if constexpr (ks == 5)
#pragma unroll
                    for (int v = 4; v < 8; ++v) e[v] = raw[v] - m_ref;
                if constexpr (ks == 6) {
                    if (lim < kTile) {             // scalar: the chunk's last two tiles only
#pragma unroll
                        for (int v = 0; v < 8; ++v)
                            if (row_of(v) >= lim) e[v] = -__builtin_inff();
                    }
                }
                if constexpr (ks == 7)
                    emax = __builtin_fmaxf(__builtin_fmaxf(__builtin_fmaxf(e[0], e[1]), __builtin_fmaxf(e[2], e[3])),
                                           __builtin_fmaxf(__builtin_fmaxf(e[4], e[5]), __builtin_fmaxf(e[6], e[7])));
                if constexpr (ks == 8) {
                    m_max = __builtin_fmaxf(m_max, emax + m_ref);
                    need_redo |= emax > kRefSlack;     // P could overflow fp16
                }
                if constexpr (ks >= 9 && ks < 13)
#pragma unroll
                    for (int v = 2 * (ks - 9); v < 2 * (ks - 9) + 2; ++v) e[v] = __builtin_amdgcn_exp2f(e[v]);
                if constexpr (ks == 13) {
#pragma unroll
                    for (int v = 0; v < 8; ++v) ph[v] = (_Float16)e[v];   // exp2(-inf) = 0
                }
                if constexpr (ks == 14) {
                    ls0 = __builtin_amdgcn_fdot2(half2_t{ph[0], ph[1]}, one2, 0.0f, false);
                    ls1 = __builtin_amdgcn_fdot2(half2_t{ph[4], ph[5]}, one2, 0.0f, false);
                    ls0 = __builtin_amdgcn_fdot2(half2_t{ph[2], ph[3]}, one2, ls0, false);
                    ls1 = __builtin_amdgcn_fdot2(half2_t{ph[6], ph[7]}, one2, ls1, false);
                }
                if constexpr (ks == 15) {
                    l_run += ls0 + ls1;
                    lds_st<half8_t>(px_w, ph);
                }
                __builtin_amdgcn_sched_barrier(0);
            });
            sacc = acc;
        };
        // phase 1: softmax of t, scores of t + 1; phase 2: the swap of t + 1's
        // partials (the P.V wavefronts dequantize and gather whole rows)
        auto iteration = [&](int t, uint32_t bB) {
            if (t + 1 < n_t) scores_softmax(bB, tile_lim(t));
            else softmax(tile_lim(t), lds_ld<floatx4_t>(x_r), lds_ld<floatx4_t>(x_r + 16));
            __syncthreads();
            if (t + 1 < n_t) exchange();
            __syncthreads();
        };

        for (int pass = 0; pass < 2; ++pass) {
            l_run = 0.0f;
            for (int c_lo = e_lo; c_lo < e_hi; c_lo += kSlotCap) {
                const int c_hi = min(e_hi, c_lo + kSlotCap);
                if (c_lo != e_lo || (pass == 1 && e_hi - e_lo > kSlotCap)) fresh_chunk(c_lo, c_hi);
                chunk_tiles();
                if (n_real == 0) continue;         // nothing valid in this chunk (uniform)
                __syncthreads();                   // tiles 0 and 1 in LDS
                scores(K0);
                exchange();
                __syncthreads();
                if (!have_ref) {                   // first tile with entries: agree on each head's reference
                    float raw[8];
                    row_raw(lds_ld<floatx4_t>(x_r), lds_ld<floatx4_t>(x_r + 16), raw);
                    float tmax = -__builtin_inff();
                    const int lim = tile_lim(0);
#pragma unroll
                    for (int v = 0; v < 8; ++v)
                        if (row_of(v) < lim) tmax = __builtin_fmaxf(tmax, raw[v]);
                    tmax = __builtin_fmaxf(tmax, __shfl_xor(tmax, 32));
                    if (g == 0) red[(hg * 2 + half) * 32 + l32] = tmax;
                    __syncthreads();
                    m_ref = __builtin_fmaxf(red[(hg * 2) * 32 + l32], red[(hg * 2 + 1) * 32 + l32]);
                    have_ref = true;
                }
                uint32_t bA = K0, bB = K1, bC = K2;
                for (int t = 0; t < n_t; t += 2) {
                    iteration(t, bB);
                    iteration(t + 1, bC);
                    const uint32_t a0 = bA;        // tiles t + 2, t + 3, t + 4 go to bC, bA, bB
                    bA = bC;
                    bC = bB;
                    bB = a0;
                }
            }
            if (need_redo) *flag = 1;
            {   // this pass's row sums and reference (the final ones unless a second pass follows)
                const float l2 = l_run + __shfl_xor(l_run, 32);
                if (g == 0) row_sum[(hg * 2 + half) * 32 + l32] = l2;
                if (g == 0 && half == 0) row_ref[hg * 32 + l32] = have_ref ? m_ref : 0.0f;
            }
            __syncthreads();
            if (pass == 1 || *flag == 0) break;    // uniform: read after the barrier
            // second pass: the exact maximum of every head as its reference
            const float mm = __builtin_fmaxf(m_max, __shfl_xor(m_max, 32));
            if (g == 0) red[(hg * 2 + half) * 32 + l32] = mm;
            __syncthreads();
            m_ref = __builtin_fmaxf(red[(hg * 2) * 32 + l32], red[(hg * 2 + 1) * 32 + l32]);
        }

        if (err && p.err_word) atomicOr(p.err_word, err);
        __syncthreads();                           // the P.V wavefronts have staged the output
        store_out();
    } else {
        // ================================================ P.V wavefronts
        const int dq = w - 4;
        // parts 8..15 of a tile's rows, no rope (unit 0), and parts 0..7 with
        // the rope (unit 1)
        constexpr int kUnits = 2;
        GSet<ROPE> G0[kUnits], G1[kUnits];
        auto gather_units = [&](int tile, GSet<ROPE> (&G)[kUnits]) {
            const int32_t slot = slots[tile * kTile + gr];
            gather_set<ROPE, false>(p.pool, stand_in, slot, gp, G[0]);
            if constexpr (kUnits == 2) gather_set<ROPE>(p.pool, stand_in, slot, gp - 8, G[1]);
        };
        auto dequant_units = [&](uint32_t kb, const GSet<ROPE> (&G)[kUnits]) {
            dequant_set<ROPE>(kb, gr, gp, false, G[0]);
            if constexpr (kUnits == 2) dequant_set<ROPE>(kb, gr, gp - 8, true, G[1]);
        };
        if (nv > 0) {
            gather_units(0, G0);
            gather_units(1, G1);
        }
        __syncthreads();                           // the score wavefronts have read the staged queries
        // transposing reads (A of O^T = V^T P^T): this lane names row j4 + 4g
        // (+8 for the second read of a k-step, +16 for the second k-step), 8
        // bytes at latent dims 128 dq + 32 md + 8 cc + 4 (lane & 1) .. +3, so
        // each lane receives a column of a row-major 4 x 16 block
        const int cc = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1), j4 = (lane >> 2) & 3;
        const uint32_t tr_off0 = (16 * dq + cc) * kChunkB + 16 * (j4 + 4 * (g ^ (cc & 1)) + 8 * (cc >> 1)) + 8 * (lane & 1);
        const uint32_t tr_off1 = (16 * dq + cc) * kChunkB + 16 * (j4 + 4 * (g ^ (cc & 1)) + 8 * (1 ^ (cc >> 1))) + 8 * (lane & 1);
        // B operand of k-step kk for heads 32 hb .. +31: head l32, P rows at 16kk + 8g
        const uint32_t px_r = L + kOffPX + l32 * kPXHead + 2 * (8 * g);
        floatx16_t o[4][2];                        // [dims block md][head block hb]

        // O^T += V^T P^T for the K tile at kb, both head blocks sharing each V^T
        // operand; the transposing reads go out kTrAhead MFMA pairs ahead
        auto pv = [&](uint32_t kb) {
            const uint32_t t0 = kb + tr_off0, t1 = kb + tr_off1;
            half8_t pb[2][2];
#pragma unroll
            for (int hb = 0; hb < 2; ++hb)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) pb[hb][kk] = lds_ld<half8_t>(px_r + hb * (32 * kPXHead) + 32 * kk);
            short4_t lo[kTrAhead], hi[kTrAhead];
            auto issue = [&](int j) {              // pair j: k-step kk = j / 4, dims block md = j % 4
                const int md = j & 3, kk = j >> 2;
                lo[j % kTrAhead] = lds_read_tr16(t0 + 4 * kChunkB * md + 256 * kk);
                hi[j % kTrAhead] = lds_read_tr16(t1 + 4 * kChunkB * md + 256 * kk);
            };
#pragma unroll
            for (int j = 0; j < kTrAhead; ++j) issue(j);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int md = j & 3, kk = j >> 2;
                const half8_t a = __builtin_bit_cast(
                    half8_t, __builtin_shufflevector(lo[j % kTrAhead], hi[j % kTrAhead], 0, 1, 2, 3, 4, 5, 6, 7));
                o[md][0] = mfma32(a, pb[0][kk], o[md][0]);
                o[md][1] = mfma32(a, pb[1][kk], o[md][1]);
                if (j + kTrAhead < 8) issue(j + kTrAhead);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        // phase 1: dequantization of t + 2 (latent dims 256..511) and the
        // gather of t + 4; phase 2: P.V of t
        auto iteration = [&](int t, GSet<ROPE> (&G)[kUnits], uint32_t bA, uint32_t bC) {
            if (t + 2 < n_t) dequant_units(bC, G);
            gather_units(min(t + 4, n_t - 1), G);
            __syncthreads();
            pv(bA);
            __syncthreads();
        };

        for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
            for (int md = 0; md < 4; ++md) o[md][0] = o[md][1] = floatx16_t{};
            for (int c_lo = e_lo; c_lo < e_hi; c_lo += kSlotCap) {
                const int c_hi = min(e_hi, c_lo + kSlotCap);
                if (c_lo != e_lo || (pass == 1 && e_hi - e_lo > kSlotCap)) fresh_chunk(c_lo, c_hi);
                chunk_tiles();
                if (n_real == 0) continue;
                if (pass == 1 || c_lo != e_lo) {
                    gather_units(0, G0);
                    gather_units(1, G1);
                }
                dequant_units(K0, G0);
                gather_units(min(2, n_t - 1), G0);
                dequant_units(K1, G1);
                gather_units(min(3, n_t - 1), G1);
                __syncthreads();                   // tiles 0 and 1 in LDS
                __syncthreads();                   // the score wavefronts' tile-0 partials are swapped
                if (!have_ref) {
                    __syncthreads();               // the reference is agreed
                    have_ref = true;
                }
                uint32_t bA = K0, bB = K1, bC = K2;
                for (int t = 0; t < n_t; t += 2) {
                    iteration(t, G0, bA, bC);
                    iteration(t + 1, G1, bB, bA);
                    const uint32_t a0 = bA;
                    bA = bC;
                    bC = bB;
                    bB = a0;
                }
            }
            __syncthreads();
            if (pass == 1 || *flag == 0) break;
            __syncthreads();                       // the second pass's reference is agreed
        }

        if (err && p.err_word) atomicOr(p.err_word, err);
        // O = O_acc / l (the row sums were written before the passes' last
        // barrier) staged for the coalesced store: lane (l32, g) of o[md][hb]
        // holds head 32 hb + l32, dims 128 dq + 32 md + 8 vq + 4 g .. +3 in
        // registers 4 vq .. 4 vq + 3
        auto stage = [&](auto half_out) {
            constexpr bool kH = decltype(half_out)::value;
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
                const float l_tot = row_sum[(hb * 2) * 32 + l32] + row_sum[(hb * 2 + 1) * 32 + l32];
                const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
                const uint32_t row = L + (32 * hb + l32) * (kH ? kORowH : kORowF);
#pragma unroll
                for (int md = 0; md < 4; ++md)
#pragma unroll
                    for (int vq = 0; vq < 4; ++vq) {
                        const int dim = 128 * dq + 32 * md + 8 * vq + 4 * g;
                        const floatx4_t v = floatx4_t{o[md][hb][4 * vq], o[md][hb][4 * vq + 1], o[md][hb][4 * vq + 2],
                                                      o[md][hb][4 * vq + 3]} * inv;
                        if constexpr (kH) lds_st<half4_t>(row + 2 * dim, __builtin_convertvector(v, half4_t));
                        else lds_st<floatx4_t>(row + 4 * dim, v);
                    }
            }
        };
        if (p.out_h) stage(std::true_type{});
        else stage(std::false_type{});
        if (dq == 0 && g == 0 && p.lse) {          // lse = ln(l) + m_ref ln 2 of heads 32 hb + l32
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
                const int head = h0 + 32 * hb + l32;
                const float l_tot = row_sum[(hb * 2) * 32 + l32] + row_sum[(hb * 2 + 1) * 32 + l32];
                const float lse = l_tot > 0.0f ? (row_ref[hb * 32 + l32] + __builtin_log2f(l_tot)) * 0.69314718055994530942f
                                               : -__builtin_inff();
                if (head < p.n_heads) p.lse[(int64_t)split * p.lse_split_stride + (int64_t)r * p.lse_row_stride + head] = lse;
            }
        }
        __syncthreads();
        store_out();
    }
}

// ------------------------------------------------ bf16 queries
// Same workgroup, task, front end, gathers and K-tile layout as above, with the
// score wavefronts arranged so that each owns whole scores: wavefront w < 4 =
// (head group hg = w % 2 of 32 heads, row half rh = w / 2 of each tile) holds
// the queries of its 32 heads over all kD dims (144 registers) and computes
// S^T[16 rows x 32 heads] with v_mfma_f32_16x16x32_f16, two head blocks of 16
// sharing each K operand read.  With no partial scores to swap, the softmax of
// a tile follows its scores in the same phase, and every tile takes one
// barrier:
//   iteration t: scores and softmax of t + 1 (P into P buffer (t + 1) % 2),
//                P.V of t (from P buffer t % 2), dequantization of t + 2 by
//                both roles, gathers of t + 4; barrier.
// Three K tiles are in use in an iteration (t, t + 1, t + 2), so the three
// buffers rotate as before.  K reads for the scores stay at two per element
// (one per head group) and the swap's 16 KB of LDS traffic per tile is gone.
constexpr int kOffP2 = kNBuf * kKTileB;                // two P buffers
static_assert(kOffP2 + 2 * kPXB <= kStageBytes, "P buffers overlap the slot list");

__device__ __forceinline__ floatx4_t mfma16(half8_t a, half8_t b, floatx4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

template <bool ROPE>
__global__ __launch_bounds__(kThreads) void sparse_mla_bf16_kernel(AttnParams p) {
    constexpr int kD = ROPE ? kDim : kLatent;
    constexpr int kKs = kD / 32;               // MFMA k-steps of 32 dims over the whole row
    constexpr int kAhead = 4;                  // score operands read ahead of their MFMAs
    constexpr int kTrAhead = 4;                // P.V operand pairs read ahead
    __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
    int32_t *slots = reinterpret_cast<int32_t *>(lds + kOffSlots);
    int32_t *counts = reinterpret_cast<int32_t *>(lds + kOffCounts);
    float *red = reinterpret_cast<float *>(lds + kOffRed);          // [hg][rh][head]: reference agreement
    float *row_sum = reinterpret_cast<float *>(lds + kOffRowSum);   // [hg][rh][head]: the row halves' l
    float *row_ref = reinterpret_cast<float *>(lds + kOffRowRef);   // [hg][head]: the reference m_ref
    int32_t *flag = reinterpret_cast<int32_t *>(lds + kOffFlag);
    const uint32_t L = lds_addr(lds) + kOffK;      // base of the K tiles and the areas sharing their space

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, g = lane >> 5;
    const int gr = tid & 31, gp = tid >> 5;
    const int r = blockIdx.x, split = blockIdx.y, h0 = blockIdx.z * 64;

    const int n_tiles = (p.k + kTile - 1) / kTile;
    const int t_lo = split * p.tiles_per_split;
    const int t_hi = min(n_tiles, t_lo + p.tiles_per_split);
    const int e_lo = t_lo * kTile;
    const int e_hi = min(p.k, t_hi * kTile);

    const ListCtx lc = list_ctx(p, r);
    const uint8_t *stand_in = reinterpret_cast<const uint8_t *>(p.q);
    uint32_t err = 0;

    // ---- Prologue.  Three dependent round trips (list entries, page-table
    // entries, the first rows) come before the first tile.  A wavefront's
    // loads complete in issue order, so the page-table entries go out as
    // soon as the list is back and before this row's queries (74 KB:
    // consecutive threads take consecutive 16-byte chunks of a head's row);
    // the slots are packed once the entries are back, the first tile's rows
    // are gathered, and only then are the queries converted to fp16 and
    // staged in LDS (in the third K tile and the P buffers, untouched until
    // the first tile's softmax; rows padded by 16 bytes), while the rows are
    // on their way; then the second tile's rows are gathered.  A barrier
    // orders the staged queries before their readers.
    constexpr int kQRow = kD * 2 + 16;
    constexpr int kQChunks = kD * 2 / 16;
    constexpr int kTPH = kThreads / 64;                    // threads per head row
    constexpr int kQPer = kQChunks / kTPH;                 // chunks per thread
    static_assert(kQChunks == kTPH * kQPer, "query chunks do not divide");
    static_assert(2 * kKTileB + 64 * kQRow <= kStageBytes, "staged queries overlap the slot list");
    const uint32_t Lq = L + 2 * kKTileB;
    const uint8_t *qr = reinterpret_cast<const uint8_t *>(p.q) + (int64_t)r * p.q_row_stride * 2;
    const int q_hh = tid / kTPH, q_part = tid % kTPH;
    u32x4_t qc[kQPer];

    int32_t pos[kPosPerLane], phys[kPosPerLane];
    const int first_hi = min(e_hi, e_lo + kSlotCap);
    // The queries as the score MFMAs take them, made by every thread from the
    // 72 values it loaded: a head's 8 threads (consecutive lanes) agree on its
    // largest |q| (non-negative bf16 values order as integers; NaN counts as
    // infinity), whose power-of-two scale qs puts it in [2^13, 2^14), exact
    // in fp16; each value becomes fp16(q qs) (exact unless below fp16's
    // normal range) in place of its bf16, and the head's qs goes to q_scale.
    // Heads past the last take zeros.
    float *q_scale = red;                          // [head]; red is next written after the first tile
    auto stage_q = [&]() {
        const uint32_t keep = h0 + q_hh < p.n_heads ? ~0u : 0u;
#pragma unroll
        for (int i = 0; i < kQPer; ++i) qc[i] &= keep;
        ushort2_t m2 = {0, 0};
#pragma unroll
        for (int i = 0; i < kQPer; ++i)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(ushort2_t, qc[i][c] & 0x7FFF7FFFu));
        uint32_t mb = min(max((uint32_t)m2[0], (uint32_t)m2[1]), 0x7F80u);
        mb = max(mb, (uint32_t)__shfl_xor((int)mb, 1));
        mb = max(mb, (uint32_t)__shfl_xor((int)mb, 2));
        mb = max(mb, (uint32_t)__shfl_xor((int)mb, 4));
        const float qmax = __uint_as_float(mb << 16);
        int ex = 0;
        if (qmax > 0.0f) (void)__builtin_frexpf(qmax, &ex);
        const float qs = __builtin_ldexpf(1.0f, 14 - ex);
        if (q_part == 0) q_scale[q_hh] = qs;
        const uint32_t dst = Lq + q_hh * kQRow + 16 * q_part;
#pragma unroll
        for (int i = 0; i < kQPer; ++i) {
            half8_t h;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                h[2 * c] = (_Float16)(__uint_as_float(qc[i][c] << 16) * qs);
                h[2 * c + 1] = (_Float16)(__uint_as_float(qc[i][c] & 0xFFFF0000u) * qs);
            }
            lds_st<half8_t>(dst + 16 * kTPH * i, h);
        }
    };

    load_positions(lc, e_lo, e_lo < e_hi ? first_hi : e_lo, tid, pos);
    load_pages(p, lc, pos, phys);
    __builtin_amdgcn_sched_barrier(0);             // the page-table loads issue before the query loads
    {
        const uint8_t *src = qr + (int64_t)min(h0 + q_hh, p.n_heads - 1) * p.q_head_stride * 2 + 16 * q_part;
#pragma unroll
        for (int i = 0; i < kQPer; ++i) qc[i] = *reinterpret_cast<const u32x4_t *>(src + 16 * kTPH * i);
    }
    __builtin_amdgcn_sched_barrier(0);
    int nv = __builtin_amdgcn_readfirstlane(pack_slots(p, lc, pos, phys, tid, slots, counts, err));
    if (tid == 0) *flag = 0;
    __syncthreads();
    // the first two tiles' gathers, whether or not the list holds entries
    // (skipped ones read the stand-in): a load count that does not depend on
    // the list lets the query conversion wait for the queries alone.  Tile
    // 0's go out before the conversion and tile 1's after it, so the first
    // burst of row fetches is one tile per workgroup (tile 1 is converted
    // after tile 0's scores).  Parts 0..7 (the score wavefronts') carry the
    // rope.
    GSet<ROPE> G0, G1;
    if (w < 4) gather_set<ROPE>(p.pool, stand_in, slots[gr], gp, G0);
    else gather_set<ROPE, false>(p.pool, stand_in, slots[gr], gp, G0);
    __builtin_amdgcn_sched_barrier(0);             // tile 0's gathers out before the first wait on a query
    stage_q();
    __builtin_amdgcn_sched_barrier(0);
    if (w < 4) gather_set<ROPE>(p.pool, stand_in, slots[kTile + gr], gp, G1);
    else gather_set<ROPE, false>(p.pool, stand_in, slots[kTile + gr], gp, G1);
    __syncthreads();                               // queries staged

    const uint32_t K0 = L, K1 = L + kKTileB, K2 = L + 2 * kKTileB;
    int n_t = 0, n_real = 0, last_rows = kTile;
    bool have_ref = false;
    auto chunk_tiles = [&]() {
        n_real = (nv + kTile - 1) / kTile;
        n_t = (n_real + 1) & ~1;
        last_rows = nv - kTile * (n_real - 1);
    };
    auto tile_lim = [&](int t) { return t < n_real - 1 ? kTile : t == n_real - 1 ? last_rows : 0; };
    auto fresh_chunk = [&](int c_lo, int c_hi) {
        __syncthreads();
        load_positions(lc, c_lo, c_hi, tid, pos);
        load_pages(p, lc, pos, phys);
        nv = __builtin_amdgcn_readfirstlane(pack_slots(p, lc, pos, phys, tid, slots, counts, err));
        __syncthreads();
    };
    auto store_out = [&]() {
        const int n_live = min(64, p.n_heads - h0);
        const int64_t base = (int64_t)split * p.out_split_stride + (int64_t)r * p.out_row_stride + (int64_t)h0 * kLatent;
        const int pc = tid & 127;
        if (p.out_h) {
            _Float16 *ob = p.out_h + base;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int hh = 4 * i + (tid >> 7);
                if (hh < n_live)
                    *reinterpret_cast<half4_t *>(ob + (hh * kLatent + 4 * pc)) = lds_ld<half4_t>(L + hh * kORowH + 8 * pc);
            }
        } else {
            float *ob = p.out + base;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int hh = 8 * i + (tid >> 6);
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int pj = 64 * j + (tid & 63);
                    if (hh < n_live)   // the final fp32 output, non-temporal (prefill 1% faster)
                        __builtin_nontemporal_store(lds_ld<floatx4_t>(L + hh * kORowF + 16 * pj),
                                                    reinterpret_cast<floatx4_t *>(ob + (hh * kLatent + 4 * pj)));
                }
            }
        }
    };

    if (w < 4) {
        // ================================================ score wavefronts
        const int hg = w & 1, rh = w >> 1;
        const int l16 = lane & 15, q4 = lane >> 4;

        // k-step ks of lane group q4 covers chunk C(ks, q4) = 8 (ks / 2) +
        // 2 (ks % 2) + cq, cq = q4 / 2 + 4 (q4 % 2): the two 16-lane groups of
        // a half-wavefront then read chunks 4 apart, whose rows the K-tile
        // layout permutes alike, which a ds_read_b128 needs to be free of bank
        // conflicts (groups with different permutations in one half-wavefront
        // conflict two-way).  Any assignment of dims to (ks, q4) gives the same
        // scores as long as queries and keys share it.
        const int cq = (q4 >> 1) + 4 * (q4 & 1);
        // queries: B operand of S^T = K Q^T.  Lane (l16, q4) holds head h0 +
        // 32 hg + 16 hb + l16, dims 8 C(ks, q4) .. +7, as staged in fp16;
        // score_mul = sm_scale log2(e) / qs turns scores into log2 units.
        half8_t qb[2][kKs];
        float score_mul[2];
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
            const uint32_t qf = Lq + (32 * hg + 16 * hb + l16) * kQRow + 16 * cq;
#pragma unroll
            for (int ks = 0; ks < kKs; ++ks) qb[hb][ks] = lds_ld<half8_t>(qf + 128 * (ks >> 1) + 32 * (ks & 1));
            score_mul[hb] = p.score_mul / q_scale[32 * hg + 16 * hb + l16];
        }

        // score operand (A of 16x16x32): row 16 rh + l16, chunk C(ks, q4), at
        // a_off[ks % 2] + 8 kChunkB (ks / 2) (C % 4 = 2 (ks % 2) + q4 / 2)
        const uint32_t a_off0 = cq * kChunkB + 16 * ((16 * rh + l16) ^ (4 * (q4 >> 1)));
        const uint32_t a_off1 = (cq + 2) * kChunkB + 16 * ((16 * rh + l16) ^ (4 * (2 + (q4 >> 1))));
        // P of head 32 hg + 16 hb + l16, rows 16 rh + 4 q4 + 0..3: 8 contiguous
        // bytes in the P.V operand order (row bits 2 and 3 swapped)
        const uint32_t px_w = L + kOffP2 + (32 * hg + l16) * kPXHead + 2 * (16 * rh + 8 * (q4 & 1) + 4 * (q4 >> 1));
        const int row0 = 16 * rh + 4 * q4;         // this lane's first row

        float m_ref[2] = {-__builtin_inff(), -__builtin_inff()};
        float m_rel[2] = {-__builtin_inff(), -__builtin_inff()};   // largest s - m_ref of this pass
        float l_run[2] = {0.0f, 0.0f};

        auto scores = [&](uint32_t kb, floatx4_t (&acc)[2]) {
            const uint32_t a0 = kb + a_off0, a1 = kb + a_off1;
            auto a_at = [&](int ks) { return (ks & 1 ? a1 : a0) + 8 * kChunkB * (ks >> 1); };
            half8_t a[kAhead];
#pragma unroll
            for (int i = 0; i < kAhead; ++i) a[i] = lds_ld<half8_t>(a_at(i));
            __builtin_amdgcn_sched_barrier(0);
            acc[0] = floatx4_t{0, 0, 0, 0};
            acc[1] = floatx4_t{0, 0, 0, 0};
#pragma unroll
            for (int ks = 0; ks < kKs; ++ks) {
                const half8_t cur = a[ks % kAhead];
                acc[0] = mfma16(cur, qb[0][ks], acc[0]);
                acc[1] = mfma16(cur, qb[1][ks], acc[1]);
                if (ks + kAhead < kKs) a[ks % kAhead] = lds_ld<half8_t>(a_at(ks + kAhead));
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        // the same, with the dequantization of set G into the K tile at kd laid
        // between the first MFMAs (an in-order wavefront then issues its
        // conversions and stores while the matrix pipe works) and, once G is
        // consumed, the gather of slot `next` into it: as early in the phase
        // as possible, for the longest time in flight
        auto scores_dq = [&](uint32_t kb, floatx4_t (&acc)[2], uint32_t kd, GSet<ROPE> &G, int32_t next) {
            const uint32_t a0 = kb + a_off0, a1 = kb + a_off1;
            auto a_at = [&](int ks) { return (ks & 1 ? a1 : a0) + 8 * kChunkB * (ks >> 1); };
            half8_t a[kAhead];
#pragma unroll
            for (int i = 0; i < kAhead; ++i) a[i] = lds_ld<half8_t>(a_at(i));
            __builtin_amdgcn_sched_barrier(0);
            acc[0] = floatx4_t{0, 0, 0, 0};
            acc[1] = floatx4_t{0, 0, 0, 0};
            half2_t dd;
            static_for<0, kKs>([&](auto slot) {
                constexpr int ks = decltype(slot)::value;
                const half8_t cur = a[ks % kAhead];
                acc[0] = mfma16(cur, qb[0][ks], acc[0]);
                acc[1] = mfma16(cur, qb[1][ks], acc[1]);
                if constexpr (ks + kAhead < kKs) a[ks % kAhead] = lds_ld<half8_t>(a_at(ks + kAhead));
                if constexpr (ks == 0) dd = dq_scales<ROPE>(G, gp);
                if constexpr (ks >= 1 && ks <= 4) dq_chunk<ROPE>(kd, gr, gp, ks - 1, dd, G);
                if constexpr (ROPE && ks == 5) dq_rope<ROPE>(kd, gr, gp, G);
                if constexpr (ks == 6) gather_set<ROPE>(p.pool, stand_in, next, gp, G);
                __builtin_amdgcn_sched_barrier(0);
            });
        };
        // P = 2^(s - m_ref) of this lane's 4 rows x 2 heads into P buffer pb;
        // rows >= lim are padding
        // (the padding rows' masking only in a chunk's last tile, a uniform
        // branch; whether P could overflow fp16 is judged from m_rel once per
        // pass)
        auto softmax = [&](const floatx4_t (&acc)[2], int lim, int pb) {
            float e[2][4];
#pragma unroll
            for (int hb = 0; hb < 2; ++hb)
#pragma unroll
                for (int i = 0; i < 4; ++i) e[hb][i] = __builtin_fmaf(acc[hb][i], score_mul[hb], -m_ref[hb]);
            if (lim < kTile) {
#pragma unroll
                for (int hb = 0; hb < 2; ++hb)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (row0 + i >= lim) e[hb][i] = -__builtin_inff();
            }
#pragma unroll
            for (int hb = 0; hb < 2; ++hb)
                m_rel[hb] = __builtin_fmaxf(m_rel[hb], __builtin_fmaxf(__builtin_fmaxf(e[hb][0], e[hb][1]),
                                                                        __builtin_fmaxf(e[hb][2], e[hb][3])));
            const half2_t one2 = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
                half4_t ph;
#pragma unroll
                for (int i = 0; i < 4; ++i) ph[i] = (_Float16)__builtin_amdgcn_exp2f(e[hb][i]);   // exp2(-inf) = 0
                float ls = __builtin_amdgcn_fdot2(half2_t{ph[0], ph[1]}, one2, 0.0f, false);
                ls = __builtin_amdgcn_fdot2(half2_t{ph[2], ph[3]}, one2, ls, false);
                l_run[hb] += ls;
                lds_st<half4_t>(px_w + pb * kPXB + hb * (16 * kPXHead), ph);
            }
        };
        // phase: scores and softmax of t + 1, with the dequantization of t + 2
        // (latent dims 0..255 and the rope) and the gather of t + 4 (clamped
        // to the chunk's last tile: a harmless repeat) inside the scores; the
        // last phase of a chunk has no scores and needs neither
        auto iteration = [&](int t, GSet<ROPE> &G, uint32_t bB, uint32_t bC) {
            const int32_t next = slots[min(t + 4, n_t - 1) * kTile + gr];
            if (t + 1 < n_t) {
                // the dequantization runs whether tile t + 2 exists or not:
                // bC's last reader was the P.V of t - 1, and a set past the
                // chunk holds a repeat of its last tile
                floatx4_t acc[2];
                scores_dq(bB, acc, bC, G, next);
                softmax(acc, tile_lim(t + 1), (t + 1) & 1);
            }
            __syncthreads();
        };

        for (int pass = 0; pass < 2; ++pass) {
            m_rel[0] = m_rel[1] = -__builtin_inff();
            l_run[0] = l_run[1] = 0.0f;
            for (int c_lo = e_lo; c_lo < e_hi; c_lo += kSlotCap) {
                const int c_hi = min(e_hi, c_lo + kSlotCap);
                if (c_lo != e_lo || (pass == 1 && e_hi - e_lo > kSlotCap)) fresh_chunk(c_lo, c_hi);
                chunk_tiles();
                if (n_real == 0) continue;         // nothing valid in this chunk (uniform)
                if (pass == 1 || c_lo != e_lo) {   // the first chunk's were gathered before the passes
                    gather_set<ROPE>(p.pool, stand_in, slots[gr], gp, G0);
                    gather_set<ROPE>(p.pool, stand_in, slots[kTile + gr], gp, G1);
                }
                dequant_set<ROPE>(K0, gr, gp, true, G0);
                gather_set<ROPE>(p.pool, stand_in, slots[min(2, n_t - 1) * kTile + gr], gp, G0);
                __syncthreads();                   // tile 0 in LDS (tile 1 follows, under its scores)
                {
                    floatx4_t acc[2];
                    scores(K0, acc);
                    if (!have_ref) {               // first tile with entries: each head's reference
                        const int lim = tile_lim(0);
#pragma unroll
                        for (int hb = 0; hb < 2; ++hb) {
                            float tmax = -__builtin_inff();
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                if (row0 + i < lim) tmax = __builtin_fmaxf(tmax, acc[hb][i] * score_mul[hb]);
                            tmax = __builtin_fmaxf(tmax, __shfl_xor(tmax, 16));
                            tmax = __builtin_fmaxf(tmax, __shfl_xor(tmax, 32));
                            if (q4 == 0) red[(hg * 2 + rh) * 32 + 16 * hb + l16] = tmax;
                        }
                        __syncthreads();
#pragma unroll
                        for (int hb = 0; hb < 2; ++hb)
                            m_ref[hb] = __builtin_fmaxf(red[(hg * 2) * 32 + 16 * hb + l16], red[(hg * 2 + 1) * 32 + 16 * hb + l16]);
                        have_ref = true;
                    }
                    softmax(acc, tile_lim(0), 0);
                }
                dequant_set<ROPE>(K1, gr, gp, true, G1);
                gather_set<ROPE>(p.pool, stand_in, slots[min(3, n_t - 1) * kTile + gr], gp, G1);
                __syncthreads();                   // P of tile 0 in P buffer 0, tile 1 in LDS
                uint32_t bA = K0, bB = K1, bC = K2;
                for (int t = 0; t < n_t; t += 2) {
                    iteration(t, G0, bB, bC);      // G0: tile t + 2 -> bC, then t + 4
                    iteration(t + 1, G1, bC, bA);  // G1: tile t + 3 -> bA, then t + 5
                    const uint32_t a0 = bA;        // tiles t + 2, t + 3, t + 4 go to bC, bA, bB
                    bA = bC;
                    bC = bB;
                    bB = a0;
                }
            }
            if (__builtin_fmaxf(m_rel[0], m_rel[1]) > kRefSlack) *flag = 1;   // P could have overflowed fp16
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {       // this pass's row sums and reference
                float l2 = l_run[hb] + __shfl_xor(l_run[hb], 16);
                l2 += __shfl_xor(l2, 32);
                if (q4 == 0) row_sum[(hg * 2 + rh) * 32 + 16 * hb + l16] = l2;
                if (q4 == 0 && rh == 0) row_ref[hg * 32 + 16 * hb + l16] = have_ref ? m_ref[hb] : 0.0f;
            }
            __syncthreads();
            if (pass == 1 || *flag == 0) break;    // uniform: read after the barrier
            // second pass: the exact maximum of every head as its reference
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
                // the largest e + m_ref of the pass: rounding is monotonic, so
                // adding m_ref after the maximum gives the same value
                const float m_abs = m_rel[hb] + m_ref[hb];
                float mm = __builtin_fmaxf(m_abs, __shfl_xor(m_abs, 16));
                mm = __builtin_fmaxf(mm, __shfl_xor(mm, 32));
                if (q4 == 0) red[(hg * 2 + rh) * 32 + 16 * hb + l16] = mm;
            }
            __syncthreads();
#pragma unroll
            for (int hb = 0; hb < 2; ++hb)
                m_ref[hb] = __builtin_fmaxf(red[(hg * 2) * 32 + 16 * hb + l16], red[(hg * 2 + 1) * 32 + 16 * hb + l16]);
        }

        if (err && p.err_word) atomicOr(p.err_word, err);
        __syncthreads();                           // the P.V wavefronts have staged the output
        store_out();
    } else {
        // ================================================ P.V wavefronts
        const int dq = w - 4;
        // parts 8..15 of a tile's rows, no rope
        auto gather_units = [&](int tile, GSet<ROPE> &G) {
            gather_set<ROPE, false>(p.pool, stand_in, slots[tile * kTile + gr], gp, G);
        };

        // transposing reads (A of O^T = V^T P^T), as in the fp32-query kernel
        const int cc = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1), j4 = (lane >> 2) & 3;
        const uint32_t tr_off0 = (16 * dq + cc) * kChunkB + 16 * (j4 + 4 * (g ^ (cc & 1)) + 8 * (cc >> 1)) + 8 * (lane & 1);
        const uint32_t tr_off1 = (16 * dq + cc) * kChunkB + 16 * (j4 + 4 * (g ^ (cc & 1)) + 8 * (1 ^ (cc >> 1))) + 8 * (lane & 1);
        const uint32_t px_r = L + kOffP2 + l32 * kPXHead + 2 * (8 * g);
        floatx16_t o[4][2];

        auto pv = [&](uint32_t kb, int pb, uint32_t kd, GSet<ROPE> &G, int32_t next) {
            const uint32_t t0 = kb + tr_off0, t1 = kb + tr_off1;
            half8_t pbv[2][2];
#pragma unroll
            for (int hb = 0; hb < 2; ++hb)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
                    pbv[hb][kk] = lds_ld<half8_t>(px_r + pb * kPXB + hb * (32 * kPXHead) + 32 * kk);
            short4_t lo[kTrAhead], hi[kTrAhead];
            auto issue = [&](int j) {
                const int md = j & 3, kk = j >> 2;
                lo[j % kTrAhead] = lds_read_tr16(t0 + 4 * kChunkB * md + 256 * kk);
                hi[j % kTrAhead] = lds_read_tr16(t1 + 4 * kChunkB * md + 256 * kk);
            };
#pragma unroll
            for (int j = 0; j < kTrAhead; ++j) issue(j);
            __builtin_amdgcn_sched_barrier(0);
            static_for<0, 8>([&](auto step) {
                constexpr int j = decltype(step)::value;
                constexpr int md = j & 3, kk = j >> 2;
                const half8_t a = __builtin_bit_cast(
                    half8_t, __builtin_shufflevector(lo[j % kTrAhead], hi[j % kTrAhead], 0, 1, 2, 3, 4, 5, 6, 7));
                o[md][0] = mfma32(a, pbv[0][kk], o[md][0]);
                o[md][1] = mfma32(a, pbv[1][kk], o[md][1]);
                if constexpr (j + kTrAhead < 8) issue(j + kTrAhead);
                __builtin_amdgcn_sched_barrier(0);
            });
            // the dequantization after the MFMAs are issued: the matrix pipe
            // is then this wavefront's alone (the score wavefront's MFMAs are
            // done), so the conversions overlap its last MFMAs
            const half2_t dd = dq_scales<ROPE>(G, gp);
#pragma unroll
            for (int i = 0; i < 4; ++i) dq_chunk<ROPE>(kd, gr, gp, i, dd, G);
            gather_set<ROPE, false>(p.pool, stand_in, next, gp, G);   // G consumed: refill
        };
        // phase: P.V of t, then the dequantization of t + 2 (latent dims
        // 256..511; it runs whether t + 2 exists or not, as on the score
        // side) and the gather of t + 4
        auto iteration = [&](int t, GSet<ROPE> &G, uint32_t bA, uint32_t bC) {
            // the slot read first: waiting for it later would wait for every
            // LDS access issued since
            const int32_t next = slots[min(t + 4, n_t - 1) * kTile + gr];
            pv(bA, t & 1, bC, G, next);
            __syncthreads();
        };

        for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
            for (int md = 0; md < 4; ++md) o[md][0] = o[md][1] = floatx16_t{};
            for (int c_lo = e_lo; c_lo < e_hi; c_lo += kSlotCap) {
                const int c_hi = min(e_hi, c_lo + kSlotCap);
                if (c_lo != e_lo || (pass == 1 && e_hi - e_lo > kSlotCap)) fresh_chunk(c_lo, c_hi);
                chunk_tiles();
                if (n_real == 0) continue;
                if (pass == 1 || c_lo != e_lo) {
                    gather_units(0, G0);
                    gather_units(1, G1);
                }
                dequant_set<ROPE>(K0, gr, gp, false, G0);
                gather_units(min(2, n_t - 1), G0);
                __syncthreads();                   // tile 0 in LDS
                dequant_set<ROPE>(K1, gr, gp, false, G1);   // while tile 0 is scored
                gather_units(min(3, n_t - 1), G1);
                if (!have_ref) {
                    __syncthreads();               // the reference is agreed
                    have_ref = true;
                }
                __syncthreads();                   // P of tile 0 in P buffer 0, tile 1 in LDS
                uint32_t bA = K0, bB = K1, bC = K2;
                for (int t = 0; t < n_t; t += 2) {
                    iteration(t, G0, bA, bC);
                    iteration(t + 1, G1, bB, bA);
                    const uint32_t a0 = bA;
                    bA = bC;
                    bC = bB;
                    bB = a0;
                }
            }
            __syncthreads();
            if (pass == 1 || *flag == 0) break;
            __syncthreads();                       // the second pass's reference is agreed
        }

        if (err && p.err_word) atomicOr(p.err_word, err);
        // O = O_acc / l staged for the coalesced store (row sums and the
        // reference were written before the passes' last barrier)
        // the lane index read afresh (not derived from values kept through
        // the loop, which would hold registers there)
        int ln;
        asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
        const int el32 = ln & 31, eg = ln >> 5;
        auto stage = [&](auto half_out) {
            constexpr bool kH = decltype(half_out)::value;
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
                const float l_tot = row_sum[(hb * 2) * 32 + el32] + row_sum[(hb * 2 + 1) * 32 + el32];
                const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
                const uint32_t row = L + (32 * hb + el32) * (kH ? kORowH : kORowF);
#pragma unroll
                for (int md = 0; md < 4; ++md)
#pragma unroll
                    for (int vq = 0; vq < 4; ++vq) {
                        const int dim = 128 * dq + 32 * md + 8 * vq + 4 * eg;
                        const floatx4_t v = floatx4_t{o[md][hb][4 * vq], o[md][hb][4 * vq + 1], o[md][hb][4 * vq + 2],
                                                      o[md][hb][4 * vq + 3]} * inv;
                        if constexpr (kH) lds_st<half4_t>(row + 2 * dim, __builtin_convertvector(v, half4_t));
                        else lds_st<floatx4_t>(row + 4 * dim, v);
                    }
            }
        };
        if (p.out_h) stage(std::true_type{});
        else stage(std::false_type{});
        if (dq == 0 && g == 0 && p.lse) {
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
                const int head = h0 + 32 * hb + l32;
                const float l_tot = row_sum[(hb * 2) * 32 + l32] + row_sum[(hb * 2 + 1) * 32 + l32];
                const float lse = l_tot > 0.0f ? (row_ref[hb * 32 + l32] + __builtin_log2f(l_tot)) * 0.69314718055994530942f
                                               : -__builtin_inff();
                if (head < p.n_heads) p.lse[(int64_t)split * p.lse_split_stride + (int64_t)r * p.lse_row_stride + head] = lse;
            }
        }
        __syncthreads();
        store_out();
    }
}

hipError_t launch_sparse_mla(const AttnParams &p, bool q_f32, int32_t n_splits, hipStream_t stream) {
    if (p.n_rows == 0) return hipSuccess;
    const dim3 grid((unsigned)p.n_rows, (unsigned)n_splits, (unsigned)((p.n_heads + 63) / 64));
    if (p.rope_dims == kRope) {
        if (q_f32) hipLaunchKernelGGL((sparse_mla_f32q_kernel<true>), grid, dim3(kThreads), 0, stream, p);
        else hipLaunchKernelGGL((sparse_mla_bf16_kernel<true>), grid, dim3(kThreads), 0, stream, p);
    } else {
        if (q_f32) hipLaunchKernelGGL((sparse_mla_f32q_kernel<false>), grid, dim3(kThreads), 0, stream, p);
        else hipLaunchKernelGGL((sparse_mla_bf16_kernel<false>), grid, dim3(kThreads), 0, stream, p);
    }
    return hipGetLastError();
}

// --------------------------------------------------- dequantizing gather

// A test and debugging aid that runs the attention kernel's own front end:
// one workgroup per (query row, chunk of 2048 entries) translates the chunk
// with load_positions / load_pages / pack_slots and dequantizes each tile with
// gather_set / dequant_set into an LDS K tile, which it then copies out
// row-major.  Entry j of a chunk's output is the j-th valid entry of the chunk
// (list order), as the attention kernel's tiles hold it; entries past the valid
// count get slot -1 and zeros.
template <bool ROPE>
__global__ __launch_bounds__(kThreads) void gather_dequant_kernel(AttnParams p, uint16_t *__restrict__ out,
                                                                  int32_t *__restrict__ slots_out) {
    constexpr int kD = ROPE ? kDim : kLatent;
    __shared__ __attribute__((aligned(16))) uint8_t lds[kKTileB + kSlotCap * 4 + kPosPerLane * 8 * 4];
    int32_t *slots = reinterpret_cast<int32_t *>(lds + kKTileB);
    int32_t *counts = reinterpret_cast<int32_t *>(lds + kKTileB + kSlotCap * 4);
    const uint32_t kb = lds_addr(lds);
    const int tid = threadIdx.x, gr = tid & 31, gp = tid >> 5;
    const int r = blockIdx.x;
    const int c_lo = blockIdx.y * kSlotCap, c_hi = min(p.k, c_lo + kSlotCap);
    const ListCtx lc = list_ctx(p, r);
    uint32_t err = 0;
    int32_t pos[kPosPerLane], phys[kPosPerLane];
    load_positions(lc, c_lo, c_hi, tid, pos);
    load_pages(p, lc, pos, phys);
    const int nv = pack_slots(p, lc, pos, phys, tid, slots, counts, err);
    __syncthreads();
    if (err && p.err_word) atomicOr(p.err_word, err);
    const int64_t base = (int64_t)r * p.k + c_lo;
    if (slots_out)
        for (int e = tid; e < c_hi - c_lo; e += kThreads) slots_out[base + e] = e < nv ? slots[e] : -1;
    const int n_t = (nv + kTile - 1) / kTile;
    const uint8_t *stand_in = reinterpret_cast<const uint8_t *>(out);   // any 352 readable bytes: the output (>= 1024)
    for (int t = 0; t * kTile < c_hi - c_lo; ++t) {
        if (t < n_t) {
            GSet<ROPE> G;
            gather_set<ROPE>(p.pool, stand_in, slots[t * kTile + gr], gp, G);
            dequant_set<ROPE>(kb, gr, gp, tid < 256, G);
        }
        __syncthreads();
        for (int i = tid; i < kTile * (kD / 8); i += kThreads) {       // (row, chunk) pieces of 16 bytes
            const int row = i / (kD / 8), c = i % (kD / 8), e = t * kTile + row;
            if (e < c_hi - c_lo) {
                const u32x4_t v = t < n_t ? lds_ld<u32x4_t>(kb + kswz(row, c)) : u32x4_t{0, 0, 0, 0};
                *reinterpret_cast<u32x4_t *>(out + (base + e) * kD + 8 * c) = v;
            }
        }
        __syncthreads();
    }
}

hipError_t launch_gather_dequant(const AttnParams &p, uint16_t *out, int32_t *slots_out, hipStream_t stream) {
    if (p.n_rows == 0 || p.k == 0) return hipSuccess;
    const dim3 grid((unsigned)p.n_rows, (unsigned)((p.k + kSlotCap - 1) / kSlotCap));
    if (p.rope_dims == kRope) hipLaunchKernelGGL(gather_dequant_kernel<true>, grid, dim3(kThreads), 0, stream, p, out, slots_out);
    else hipLaunchKernelGGL(gather_dequant_kernel<false>, grid, dim3(kThreads), 0, stream, p, out, slots_out);
    return hipGetLastError();
}

// ----------------------------------------------------------------- merge

// One wavefront per state t and 256 dims of it, a lane owning 4 consecutive
// dims, or 512 (W = 2 pieces of 4 per lane) when the grid has wavefronts to
// spare: half the wavefronts, each with twice the loads in flight.  Lane s loads part s's lse (at most 64 parts) and computes its weight;
// the lanes read the maximum, the weights and their sum across the wavefront,
// so there is no LDS and no barrier.  With at most 32 parts (decode's case) the
// parts' o are loaded together with the lse, one round trip for all.  With M the
// largest lse: w_s = exp(lse_s - M) (an empty part weighs 0), W = the w_s
// summed in part order, o = (the w_s o_s summed in part order) / W, lse = M +
// ln W; all parts empty gives o = 0, lse = -inf.
constexpr int kMergeSeg = 256;                 // dims per wavefront and piece per lane
constexpr int kMergeWaves = 4;                 // wavefronts per workgroup
// at least this many 256-dim tasks (16 wavefronts per CU), at most 8 parts, dim
// a multiple of 8 and 16-byte aligned parts: 512 dims per wavefront, fp16
// parts read 16 bytes a lane and part.  Measured: the long-context decode step's merge
// (4096 states, 4 parts) 0.4 us faster; 8 requests x 64 heads with 16 parts
// (1024 tasks) 1 us slower.
constexpr int64_t kWideMergeTasks = 4096;

// four consecutive dims of one part's o as stored (fp16 parts stay fp16 until
// used), and widened to fp32 (exact)
template <bool F16>
using PartPiece = std::conditional_t<F16, half4_t, floatx4_t>;
template <bool F16>
__device__ __forceinline__ PartPiece<F16> load_piece(const MergeParams &p, int64_t off) {
    if constexpr (F16) return *reinterpret_cast<const half4_t *>(p.part_o_h + off);
    else return *reinterpret_cast<const floatx4_t *>(p.part_o + off);
}
template <bool F16>
__device__ __forceinline__ floatx4_t widen(PartPiece<F16> x) {
    if constexpr (F16) return __builtin_convertvector(x, floatx4_t);
    else return x;
}

// task = (state t, segment of 256 W dims) for the calling wavefront; the lane
// owns dims d + 4j (j < W).  B > 0: at most B parts, all loaded before any is
// used (a part past the last re-reads the last; it is not used); B = 0: any
// count, loaded as used.
template <bool F16, int B, int W>
__device__ __forceinline__ void merge_task(const MergeParams &p, int64_t task, int n_seg, int lane) {
    const int64_t t = task / n_seg;
    const int seg = (int)(task - t * n_seg);
    const int d = seg * kMergeSeg * W + 4 * W * lane;
    const int S = p.n_parts;
    bool live[W];
    int64_t o_t[W];                                             // part s at s * n_states * dim
#pragma unroll
    for (int j = 0; j < W; ++j) {
        live[j] = d + 4 * j < p.dim;
        o_t[j] = t * p.dim + (live[j] ? d + 4 * j : 0);
    }
    const int64_t o_stride = p.n_states * (int64_t)p.dim;
    // lane s holds part s's lse and, once M is known, its weight; every lane
    // reads them from there in part order
    // (no load sits under a branch, so none waits for another)
    const float my_raw = p.part_lse[t + (int64_t)min(lane, S - 1) * p.n_states];
    PartPiece<F16> v[B > 0 ? B : 1][W];
    if constexpr (B > 0) {
#pragma unroll
        for (int s = 0; s < B; ++s) {
            if constexpr (W == 2 && F16) {     // dim % 8 == 0 and 16-byte aligned parts (checked at launch)
                const half8_t x = *reinterpret_cast<const half8_t *>(p.part_o_h + o_t[0] + min(s, S - 1) * o_stride);
                v[s][0] = half4_t{x[0], x[1], x[2], x[3]};
                v[s][1] = half4_t{x[4], x[5], x[6], x[7]};
            } else {
#pragma unroll
                for (int j = 0; j < W; ++j) v[s][j] = load_piece<F16>(p, o_t[j] + min(s, S - 1) * o_stride);
            }
        }
    }
    const float my = lane < S ? my_raw : -__builtin_inff();
    auto lane_val = [](float x, int s) {
        return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), s));
    };
    float M = -__builtin_inff();
    for (int s = 0; s < S; ++s) M = __builtin_fmaxf(M, lane_val(my, s));
    const float my_w = my == -__builtin_inff() || M == -__builtin_inff() ? 0.0f : expf(my - M);
    auto weight = [&](int s) { return lane_val(my_w, s); };
    float Wsum = 0.0f;
    if (M != -__builtin_inff())
        for (int s = 0; s < S; ++s) Wsum += weight(s);
    if (seg == 0 && lane == 0 && p.lse) p.lse[t] = M == -__builtin_inff() ? M : M + logf(Wsum);
    const float inv = Wsum > 0.0f ? 1.0f / Wsum : 0.0f;
    floatx4_t acc[W];
#pragma unroll
    for (int j = 0; j < W; ++j) acc[j] = floatx4_t{0, 0, 0, 0};
    if (Wsum > 0.0f) {
        if constexpr (B > 0) {
#pragma unroll
            for (int s = 0; s < B; ++s) {
                if (s < S) {
                    const float ws = weight(s);
                    if (ws != 0.0f)
#pragma unroll
                        for (int j = 0; j < W; ++j) acc[j] += ws * widen<F16>(v[s][j]);
                }
            }
        } else {
            for (int s = 0; s < S; ++s) {
                const float ws = weight(s);
                if (ws != 0.0f)
#pragma unroll
                    for (int j = 0; j < W; ++j) acc[j] += ws * widen<F16>(load_piece<F16>(p, o_t[j] + s * o_stride));
            }
        }
    }
    float *orow = p.out + (t / p.states_per_row) * p.out_row_stride + (t % p.states_per_row) * p.out_col_stride;
    // non-temporal: the result is not read again here, and keeping it out of
    // L2 spares the write-back at the kernel's end (C3 step 1% faster)
#pragma unroll
    for (int j = 0; j < W; ++j)
        if (live[j]) __builtin_nontemporal_store(acc[j] * inv, reinterpret_cast<floatx4_t *>(orow + d + 4 * j));
}

// wavefronts take tasks in order, the grid's wavefronts apart
// Workgroup b takes tasks [kMergeWaves v, +kMergeWaves), v = b unless the
// placement hint applies (one pass over whole groups of states, a whole number
// of workgroups per group, groups a multiple of 8): then workgroup b, dealt to
// XCD b % 8, takes the groups g = b % 8 (mod 8), so it reads the parts that
// workgroups on its own XCD wrote.
__device__ __forceinline__ int64_t merge_block(const MergeParams &p, int n_seg) {
    const int64_t b = blockIdx.x;
    if (p.xcd_group <= 0 || p.n_states % (8 * p.xcd_group)) return b;
    const int64_t per_group = p.xcd_group * n_seg;          // tasks of a group
    if (per_group % kMergeWaves) return b;
    const int64_t wg_per_group = per_group / kMergeWaves;
    if ((int64_t)gridDim.x != (p.n_states / p.xcd_group) * wg_per_group) return b;
    const int64_t j = b / 8;
    return (8 * (j / wg_per_group) + b % 8) * wg_per_group + j % wg_per_group;
}

template <bool F16, int B, int W>
__global__ __launch_bounds__(64 * kMergeWaves) void merge_states_kernel(MergeParams p) {
    const int n_seg = (p.dim + kMergeSeg * W - 1) / (kMergeSeg * W);
    const int64_t tasks = p.n_states * n_seg;
    const int64_t stride = (int64_t)gridDim.x * kMergeWaves;
    for (int64_t task = merge_block(p, n_seg) * kMergeWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
         task < tasks; task += stride)
        merge_task<F16, B, W>(p, task, n_seg, threadIdx.x & 63);
}

template <bool F16>
void launch_merge(const MergeParams &p, bool wide, dim3 grid, dim3 block, hipStream_t stream) {
    if (wide && p.n_parts <= 4) hipLaunchKernelGGL((merge_states_kernel<F16, 4, 2>), grid, block, 0, stream, p);
    else if (wide) hipLaunchKernelGGL((merge_states_kernel<F16, 8, 2>), grid, block, 0, stream, p);
    else if (p.n_parts <= 4) hipLaunchKernelGGL((merge_states_kernel<F16, 4, 1>), grid, block, 0, stream, p);
    else if (p.n_parts <= 8) hipLaunchKernelGGL((merge_states_kernel<F16, 8, 1>), grid, block, 0, stream, p);
    else if (p.n_parts <= 16) hipLaunchKernelGGL((merge_states_kernel<F16, 16, 1>), grid, block, 0, stream, p);
    else if (p.n_parts <= 32) hipLaunchKernelGGL((merge_states_kernel<F16, 32, 1>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((merge_states_kernel<F16, 0, 1>), grid, block, 0, stream, p);
}

hipError_t launch_merge_states(const MergeParams &p, hipStream_t stream) {
    if (p.n_states == 0) return hipSuccess;
    const bool aligned = !p.part_o_h || reinterpret_cast<uintptr_t>(p.part_o_h) % 16 == 0;
    const bool wide = p.n_parts <= 8 && p.dim % 8 == 0 && aligned &&
                      p.n_states * ((p.dim + kMergeSeg - 1) / kMergeSeg) >= kWideMergeTasks;
    const int seg = kMergeSeg * (wide ? 2 : 1);
    const int64_t tasks = p.n_states * ((p.dim + seg - 1) / seg);
    const dim3 grid((unsigned)std::min<int64_t>((tasks + kMergeWaves - 1) / kMergeWaves, 1 << 20)),
        block(64 * kMergeWaves);
    if (p.part_o_h) launch_merge<true>(p, wide, grid, block, stream);
    else launch_merge<false>(p, wide, grid, block, stream);
    return hipGetLastError();
}

}  // namespace kv4
