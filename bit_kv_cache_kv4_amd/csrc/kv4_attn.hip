// Sparse MLA attention over the 4-bit pool: decode (split-K) and prefill.
//
// README "60+ inference optimizations & kernels": section "4-bit KV cache"
// (kv4mla dequantizes the 4-bit rows on chip instead of into an FP8 scratch
// copy), section "AMD MI355X" (hand-written HIP sparse MLA decode whose K tile
// in LDS is also the PV operand; split-K decode), "Parallelism and
// disaggregation" (per-part (o, lse) and a merge).  sgl-amd-mono GLM-5.3 PR,
// "Modifications": 64-token page table and its stride as launch arguments;
// one split task serves 16 heads so each key row is gathered once per task.
//
// Workgroup = 4 wavefronts = (query row r, split s, chunk of up to 64 heads).
// Wavefront w owns 16 heads.  Per tile of 32 list entries:
//   1. the entries' pool slots (translated once per chunk of 2048 entries and
//      kept in LDS) name 32 rows; the 256 lanes gather them straight from HBM
//      (lane = row pair x 16-byte code chunk), one tile ahead of the math;
//   2. the lanes dequantize codes x block scale and rope to fp16 (every such
//      product is exact in fp16) into two LDS layouts: K[32 rows][576] for the
//      scores and V^T[512 dims][32 rows] for P.V;
//   3. each wavefront computes S^T[32 rows x 16 heads] = K Q^T with
//      v_mfma_f32_16x16x32_f16 (Q in registers, pre-scaled per head by a power
//      of two so bf16/fp32 queries fit fp16 exactly), an online softmax in
//      base 2 with lazy rescaling, and O^T[512 x 16] += V^T P^T with the same
//      MFMA, P staying in the registers the scores came out in.
// The per-split result is written normalised with its lse; a split count of 1
// writes the final output.
#include "kv4_device.h"
#include "kv4_launch.h"

namespace kv4 {

constexpr int kTile = 32;                              // list entries per tile
constexpr int kKPitchHalf = 584;                       // 576 + 8 pad: conflict-free 16-byte reads
constexpr int kKPitchDw = kKPitchHalf / 2;
constexpr int kKTileDw = kTile * kKPitchDw;            // 9344 dwords
constexpr int kVtPitchDw = 16;                         // 32 rows of fp16 per latent dim, swizzled
constexpr int kVtDw = kLatent * kVtPitchDw;            // 8192 dwords
constexpr int kSlotCap = 2048;                         // entries translated per chunk
constexpr int kLdsDw = kKTileDw + kVtDw + kSlotCap;    // 78336 bytes
constexpr float kRescaleSlack = 8.0f;                  // log2 units the running max may lag

// V^T row layout: the 32 rows of a tile sit in the order the score
// accumulator hands them to each lane group g: positions 8g..8g+3 hold rows
// 4g..4g+3 and 8g+4..8g+7 hold rows 16+4g..16+4g+3.  Rows 2p and 2p+1 share a
// dword; vt_pair_dw(p) is that dword.  The dword index is XOR-swizzled by
// latent dim so 16-byte reads of eight consecutive dims hit distinct banks.
__device__ __forceinline__ int vt_pair_dw(int p) { return 4 * ((p & 7) >> 1) + 2 * (p >> 3) + (p & 1); }
__device__ __forceinline__ int vt_swz(int d) { return 4 * ((d >> 1) & 3); }
__device__ __forceinline__ int vt_addr(int d, int dw) { return d * kVtPitchDw + (dw ^ vt_swz(d)); }

__device__ __forceinline__ floatx4_t mfma16(half8_t a, half8_t b, floatx4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

template <bool QF32>
__global__ __launch_bounds__(256, 1) void sparse_mla_kernel(AttnParams p) {
    __shared__ uint32_t lds[kLdsDw];
    uint32_t *ktile = lds;
    uint32_t *vt = lds + kKTileDw;
    int32_t *slots = reinterpret_cast<int32_t *>(lds + kKTileDw + kVtDw);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = blockIdx.x, split = blockIdx.y;
    const int hg = blockIdx.z * 4 + wave;
    const bool active = hg < (p.n_heads >> 4);
    const int lr = lane & 15, g = lane >> 4;
    const int head = hg * 16 + lr;

    const int n_tiles = (p.k + kTile - 1) / kTile;
    const int t_lo = split * p.tiles_per_split;
    const int t_hi = min(n_tiles, t_lo + p.tiles_per_split);
    const int e_lo = t_lo * kTile;
    const int e_hi = min(p.k, t_hi * kTile);

    // ---- queries: B operand of S^T = K Q^T.  Lane (lr, g) holds head lr,
    // dims 32ks + 8g .. +7 for ks = 0..17.
    half8_t qb[18];
    half8_t ql[QF32 ? 18 : 1];
    float score_mul = 0.0f;
    if (active) {
        const int64_t qoff = (int64_t)r * p.q_row_stride + (int64_t)head * p.q_head_stride + 8 * g;
        float qmax = 0.0f;
        if constexpr (QF32) {
            const float *qp = reinterpret_cast<const float *>(p.q) + qoff;
            float4 raw[36];
#pragma unroll
            for (int ks = 0; ks < 18; ++ks) {
                raw[2 * ks] = *reinterpret_cast<const float4 *>(qp + 32 * ks);
                raw[2 * ks + 1] = *reinterpret_cast<const float4 *>(qp + 32 * ks + 4);
            }
#pragma unroll
            for (int i = 0; i < 36; ++i)
                qmax = __builtin_fmaxf(qmax, __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(raw[i].x), __builtin_fabsf(raw[i].y)),
                                                             __builtin_fmaxf(__builtin_fabsf(raw[i].z), __builtin_fabsf(raw[i].w))));
            qmax = __builtin_fmaxf(qmax, __shfl_xor(qmax, 16));
            qmax = __builtin_fmaxf(qmax, __shfl_xor(qmax, 32));
            int ex = 0;
            if (qmax > 0.0f) (void)__builtin_frexpf(qmax, &ex);
            const float qs = __builtin_ldexpf(1.0f, 14 - ex);     // qmax * qs < 2^14
#pragma unroll
            for (int ks = 0; ks < 18; ++ks) {
                const float v[8] = {raw[2 * ks].x, raw[2 * ks].y, raw[2 * ks].z, raw[2 * ks].w,
                                    raw[2 * ks + 1].x, raw[2 * ks + 1].y, raw[2 * ks + 1].z, raw[2 * ks + 1].w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = v[e] * qs;
                    const _Float16 hi = (_Float16)x;
                    qb[ks][e] = hi;
                    ql[ks][e] = (_Float16)(x - (float)hi);
                }
            }
            score_mul = p.score_mul / qs;
        } else {
            const uint16_t *qp = reinterpret_cast<const uint16_t *>(p.q) + qoff;
            u32x4_t raw[18];
#pragma unroll
            for (int ks = 0; ks < 18; ++ks) raw[ks] = *reinterpret_cast<const u32x4_t *>(qp + 32 * ks);
#pragma unroll
            for (int ks = 0; ks < 18; ++ks)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const uint32_t w = raw[ks][c];
                    qmax = __builtin_fmaxf(qmax, __builtin_fmaxf(__builtin_fabsf(__uint_as_float(w << 16)),
                                                                 __builtin_fabsf(__uint_as_float(w & 0xFFFF0000u))));
                }
            qmax = __builtin_fmaxf(qmax, __shfl_xor(qmax, 16));
            qmax = __builtin_fmaxf(qmax, __shfl_xor(qmax, 32));
            int ex = 0;
            if (qmax > 0.0f) (void)__builtin_frexpf(qmax, &ex);
            const float qs = __builtin_ldexpf(1.0f, 14 - ex);
#pragma unroll
            for (int ks = 0; ks < 18; ++ks)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const uint32_t w = raw[ks][c];
                    qb[ks][2 * c] = (_Float16)(__uint_as_float(w << 16) * qs);
                    qb[ks][2 * c + 1] = (_Float16)(__uint_as_float(w & 0xFFFF0000u) * qs);
                }
            score_mul = p.score_mul / qs;
        }
    }

    floatx4_t o[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) o[i] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = -__builtin_inff();
    float l_run = 0.0f;
    uint32_t err = 0;

    const int32_t req = p.row_req ? p.row_req[r] : r;
    const bool bad_req = p.page_table && (req < 0 || req >= p.pt_n_rows);
    const int32_t *pt_row = p.page_table && !bad_req ? p.page_table + (int64_t)req * p.pt_row_stride : nullptr;
    const int32_t *list = p.topk + (int64_t)r * p.topk_row_stride;

    // gather lane roles
    const int pp = tid & 15;          // rows 2pp, 2pp+1 of the tile
    const int qc = tid >> 4;          // 16-byte code chunk: latent dims 32qc..32qc+31
    const int rope_row = tid >> 2;    // tid < 128: rope bytes 16*(tid&3).. of row tid>>2
    const int vt_dw_pair = vt_pair_dw(pp);

    u32x4_t ca, cb, rp;
    uint32_t sab;

    auto gather = [&](int tile) {
        const int32_t sa = slots[tile * kTile + 2 * pp];
        const int32_t sb = slots[tile * kTile + 2 * pp + 1];
        ca = u32x4_t{0, 0, 0, 0};
        cb = u32x4_t{0, 0, 0, 0};
        rp = u32x4_t{0, 0, 0, 0};
        uint32_t s0 = 0, s1 = 0;
        if (sa >= 0) {
            const uint8_t *row = p.pool + (int64_t)sa * kRowBytes;
            ca = *reinterpret_cast<const u32x4_t *>(row + 16 * qc);
            s0 = *reinterpret_cast<const uint16_t *>(row + kScaleOff + 2 * qc);
        }
        if (sb >= 0) {
            const uint8_t *row = p.pool + (int64_t)sb * kRowBytes;
            cb = *reinterpret_cast<const u32x4_t *>(row + 16 * qc);
            s1 = *reinterpret_cast<const uint16_t *>(row + kScaleOff + 2 * qc);
        }
        sab = s0 | (s1 << 16);
        if (tid < 128) {
            const int32_t sr = slots[tile * kTile + rope_row];
            if (sr >= 0)
                rp = *reinterpret_cast<const u32x4_t *>(p.pool + (int64_t)sr * kRowBytes + kRopeOff + 16 * (tid & 3));
        }
    };

    auto dequant_store = [&]() {
        const half2_t da0 = block_scale_half(sab & 0xFFu), da1 = block_scale_half((sab >> 8) & 0xFFu);
        const half2_t db0 = block_scale_half((sab >> 16) & 0xFFu), db1 = block_scale_half(sab >> 24);
        uint32_t *ka_row = ktile + (2 * pp) * kKPitchDw + 16 * qc;
        uint32_t *kb_row = ka_row + kKPitchDw;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            uint32_t ka[4], kb[4];
            e2m1x8_to_half(ca[c], c < 2 ? da0 : da1, ka);
            e2m1x8_to_half(cb[c], c < 2 ? db0 : db1, kb);
            *reinterpret_cast<u32x4_t *>(ka_row + 4 * c) = u32x4_t{ka[0], ka[1], ka[2], ka[3]};
            *reinterpret_cast<u32x4_t *>(kb_row + 4 * c) = u32x4_t{kb[0], kb[1], kb[2], kb[3]};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d0 = 32 * qc + 8 * c + 2 * i;
                vt[vt_addr(d0, vt_dw_pair)] = __builtin_amdgcn_perm(kb[i], ka[i], 0x05040100u);
                vt[vt_addr(d0 + 1, vt_dw_pair)] = __builtin_amdgcn_perm(kb[i], ka[i], 0x07060302u);
            }
        }
        if (tid < 128) {
            uint32_t h[8];
            dequant_rope16(rp, h);
            uint32_t *dst = ktile + rope_row * kKPitchDw + kLatent / 2 + 8 * (tid & 3);
            *reinterpret_cast<u32x4_t *>(dst) = u32x4_t{h[0], h[1], h[2], h[3]};
            *reinterpret_cast<u32x4_t *>(dst + 4) = u32x4_t{h[4], h[5], h[6], h[7]};
        }
    };

    const _Float16 *kth = reinterpret_cast<const _Float16 *>(ktile);

    for (int c_lo = e_lo; c_lo < e_hi; c_lo += kSlotCap) {
        const int c_hi = min(e_hi, c_lo + kSlotCap);
        const int n_t = (c_hi - c_lo + kTile - 1) / kTile;
        __syncthreads();                               // slots of the previous chunk are no longer read
        for (int e = tid; e < n_t * kTile; e += 256) {
            int64_t s = -1;
            if (c_lo + e < c_hi) {
                const int32_t pos = list[c_lo + e];
                if (bad_req) err |= pos >= 0 ? kErrPage : 0u;
                else s = translate_slot(pos, pt_row, p.pt_n_pages, p.page_shift, p.n_slots, err);
            }
            slots[e] = (int32_t)s;
        }
        __syncthreads();
        gather(0);
        for (int tt = 0; tt < n_t; ++tt) {
            dequant_store();
            const bool valid_lane = lane < kTile && slots[tt * kTile + lane] >= 0;
            const uint64_t vmask = __ballot(valid_lane);
            __syncthreads();
            if (tt + 1 < n_t) gather(tt + 1);
            if (active) {
                // ---- scores S^T[32 rows x 16 heads]
                floatx4_t s0a = {0, 0, 0, 0}, s0b = {0, 0, 0, 0}, s1a = {0, 0, 0, 0}, s1b = {0, 0, 0, 0};
#pragma unroll
                for (int ks = 0; ks < 18; ++ks) {
                    const half8_t a0 = *reinterpret_cast<const half8_t *>(kth + lr * kKPitchHalf + 32 * ks + 8 * g);
                    const half8_t a1 = *reinterpret_cast<const half8_t *>(kth + (16 + lr) * kKPitchHalf + 32 * ks + 8 * g);
                    if (ks & 1) {
                        s0b = mfma16(a0, qb[ks], s0b);
                        s1b = mfma16(a1, qb[ks], s1b);
                        if constexpr (QF32) {
                            s0a = mfma16(a0, ql[ks], s0a);
                            s1a = mfma16(a1, ql[ks], s1a);
                        }
                    } else {
                        s0a = mfma16(a0, qb[ks], s0a);
                        s1a = mfma16(a1, qb[ks], s1a);
                        if constexpr (QF32) {
                            s0b = mfma16(a0, ql[ks], s0b);
                            s1b = mfma16(a1, ql[ks], s1b);
                        }
                    }
                }
                const floatx4_t s0 = s0a + s0b, s1 = s1a + s1b;
                // ---- online softmax (base 2).  Lane holds rows 4g+i and 16+4g+i of head lr.
                float sc[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int ra = 4 * g + i, rb = 16 + 4 * g + i;
                    sc[i] = ((vmask >> ra) & 1) ? s0[i] * score_mul : -__builtin_inff();
                    sc[4 + i] = ((vmask >> rb) & 1) ? s1[i] * score_mul : -__builtin_inff();
                }
                float tmax = sc[0];
#pragma unroll
                for (int i = 1; i < 8; ++i) tmax = __builtin_fmaxf(tmax, sc[i]);
                tmax = __builtin_fmaxf(tmax, __shfl_xor(tmax, 16));
                tmax = __builtin_fmaxf(tmax, __shfl_xor(tmax, 32));
                const bool need = tmax > m_run + kRescaleSlack;
                if (__any(need)) {
                    const float m_new = need ? tmax : m_run;
                    const float alpha = m_new == m_run ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
                    l_run *= alpha;
#pragma unroll
                    for (int i = 0; i < 32; ++i) o[i] *= alpha;
                    m_run = m_new;
                }
                half8_t pb;
                float lsum = 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float pv = sc[i] == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(sc[i] - m_run);
                    lsum += pv;
                    pb[i] = (_Float16)pv;
                }
                l_run += lsum;
                // ---- O^T[512 x 16] += V^T[512 x 32] P^T[32 x 16]
#pragma unroll
                for (int md = 0; md < 32; ++md) {
                    const int d = 16 * md + lr;
                    const half8_t a = *reinterpret_cast<const half8_t *>(vt + vt_addr(d, 4 * g));
                    o[md] = mfma16(a, pb, o[md]);
                }
            }
            __syncthreads();
        }
    }

    if (err && p.err_word) atomicOr(p.err_word, err);
    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    if (!active) return;
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    float *orow = p.out + (int64_t)split * p.out_split_stride + (int64_t)r * p.out_row_stride + (int64_t)head * kLatent;
#pragma unroll
    for (int md = 0; md < 32; ++md) *reinterpret_cast<floatx4_t *>(orow + 16 * md + 4 * g) = o[md] * inv;
    if (g == 0 && p.lse) {
        const float lse = l_tot > 0.0f ? (m_run + __builtin_log2f(l_tot)) * 0.69314718055994530942f : -__builtin_inff();
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
