// Quantized row write with MSE-searched block scales (README "60+ inference
// optimizations & kernels", section "4-bit KV cache": the DeepSeek V4 Pro
// pools quantize with an MSE-searched scale).
//
// Every finite non-negative E4M3 scale d is a candidate.  A block's error
// under d is the fp32 sum, in index order, of (x - c d)^2 over its 16 values,
// one fused multiply-add per value, where c is the E2M1 code of the fp32
// quotient x / d (no code when d = 0).  The amax/6 scale stays unless a
// candidate is strictly better; among better ones the smallest code wins.
//
// One lane per block of 16 values, two rows per wavefront: lanes 32h..32h+31
// hold the 32 blocks of row 2w + h.  A candidate is d = (1 + m/8) 2^e, and
// x / d = (x / (1 + m/8)) 2^-e exactly whenever that is a normal float; where
// it is not (a quotient under 2^-117 or past the fp32 range) both forms give
// the same code (zero, or saturation at 6).  So a lane divides its values by
// the eight mantissas once, and the conversion to FP4 applies 2^-e.
// Candidates that cannot be chosen are not evaluated:
//  * below: when 6d <= amax, the block's largest value errs by at least
//    amax - 6d under d, and an fp32 sum of squares never falls below one of
//    its terms, so fl(fl(amax - 6d)^2) >= the amax/6 error rules d out;
//  * above: once amax / 2^e < 1/4 every code is zero for every mantissa and
//    the error no longer depends on d, so only the smallest such code, which
//    lies at or below exponent e, can be chosen; and a d that codes a set of
//    the smallest values as zero while their squares alone reach the amax/6
//    error is ruled out too.
#include "kv4_quant_impl.h"
#include "kv4_launch.h"

namespace kv4 {

typedef float float2_t __attribute__((ext_vector_type(2)));

constexpr int kMseThreads = 256;
constexpr int kMseRowsPerBlock = kMseThreads / 32;

// Sixteen E2M1 codes (w0: values 0..7, w1: 8..15, code i in bits 4i..4i+3)
// -> their values, exactly, with gfx950's FP4 -> fp32 conversion at scale 1.
__device__ __forceinline__ void e2m1x8_to_float(uint32_t w, float c[8]) {
    const float2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    const float2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    const float2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    const float2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    c[0] = v0.x;
    c[1] = v0.y;
    c[2] = v1.x;
    c[3] = v1.y;
    c[4] = v2.x;
    c[5] = v2.y;
    c[6] = v3.x;
    c[7] = v3.y;
}

__device__ __forceinline__ void e2m1x16_to_float(uint32_t w0, uint32_t w1, float c[16]) {
    e2m1x8_to_float(w0, c);
    e2m1x8_to_float(w1, c + 8);
}

// fp32 squared error of the block x[16] coded as (w0, w1) at scale d:
// sum over i in order of e_i^2, e_i = x_i - c_i d (c_i d is exact, so one
// fused multiply-add forms the rounded difference).
__device__ __forceinline__ float block_sq_error(const float x[16], uint32_t w0, uint32_t w1, float d) {
    float c[16];
    e2m1x16_to_float(w0, w1, c);
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float e = __builtin_fmaf(-c[i], d, x[i]);
        s = __builtin_fmaf(e, e, s);
    }
    return s;
}

// E4M3 code of the candidate (1 + m/8) 2^e, or -1 when that value is not an
// E4M3 scale (exponent range [-9, 8]; subnormals are multiples of 2^-9).
__device__ __forceinline__ int e4m3_candidate_code(int m, int e) {
    if (e >= -6 && e <= 8) return (m == 7 && e == 8) ? -1 : (e + 7) * 8 + m;
    if (e == -9) return m == 0 ? 1 : -1;
    if (e == -8) return (m & 3) == 0 ? (8 + m) >> 2 : -1;
    if (e == -7) return (m & 1) == 0 ? (8 + m) >> 1 : -1;
    return -1;
}

// Exponent of the E4M3 value of code k (0 < k <= 0x7E): d = (1 + m/8) 2^e.
__device__ __forceinline__ int e4m3_code_exponent(uint32_t k) {
    if (k >= 8) return (int)(k >> 3) - 7;
    return (31 - __builtin_clz(k)) - 9;
}

// The correctly rounded quotient x / mult for mult = 1 + m/8 from the
// rounded reciprocal r and one fused correction: q0 = x r, the residual
// x - q0 mult is exact, and q0 + residual r rounds to the same float as the
// quotient for every x in [1, 2) and each of the eight divisors (checked
// exhaustively), hence for every normal x, since each step commutes with
// scaling by powers of two.  The sign is restored for zeros (+0 from the
// residual).  For subnormal x the result can differ from the quotient, but
// both code as zero of x's sign at every candidate scale.
__device__ __forceinline__ float quotient(float x, float mult, float r) {
    const float q0 = x * r;
    const float rem = __builtin_fmaf(-q0, mult, x);
    return __builtin_copysignf(__builtin_fmaf(rem, r, q0), x);
}

// E2M1 codes of q[i] / scale for a power-of-two scale (gfx950's fp32 -> FP4
// conversion divides by the scale exactly before rounding, so this equals the
// codes of the products q[i] * (1 / scale) at scale 1).
__device__ __forceinline__ uint32_t e2m1x8_div_pow2(const float q[8], float scale) {
    uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, q[0], q[1], scale, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[2], q[3], scale, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[4], q[5], scale, 2);
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[6], q[7], scale, 3);
}

// Ascending sort of 16 values (Batcher's odd-even merge network; all indices
// are compile-time constants, so the values stay in registers).
__device__ __forceinline__ void sort16(float v[16]) {
#pragma unroll
    for (int p = 1; p < 16; p <<= 1) {
#pragma unroll
        for (int k = p; k >= 1; k >>= 1) {
#pragma unroll
            for (int j = k % p; j + k < 16; j += 2 * k) {
#pragma unroll
                for (int i = 0; i < k; ++i) {
                    const int lo = i + j, hi = i + j + k;
                    if (hi < 16 && lo / (2 * p) == hi / (2 * p)) {
                        const float a = v[lo], b = v[hi];
                        v[lo] = __builtin_fminf(a, b);
                        v[hi] = __builtin_fmaxf(a, b);
                    }
                }
            }
        }
    }
}

__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
    return v;
}

template <bool ROPE>
__global__ __launch_bounds__(kMseThreads) void quant_write_mse_kernel(const float *__restrict__ kv,
                                                                       int64_t kv_row_stride,
                                                                       const int32_t *__restrict__ slots,
                                                                       int64_t n_tokens, uint8_t *__restrict__ pool,
                                                                       int64_t n_slots,
                                                                       uint32_t *__restrict__ err_word) {
    const int lane = threadIdx.x & 63;
    const int b = lane & 31;                                   // block of the row
    const int64_t row = (int64_t)blockIdx.x * kMseRowsPerBlock + (threadIdx.x >> 5);
    const bool in_range = row < n_tokens;
    // Every lane stays to the end: the cross-lane reads below span the wave.
    int32_t slot = -1;
    float x[16] = {};
    float r0 = 0.0f, r1 = 0.0f;
    if (in_range) {
        slot = slots[row];
        const float *src = kv + row * kv_row_stride;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float4 v = *reinterpret_cast<const float4 *>(src + 16 * b + 4 * j);
            x[4 * j] = v.x;
            x[4 * j + 1] = v.y;
            x[4 * j + 2] = v.z;
            x[4 * j + 3] = v.w;
        }
        if (ROPE) {
            const float2 rv = *reinterpret_cast<const float2 *>(src + kLatent + 2 * b);
            r0 = rv.x;
            r1 = rv.y;
        }
    }
    if (in_range && slot >= 0 && (int64_t)slot >= n_slots && b == 0 && err_word) atomicOr(err_word, kErrSlot);
    const bool live = in_range && slot >= 0 && (int64_t)slot < n_slots;

    // the amax/6 scale and its codes (NaN is no block's maximum)
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(x[i]));
    const uint32_t k0 = e4m3_encode_hw(amax / 6.0f);
    const float d0 = e4m3_pos_to_float(k0);
    uint32_t best_w0 = 0, best_w1 = 0;
    if (d0 != 0.0f) {
        best_w0 = e2m1x8_of_quotients(x, d0);
        best_w1 = e2m1x8_of_quotients(x + 8, d0);
    }
    const float err0 = block_sq_error(x, best_w0, best_w1, d0);
    float best_err = err0;
    int best_k = (int)k0;
    // NaN (a NaN value), +inf (an infinite or huge value) and 0 cannot be beaten
    const bool search = live && err0 > 0.0f && err0 < __builtin_inff();

    // scale 0: every code zero, error = the plain sum of squares
    if (search && amax * amax < err0) {
        const float e = block_sq_error(x, 0u, 0u, 0.0f);
        if (e < best_err) {
            best_err = e;
            best_k = 0;
            best_w0 = best_w1 = 0;
        }
    }

    // Candidates ruled out without evaluating them (each test is exact):
    //  * 6d <= amax and fl(fl(amax - 6d)^2) >= err0 (the largest value's error);
    //  * d >= 4a, with a the least magnitude whose values up to it have squares
    //    summing to err0 or more (with margin for fp32 rounding): d codes all
    //    of them as zero, so its error sum holds those squares unchanged;
    //  * exponents from e_hi on (amax < 2^(e_hi - 2)) when no such a exists:
    //    every code is zero there and the error no longer depends on d, so
    //    only the smallest such code, at or below e_hi, can be chosen.
    // For a fixed mantissa the survivors are one run of exponents, since the
    // first test rules out a prefix and the others a suffix; each lane walks
    // its own run, so a wavefront iterates over the longest run, not over the
    // union of its lanes' exponent ranges.
    int e_up = -100;
    float four_a = __builtin_inff();
    if (search) {
        int E;
        __builtin_frexpf(amax, &E);                          // amax = f 2^E, f in [0.5, 1)
        e_up = min(E + 2, 8);
        float mag[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) mag[i] = __builtin_fabsf(x[i]);
        sort16(mag);
        const float need = err0 * (1.0f + 0x1p-16f);
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            acc = __builtin_fmaf(mag[i], mag[i], acc);
            if (acc >= need && four_a == __builtin_inff()) four_a = 4.0f * mag[i];
        }
        if (four_a < __builtin_inff()) {
            int F;
            __builtin_frexpf(four_a, &F);                    // 4a < 2^F: every d with e >= F is >= 4a
            e_up = min(e_up, F - 1);
        }
    }
    // a lower start for the runs: below e_lo, 6d <= (amax - 1.01 sqrt(err0)) / 8
    // for every mantissa, far enough under amax - sqrt(err0) that the first
    // test rules d out (rounding included)
    int e_lo = -9;
    if (search) {
        const float t = (amax - 1.01f * __builtin_sqrtf(err0)) * (1.0f / 11.25f);
        if (t > 0.0f) {
            int Et;
            __builtin_frexpf(t, &Et);                        // t >= 2^(Et - 1)
            e_lo = max(-9, Et - 3);
        }
    }

    if (__builtin_amdgcn_ballot_w64(search)) {
        for (int m = 0; m < 8; ++m) {
            const float mult = 1.0f + 0.125f * (float)m;
            const float r = 1.0f / mult;                     // rounded reciprocal
            // this lane's run [e_a, e_b] for mantissa m
            int e_a = e_lo, e_b = e_up;
            if (search) {
                while (e_a <= e_b) {
                    const float six_d = 6.0f * __builtin_ldexpf(mult, e_a);
                    const float gap = amax - six_d;
                    if (!(six_d <= amax && gap * gap >= err0)) break;
                    ++e_a;
                }
                while (e_b >= e_a && four_a <= __builtin_ldexpf(mult, e_b)) --e_b;
            }
            const int n_run = search ? max(e_b - e_a + 1, 0) : 0;
            const int n_it = wave_max(n_run);
            if (n_it == 0) continue;
            float q[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) q[i] = quotient(x[i], mult, r);
            for (int it = 0; it < n_it; ++it) {
                const int e = e_a + it;
                const int k = it < n_run ? e4m3_candidate_code(m, e) : -1;
                if (k < 0) continue;
                const float d = __builtin_ldexpf(mult, e);
                const float scale = __builtin_ldexpf(1.0f, e);
                const uint32_t w0 = e2m1x8_div_pow2(q, scale), w1 = e2m1x8_div_pow2(q + 8, scale);
                const float err = block_sq_error(x, w0, w1, d);
                if (err < best_err || (err == best_err && best_k != (int)k0 && k < best_k)) {
                    best_err = err;
                    best_k = k;
                    best_w0 = w0;
                    best_w1 = w1;
                }
            }
        }
    }

    // Lanes with b % 4 == 0 gather the scale bytes of blocks b..b+3, lanes
    // with b even the rope bytes 2b..2b+3; all reads stay inside the row's
    // half of the wave.
    const uint32_t rope2 = ROPE ? (e4m3_encode_hw(r0) | (e4m3_encode_hw(r1) << 8)) : 0u;
    const uint32_t sc = (uint32_t)best_k;
    const uint32_t s1 = __shfl(sc, (lane + 1) & 63), s2 = __shfl(sc, (lane + 2) & 63),
                   s3 = __shfl(sc, (lane + 3) & 63);
    const uint32_t rn = __shfl(rope2, (lane + 1) & 63);
    if (!live) return;
    uint8_t *dst = pool + (int64_t)slot * (ROPE ? kRowBytes : kScaleOff + kLatent / 16);
    *reinterpret_cast<uint2 *>(dst + 8 * b) = make_uint2(best_w0, best_w1);
    if ((b & 3) == 0)
        *reinterpret_cast<uint32_t *>(dst + kScaleOff + b) = sc | (s1 << 8) | (s2 << 16) | (s3 << 24);
    if (ROPE && (b & 1) == 0) *reinterpret_cast<uint32_t *>(dst + kRopeOff + 2 * b) = rope2 | (rn << 16);
}

hipError_t launch_quant_write_mse(const float *kv, int64_t kv_row_stride, const int32_t *slots, int64_t n_tokens,
                                  uint8_t *pool, int64_t n_slots, bool rope, uint32_t *err_word,
                                  hipStream_t stream) {
    if (n_tokens == 0) return hipSuccess;
    const int64_t blocks = (n_tokens + kMseRowsPerBlock - 1) / kMseRowsPerBlock;
    if (rope)
        hipLaunchKernelGGL(quant_write_mse_kernel<true>, dim3((unsigned)blocks), dim3(kMseThreads), 0, stream, kv,
                           kv_row_stride, slots, n_tokens, pool, n_slots, err_word);
    else
        hipLaunchKernelGGL(quant_write_mse_kernel<false>, dim3((unsigned)blocks), dim3(kMseThreads), 0, stream, kv,
                           kv_row_stride, slots, n_tokens, pool, n_slots, err_word);
    return hipGetLastError();
}

}  // namespace kv4
