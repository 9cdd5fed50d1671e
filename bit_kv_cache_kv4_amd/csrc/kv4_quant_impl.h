// Quantized KV row write, one row per wavefront (README "60+ inference
// optimizations & kernels", section "4-bit KV cache": the quantized write of
// 352-byte NVFP4 rows).
//
// One wavefront per token row.  Lane l owns latent dims 8l..8l+7 (half of
// block l/2) and rope dim 512+l.  The block amax is one max across the lane
// pair (l, l^1); the scale is the E4M3 code nearest to the fp32 quotient
// amax/6; the eight codes of a lane pack into one dword, so the 256 code bytes
// leave as one coalesced 64-lane dword store.  Scale and rope bytes are packed
// four to a dword with cross-lane reads and stored by lanes 0..23.
#pragma once

#include "kv4_device.h"

namespace kv4 {

typedef short short2_t __attribute__((ext_vector_type(2)));

// E4M3 code of x with gfx950's conversion: its rounding is nearest, ties to
// even, and it keeps the sign of zero, as e4m3_encode; it does not saturate
// (beyond 464 it gives NaN), so x is clamped to +-448 first, and NaN gives
// 0x7F as in e4m3_encode.
__device__ __forceinline__ uint32_t e4m3_encode_hw(float x) {
    const float c = __builtin_fminf(__builtin_fmaxf(x, -448.0f), 448.0f);
    const short2_t z = {0, 0};
    const uint32_t code = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, c, c, 1.0f, false)) & 0xFFu;
    return x == x ? code : 0x7Fu;
}

// Eight E2M1 codes (code i in bits 4i..4i+3) of the values y[i], with
// gfx950's fp32 -> FP4 conversion at scale 1, which rounds like e2m1_encode
// (nearest, ties to the even code, saturation at 6, sign kept) for every
// input but NaN.
__device__ __forceinline__ uint32_t e2m1x8_hw(const float y[8]) {
    uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y[0], y[1], 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2], y[3], 1.0f, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[4], y[5], 1.0f, 2);
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[6], y[7], 1.0f, 3);
}

// E2M1 codes (code i in bits 4i..4i+3) of the eight fp32 quotients x[i] / d,
// d > 0, without eight divisions: with rd the hardware reciprocal of d (within
// 1 ulp), q = x * rd is within 2^-22 of the rounded quotient, relatively, so
// when q nudged 2^-20 down and up gives the same codes, so does the quotient
// (the conversion is monotone in magnitude and the nudge spans that gap).
// Otherwise (a quotient at or next to a rounding midpoint), or with a NaN
// present, the lane divides.
__device__ __forceinline__ uint32_t e2m1x8_of_quotients(const float x[8], float d) {
    const float rd = __builtin_amdgcn_rcpf(d);
    float lo[8], hi[8], sum = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float q = x[i] * rd;
        lo[i] = q * (1.0f - 0x1p-20f);
        hi[i] = q * (1.0f + 0x1p-20f);
        sum += x[i];
    }
    uint32_t word = e2m1x8_hw(lo);
    if (word != e2m1x8_hw(hi) || sum != sum) {
        word = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) word |= e2m1_encode(x[i] / d) << (4 * i);
    }
    return word;
}

// Row `row` written by one wavefront (lane = its lane index).  ROPE: the
// 352-byte row from 576 values; otherwise the 288-byte rope-free row (codes
// and scales) from 512.
template <bool ROPE = true>
__device__ __forceinline__ void quant_write_row(const float *__restrict__ kv, int64_t kv_row_stride,
                                                const int32_t *__restrict__ slots, int64_t n_tokens,
                                                uint8_t *__restrict__ pool, int64_t n_slots,
                                                uint32_t *__restrict__ err_word, int64_t row, int lane) {
    if (row >= n_tokens) return;                 // uniform across the wave
    // the row's values are loaded together with its slot (not after it)
    const int32_t slot = slots[row];
    const float *src = kv + row * kv_row_stride;
    const float4 v0 = *reinterpret_cast<const float4 *>(src + 8 * lane);
    const float4 v1 = *reinterpret_cast<const float4 *>(src + 8 * lane + 4);
    const float r = ROPE ? src[kLatent + lane] : 0.0f;
    if (slot < 0) return;                        // pad row: writes nothing
    if ((int64_t)slot >= n_slots) {
        if (lane == 0 && err_word) atomicOr(err_word, kErrSlot);
        return;
    }
    const float x[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};

    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(x[i]));
    amax = __builtin_fmaxf(amax, __shfl_xor(amax, 1));

    const uint32_t s = e4m3_encode_hw(amax / 6.0f);        // IEEE fp32 division; amax / 6 is never NaN
    const float d = e4m3_pos_to_float(s);
    const uint32_t word = d != 0.0f ? e2m1x8_of_quotients(x, d) : 0u;
    const uint32_t rc = e4m3_encode_hw(r);

    // Lane m < 8 gathers the scales of blocks 4m..4m+3 (held by lanes
    // 8m, 8m+2, 8m+4, 8m+6); lane 8 + m (m < 16) gathers the rope codes of
    // lanes 4m..4m+3.
    const uint32_t both = s | (rc << 8);
    int src_lane[4];
    const bool is_scale = lane < 8;
    const int m = is_scale ? lane : lane - 8;
#pragma unroll
    for (int j = 0; j < 4; ++j) src_lane[j] = (is_scale ? 8 * m + 2 * j : 4 * m + j) & 63;
    uint32_t packed = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t t = __shfl(both, src_lane[j]);
        packed |= ((is_scale ? t : (t >> 8)) & 0xFFu) << (8 * j);
    }

    uint8_t *dst = pool + (int64_t)slot * (ROPE ? kRowBytes : kScaleOff + kLatent / 16);
    reinterpret_cast<uint32_t *>(dst)[lane] = word;
    if (lane < 8) reinterpret_cast<uint32_t *>(dst + kScaleOff)[lane] = packed;
    else if (ROPE && lane < 24) reinterpret_cast<uint32_t *>(dst + kRopeOff)[lane - 8] = packed;
}

}  // namespace kv4
