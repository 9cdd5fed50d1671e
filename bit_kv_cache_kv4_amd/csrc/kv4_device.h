// Device-side helpers shared by the kv4 HIP kernels (gfx950 only).
//
// Row format (README "60+ inference optimizations & kernels", section "4-bit
// KV cache"): 352 bytes = 256 bytes of E2M1 codes (two per byte, even dim in
// the low nibble) + 32 E4M3 block scales (one per 16 latent dims) + 64 E4M3
// rope values.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kv4 {

constexpr int kLatent = 512;
constexpr int kRope = 64;
constexpr int kDim = 576;
constexpr int kRowBytes = 352;
constexpr int kScaleOff = 256;
constexpr int kRopeOff = 288;

constexpr uint32_t kErrPage = 1u;
constexpr uint32_t kErrSlot = 2u;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- encoders

// Nearest OCP E4M3 ("fn") code of x: round to nearest, ties to the even
// mantissa, magnitudes >= 448 saturate to 448, the sign bit follows x (also
// for zero).  NaN gives 0x7F.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
    const uint32_t bits = __float_as_uint(x);
    const uint32_t sign = (bits >> 24) & 0x80u;
    const float a = __builtin_fabsf(x);
    uint32_t code;
    if (!(a == a)) return 0x7Fu;
    if (a >= 448.0f) {
        code = 0x7Eu;
    } else if (a < 0.015625f) {
        // Below the smallest normal (2^-6) the codes step by 2^-9: scale by
        // 2^9 (exact) and round half to even.  A result of 8 is 2^-6, code 8.
        code = (uint32_t)__builtin_rintf(a * 512.0f);
    } else {
        // Normal range: keep 3 mantissa bits with round-half-even on the fp32
        // pattern; a carry moves into the exponent.  Rebias 127 -> 7.
        uint32_t b = __float_as_uint(a);
        b += 0x7FFFFu + ((b >> 20) & 1u);
        code = (b >> 20) - (120u << 3);
    }
    return code | sign;
}

// Exact value of a non-negative E4M3 code c (0 <= c <= 0x7E) as fp32.
__device__ __forceinline__ float e4m3_pos_to_float(uint32_t c) {
    const uint32_t e = c >> 3, m = c & 7u;
    if (e == 0) return (float)m * 0.001953125f;   // m * 2^-9
    return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// Exact value of an E4M3 code with its sign (0x7F/0xFF, the NaN codes, are
// never written by the quantizer; they read as +-480 here).
__device__ __forceinline__ float e4m3_to_float(uint32_t c) {
    const float v = e4m3_pos_to_float(c & 0x7Fu);
    return (c & 0x80u) ? -v : v;
}

// Nearest E2M1 code of y: magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}; at a tie the
// even code wins (0.25->0, 0.75->1, 1.25->1, 1.75->2, 2.5->2, 3.5->4, 5->4);
// above 6 saturates to 6; the sign follows y.
__device__ __forceinline__ uint32_t e2m1_encode(float y) {
    const float a = __builtin_fabsf(y);
    const uint32_t mag = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                         (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                         (uint32_t)(a > 5.0f);
    return mag | ((__float_as_uint(y) >> 28) & 8u);
}

// ---------------------------------------------------------------- decoders

// fp16 bit patterns of the E2M1 magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6} have a
// zero low byte; their high bytes {00 38 3C 3E 40 42 44 46} form an 8-entry
// table for v_perm_b32 (selector 0..3 -> second operand, 4..7 -> first).
constexpr uint32_t kE2m1HiLo = 0x3E3C3800u;
constexpr uint32_t kE2m1HiHi = 0x46444240u;

// Eight E2M1 codes (one dword, code i in bits 4i..4i+3) -> four fp16 pairs
// (dims 2i, 2i+1), each multiplied by the block scale d.  Every product of an
// E2M1 value and an E4M3 scale is exact in fp16, so this loses nothing.
__device__ __forceinline__ void e2m1x8_to_half(uint32_t w, half2_t d, uint32_t out[4]) {
    const uint32_t me = w & 0x07070707u;          // magnitudes of even codes
    const uint32_t mo = (w >> 4) & 0x07070707u;   // magnitudes of odd codes
    const uint32_t he = __builtin_amdgcn_perm(kE2m1HiHi, kE2m1HiLo, me) | ((w << 4) & 0x80808080u);
    const uint32_t ho = __builtin_amdgcn_perm(kE2m1HiHi, kE2m1HiLo, mo) | (w & 0x80808080u);
    // pair i = [0x00, he.byte_i, 0x00, ho.byte_i]
    uint32_t p0 = __builtin_amdgcn_perm(ho, he, 0x040c000cu);
    uint32_t p1 = __builtin_amdgcn_perm(ho, he, 0x050c010cu);
    uint32_t p2 = __builtin_amdgcn_perm(ho, he, 0x060c020cu);
    uint32_t p3 = __builtin_amdgcn_perm(ho, he, 0x070c030cu);
    half2_t h0 = __builtin_bit_cast(half2_t, p0) * d;
    half2_t h1 = __builtin_bit_cast(half2_t, p1) * d;
    half2_t h2 = __builtin_bit_cast(half2_t, p2) * d;
    half2_t h3 = __builtin_bit_cast(half2_t, p3) * d;
    out[0] = __builtin_bit_cast(uint32_t, h0);
    out[1] = __builtin_bit_cast(uint32_t, h1);
    out[2] = __builtin_bit_cast(uint32_t, h2);
    out[3] = __builtin_bit_cast(uint32_t, h3);
}

// Same result as e2m1x8_to_half with gfx950's FP4 -> fp16 conversion at
// scale 1 (exact; the code byte's low nibble is the first element) followed by
// one packed multiply by the block scale.
__device__ __forceinline__ void e2m1x8_to_half_cvt(uint32_t w, half2_t d, uint32_t out[4]) {
    out[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * d);
    out[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * d);
    out[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * d);
    out[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * d);
}

// Four E4M3 codes -> two fp16 pairs with gfx950's FP8 (OCP E4M3) -> fp16
// conversion at scale 1, exact for every code.
__device__ __forceinline__ void e4m3x4_to_half_cvt(uint32_t w, uint32_t out[2]) {
    out[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
    out[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
}

// Two E4M3 codes (bytes lo, hi of a 16-bit field) -> fp16 pair, exact.
// Magnitude bits placed at fp16 bits 13..7 read as 2^-8 times the E4M3 value
// (subnormal codes become fp16 subnormals), so one multiply by 256 finishes.
__device__ __forceinline__ uint32_t e4m3x2_to_half(uint32_t two) {
    const uint32_t y = (two & 0xFFu) | ((two & 0xFF00u) << 8);        // bytes at 0 and 16
    const uint32_t bits = ((y & 0x007F007Fu) << 7) | ((y & 0x00800080u) << 8);
    const half2_t s = {(_Float16)256.0f, (_Float16)256.0f};
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, bits) * s);
}

// An E4M3 block scale as an fp16 pair (exact).
__device__ __forceinline__ half2_t block_scale_half(uint32_t code) {
    const _Float16 f = (_Float16)e4m3_to_float(code);
    return half2_t{f, f};
}

// Four E4M3 block scales (bytes of w) as four fp16 pairs {d_i, d_i}, with the
// FP8 -> fp16 conversion at scale 1 (exact for every code).
__device__ __forceinline__ void block_scales_half_cvt(uint32_t w, half2_t d[4]) {
    const half2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
    const half2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
    d[0] = __builtin_shufflevector(lo, lo, 0, 0);
    d[1] = __builtin_shufflevector(lo, lo, 1, 1);
    d[2] = __builtin_shufflevector(hi, hi, 0, 0);
    d[3] = __builtin_shufflevector(hi, hi, 1, 1);
}

// One row's 16-byte code chunk (latent dims 32c..32c+31) and its two block
// scales (bytes of `scales16`) -> 16 fp16 pairs in dim order.
__device__ __forceinline__ void dequant_chunk(u32x4_t codes, uint32_t scales16, uint32_t out[16]) {
    const half2_t d0 = block_scale_half(scales16 & 0xFFu), d1 = block_scale_half((scales16 >> 8) & 0xFFu);
    e2m1x8_to_half(codes[0], d0, out);
    e2m1x8_to_half(codes[1], d0, out + 4);
    e2m1x8_to_half(codes[2], d1, out + 8);
    e2m1x8_to_half(codes[3], d1, out + 12);
}

// 16 rope bytes -> 8 fp16 pairs in dim order.
__device__ __forceinline__ void dequant_rope16(u32x4_t bytes, uint32_t out[8]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        out[2 * c] = e4m3x2_to_half(bytes[c] & 0xFFFFu);
        out[2 * c + 1] = e4m3x2_to_half(bytes[c] >> 16);
    }
}

// ----------------------------------------------------------------- misc

// The same translation with the page-table entry already loaded (phys is
// pt_row[pos >> page_shift] when that page is inside the table).
__device__ __forceinline__ int64_t slot_of(int32_t pos, int32_t phys, bool paged, int32_t pt_n_pages,
                                           int32_t page_shift, int64_t n_slots, uint32_t &err) {
    if (pos < 0) return -1;
    int64_t slot;
    if (paged) {
        if ((pos >> page_shift) >= pt_n_pages || phys < 0) { err |= kErrPage; return -1; }
        slot = ((int64_t)phys << page_shift) + (pos & ((1 << page_shift) - 1));
    } else {
        slot = pos;
    }
    if (slot >= n_slots) { err |= kErrSlot; return -1; }
    return slot;
}

__device__ __forceinline__ int64_t translate_slot(int32_t pos, const int32_t *pt_row, int32_t pt_n_pages,
                                                  int32_t page_shift, int64_t n_slots, uint32_t &err) {
    if (pos < 0) return -1;
    int64_t slot;
    if (pt_row) {
        const int32_t page = pos >> page_shift;
        if (page >= pt_n_pages) { err |= kErrPage; return -1; }
        const int32_t phys = pt_row[page];
        if (phys < 0) { err |= kErrPage; return -1; }
        slot = ((int64_t)phys << page_shift) + (pos & ((1 << page_shift) - 1));
    } else {
        slot = pos;
    }
    if (slot >= n_slots) { err |= kErrSlot; return -1; }
    return slot;
}

}  // namespace kv4
