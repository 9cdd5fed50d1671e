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
