// Quantized KV row write (README "60+ inference optimizations & kernels",
// section "4-bit KV cache": the quantized write of 352-byte NVFP4 rows).
//
// One wavefront per token row.  Lane l owns latent dims 8l..8l+7 (half of
// block l/2) and rope dim 512+l.  The block amax is one max across the lane
// pair (l, l^1); the scale is the E4M3 code nearest to the fp32 quotient
// amax/6; the eight codes of a lane pack into one dword, so the 256 code bytes
// leave as one coalesced 64-lane dword store.  Scale and rope bytes are packed
// four to a dword with cross-lane reads and stored by lanes 0..23.
#include "kv4_device.h"
#include "kv4_launch.h"

namespace kv4 {

constexpr int kQuantRowsPerBlock = 4;   // 4 waves of 64 lanes

__global__ __launch_bounds__(256) void quant_write_kernel(const float *__restrict__ kv, int64_t kv_row_stride,
                                                          const int32_t *__restrict__ slots, int64_t n_tokens,
                                                          uint8_t *__restrict__ pool, int64_t n_slots,
                                                          uint32_t *__restrict__ err_word) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kQuantRowsPerBlock + (threadIdx.x >> 6);
    if (row >= n_tokens) return;                 // uniform across the wave
    const int32_t slot = slots[row];
    if (slot < 0) return;                        // pad row: writes nothing
    if ((int64_t)slot >= n_slots) {
        if (lane == 0 && err_word) atomicOr(err_word, kErrSlot);
        return;
    }
    const float *src = kv + row * kv_row_stride;
    const float4 v0 = *reinterpret_cast<const float4 *>(src + 8 * lane);
    const float4 v1 = *reinterpret_cast<const float4 *>(src + 8 * lane + 4);
    const float r = src[kLatent + lane];
    const float x[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};

    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(x[i]));
    amax = __builtin_fmaxf(amax, __shfl_xor(amax, 1));

    const uint32_t s = e4m3_encode(amax / 6.0f);          // IEEE fp32 division
    const float d = e4m3_pos_to_float(s);
    uint32_t word = 0;
    if (d != 0.0f) {
#pragma unroll
        for (int i = 0; i < 8; ++i) word |= e2m1_encode(x[i] / d) << (4 * i);
    }
    const uint32_t rc = e4m3_encode(r);

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

    uint8_t *dst = pool + (int64_t)slot * kRowBytes;
    reinterpret_cast<uint32_t *>(dst)[lane] = word;
    if (lane < 8) reinterpret_cast<uint32_t *>(dst + kScaleOff)[lane] = packed;
    else if (lane < 24) reinterpret_cast<uint32_t *>(dst + kRopeOff)[lane - 8] = packed;
}

hipError_t launch_quant_write(const float *kv, int64_t kv_row_stride, const int32_t *slots, int64_t n_tokens,
                              uint8_t *pool, int64_t n_slots, uint32_t *err_word, hipStream_t stream) {
    if (n_tokens == 0) return hipSuccess;
    const int64_t blocks = (n_tokens + kQuantRowsPerBlock - 1) / kQuantRowsPerBlock;
    hipLaunchKernelGGL(quant_write_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, kv, kv_row_stride,
                       slots, n_tokens, pool, n_slots, err_word);
    return hipGetLastError();
}

}  // namespace kv4
