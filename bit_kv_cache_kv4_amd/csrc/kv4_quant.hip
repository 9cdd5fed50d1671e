// Quantized KV row write (README "60+ inference optimizations & kernels",
// section "4-bit KV cache": the quantized write of 352-byte NVFP4 rows): one
// wavefront per row, four rows per workgroup.  The row's arithmetic is in
// kv4_quant_impl.h.
#include "kv4_quant_impl.h"
#include "kv4_launch.h"

namespace kv4 {

constexpr int kQuantRowsPerBlock = 4;   // 4 waves of 64 lanes

__global__ __launch_bounds__(256) void quant_write_kernel(const float *__restrict__ kv, int64_t kv_row_stride,
                                                          const int32_t *__restrict__ slots, int64_t n_tokens,
                                                          uint8_t *__restrict__ pool, int64_t n_slots,
                                                          uint32_t *__restrict__ err_word) {
    quant_write_row(kv, kv_row_stride, slots, n_tokens, pool, n_slots, err_word,
                    (int64_t)blockIdx.x * kQuantRowsPerBlock + (threadIdx.x >> 6), threadIdx.x & 63);
}

__global__ __launch_bounds__(256) void quant_write_rope_free_kernel(const float *__restrict__ kv, int64_t kv_row_stride,
                                                                    const int32_t *__restrict__ slots, int64_t n_tokens,
                                                                    uint8_t *__restrict__ pool, int64_t n_slots,
                                                                    uint32_t *__restrict__ err_word) {
    quant_write_row<false>(kv, kv_row_stride, slots, n_tokens, pool, n_slots, err_word,
                           (int64_t)blockIdx.x * kQuantRowsPerBlock + (threadIdx.x >> 6), threadIdx.x & 63);
}

hipError_t launch_quant_write_rope_free(const float *kv, int64_t kv_row_stride, const int32_t *slots, int64_t n_tokens,
                                        uint8_t *pool, int64_t n_slots, uint32_t *err_word, hipStream_t stream) {
    if (n_tokens == 0) return hipSuccess;
    const int64_t blocks = (n_tokens + kQuantRowsPerBlock - 1) / kQuantRowsPerBlock;
    hipLaunchKernelGGL(quant_write_rope_free_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, kv, kv_row_stride,
                       slots, n_tokens, pool, n_slots, err_word);
    return hipGetLastError();
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
