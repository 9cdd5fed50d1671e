// kv4_sparse_mla_decode_noalloc: split-K decode whose split parts live in a
// scratch array the library holds, for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  It runs exactly kv4_sparse_mla_decode's kernels.
//
// `scratch` is a file-scope device array: each GPU the library runs on holds
// its own copy until the process ends.  In host code its name is only a
// host-side stand-in, so its device address is looked up once per device
// with hipGetSymbolAddress (with that device current), and that pointer is
// the only one ever handed to a kernel.  Nothing in it has to start at zero:
// the split kernel writes every part the merge reads.
#include <mutex>

#include "kv4.h"
#include "kv4_launch.h"

namespace {

constexpr size_t kScratchBytes = (size_t)32 << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_mu;
void *g_ptr[kMaxDevices] = {};

// The current device's copy of scratch, looked up on its first use.
kv4_status device_scratch(void **out) {
    int dev = 0;
    const hipError_t e0 = hipGetDevice(&dev);
    if (e0 != hipSuccess) return kv4::api_fail(KV4_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e0));
    if (dev < 0 || dev >= kMaxDevices)
        return kv4::api_fail(KV4_ERR_UNSUPPORTED, "device %d; the scratch table covers devices 0..%d", dev,
                             kMaxDevices - 1);
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return kv4::api_fail(KV4_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        g_ptr[dev] = ptr;
    }
    *out = g_ptr[dev];
    return KV4_OK;
}

}  // namespace

extern "C" {

size_t kv4_noalloc_scratch_bytes(void) { return kScratchBytes; }

kv4_status kv4_sparse_mla_decode_noalloc(const kv4_attn_args *a, int32_t num_splits, void *stream) {
    const int32_t auto_s = kv4_sparse_mla_decode_splits(a);
    if (auto_s < 0) return kv4_sparse_mla_decode(a, num_splits, nullptr, 0, stream);   // its argument error
    const size_t need = kv4_sparse_mla_decode_workspace(a, num_splits);
    if (need > kScratchBytes)
        return kv4::api_fail(KV4_ERR_WORKSPACE,
                             "these arguments need %zu bytes of split parts; kv4_sparse_mla_decode_noalloc holds "
                             "%zu (use fewer splits, or kv4_sparse_mla_decode with a workspace)",
                             need, kScratchBytes);
    void *ws = nullptr;
    if (need > 0) {
        const kv4_status st = device_scratch(&ws);
        if (st != KV4_OK) return st;
    }
    return kv4_sparse_mla_decode(a, num_splits, ws, need > 0 ? kScratchBytes : 0, stream);
}

}  // extern "C"
