// Dedup compaction of one top-k list by one workgroup (README "60+ inference
// optimizations & kernels", section "4-bit KV cache": dedup compaction); the
// algorithm is described in kv4_dedup.hip, which launches it alone.
#pragma once

#include "kv4_device.h"

namespace kv4 {

constexpr uint32_t kEmpty = 0xFFFFFFFFu;

// relaxed workgroup-scope LDS atomics: nothing orders one against another
__device__ __forceinline__ uint32_t lds_cas(uint32_t *a, uint32_t expect, uint32_t v) {
    __hip_atomic_compare_exchange_strong(a, &expect, v, __ATOMIC_RELAXED, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return expect;
}
__device__ __forceinline__ void lds_min(int32_t *a, int32_t v) {
    (void)__hip_atomic_fetch_min(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

__device__ __forceinline__ uint32_t dedup_hash(uint32_t v, int log2_table) {
    return (v * 0x9E3779B1u) >> (32 - log2_table);
}

constexpr size_t dedup_lds_words(int threads, int items, int log2_table) {
    return (size_t)2 * ((size_t)1 << log2_table) + 2 * threads + (size_t)items * threads + 4 * (threads / 64);
}

// smallest table (a power of two) with load factor <= 1/4 and at least four
// entries per lane (it is cleared 16 bytes a lane at a time)
inline int dedup_log2_table(int32_t k, int threads) {
    int l = 10;
    while ((1 << l) < 4 * k || (1 << l) < 4 * threads) ++l;
    return l;
}

// Dedup of list `list` by a workgroup of THREADS lanes; lds holds
// dedup_lds_words(THREADS, ITEMS, log2_table) 32-bit words, 16-byte aligned.
template <int THREADS, int ITEMS>
__device__ __forceinline__ void dedup_list(const int32_t *__restrict__ idx, int32_t k, int64_t idx_row_stride,
                                           int32_t *__restrict__ out_idx, int32_t *__restrict__ out_count,
                                           int log2_table, int64_t list, uint32_t *lds) {
    const int T = 1 << log2_table;
    uint32_t *keys = lds;                    // T keys, then one private dummy slot per thread
    int32_t *minpos = reinterpret_cast<int32_t *>(lds + T + THREADS);
    int32_t *stage = reinterpret_cast<int32_t *>(lds + 2 * T + 2 * THREADS);
    int32_t *wave_tot = stage + ITEMS * THREADS;
    const int tid = threadIdx.x;
    const int32_t *src = idx + list * idx_row_stride;

    {   // all of the list's loads in flight at once (k <= 256 * ITEMS), coalesced
        int32_t ld[ITEMS];
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) {
            const int j = tid + THREADS * i;
            ld[i] = j < k ? src[j] : -1;
        }
        for (int i = 4 * tid; i < T; i += 4 * THREADS) {   // T is a multiple of 4 * THREADS
            *reinterpret_cast<uint4 *>(keys + i) = uint4{kEmpty, kEmpty, kEmpty, kEmpty};
            *reinterpret_cast<int4 *>(minpos + i) = int4{0x7FFFFFFF, 0x7FFFFFFF, 0x7FFFFFFF, 0x7FFFFFFF};
        }
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) stage[tid + THREADS * i] = ld[i];
    }
    __syncthreads();

    // Insert: every item's first compare-and-swap is issued before any result
    // is looked at (unconditionally: an entry < 0 targets this thread's dummy
    // slot, so no branch separates the atomics), then the few collisions probe
    // onwards, then the non-returning minimum of the positions.
    int32_t v[ITEMS];
    uint32_t slot[ITEMS];
    bool pending[ITEMS];
    // stage holds -1 past k (written above for every entry of every thread)
    if constexpr (ITEMS % 4 == 0) {
#pragma unroll
        for (int i = 0; i < ITEMS; i += 4) {
            const int4 w = *reinterpret_cast<const int4 *>(stage + tid * ITEMS + i);
            v[i] = w.x, v[i + 1] = w.y, v[i + 2] = w.z, v[i + 3] = w.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) v[i] = stage[tid * ITEMS + i];
    }
#pragma unroll
    for (int i = 0; i < ITEMS; ++i)
        slot[i] = v[i] >= 0 ? dedup_hash((uint32_t)v[i], log2_table) : (uint32_t)(T + tid);
    uint32_t old[ITEMS];
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) old[i] = lds_cas(&keys[slot[i]], kEmpty, (uint32_t)v[i]);
    __builtin_amdgcn_sched_barrier(0);        // all of them issued before any result is read
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) pending[i] = v[i] >= 0 && old[i] != kEmpty && old[i] != (uint32_t)v[i];
    // collisions: every pending item of the wavefront probes one slot further
    // per round, all of a round's atomics issued together (the rest hit the
    // thread's dummy slot), so the rounds number the longest probe, not the sum
    bool any = false;
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) any |= pending[i];
    while (__ballot(any) != 0) {
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) {
            if (pending[i]) slot[i] = (slot[i] + 1) & (T - 1);
            old[i] = lds_cas(&keys[pending[i] ? slot[i] : (uint32_t)(T + tid)], kEmpty, (uint32_t)v[i]);
        }
        __builtin_amdgcn_sched_barrier(0);
        any = false;
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) {
            pending[i] = pending[i] && old[i] != kEmpty && old[i] != (uint32_t)v[i];
            any |= pending[i];
        }
    }
#pragma unroll
    for (int i = 0; i < ITEMS; ++i)
        if (v[i] >= 0) lds_min(&minpos[slot[i]], tid * ITEMS + i);
    __syncthreads();

    uint32_t keep = 0;
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
        const int j = tid * ITEMS + i;
        if (v[i] >= 0 && minpos[slot[i]] == j) {
            keep |= 1u << i;
            ++cnt;
        }
    }

    // exclusive prefix sum of cnt over the workgroup, in lane order
    const int lane = tid & 63, wave = tid >> 6;
    int incl = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_up(incl, off);
        if (lane >= off) incl += t;
    }
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    int base = 0, total = 0;
#pragma unroll
    for (int w = 0; w < THREADS / 64; ++w) {
        const int t = wave_tot[w];
        base += w < wave ? t : 0;
        total += t;
    }
    int pos = base + incl - cnt;
#pragma unroll
    for (int i = 0; i < ITEMS; ++i)
        if (keep & (1u << i)) stage[pos++] = v[i];   // stage was fully read before the barrier above
    __syncthreads();

    int32_t *dst = out_idx + list * (int64_t)k;
    for (int j = tid; j < k; j += THREADS) dst[j] = j < total ? stage[j] : -1;
    if (tid == 0) out_count[list] = total;
}

}  // namespace kv4
