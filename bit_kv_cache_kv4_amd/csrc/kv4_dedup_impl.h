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

// The table, the staged list and the scan's totals in LDS: dedup_lds_words
// 32-bit words, 16-byte aligned.
template <int THREADS, int ITEMS>
struct DedupLds {
    uint32_t *keys;       // T keys, then one private dummy slot per thread
    int32_t *minpos;      // T smallest positions (and THREADS unused words)
    int32_t *stage;       // ITEMS * THREADS entries: the list, then its kept entries
    int32_t *wave_tot;    // per-wavefront counts of kept entries
    __device__ DedupLds(uint32_t *lds, int T)
        : keys(lds), minpos(reinterpret_cast<int32_t *>(lds + T + THREADS)),
          stage(reinterpret_cast<int32_t *>(lds + 2 * T + 2 * THREADS)), wave_tot(stage + ITEMS * THREADS) {}
};

// the list's entries, coalesced: ld[i] = entry tid + THREADS i (-1 past k)
template <int THREADS, int ITEMS>
__device__ __forceinline__ void dedup_load(const int32_t *__restrict__ src, int32_t k, int32_t (&ld)[ITEMS]) {
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
        const int j = threadIdx.x + THREADS * i;
        ld[i] = j < k ? src[j] : -1;
    }
}

template <int THREADS, int ITEMS>
__device__ __forceinline__ void dedup_clear(const DedupLds<THREADS, ITEMS> &m, int T) {
    for (int i = 4 * threadIdx.x; i < T; i += 4 * THREADS) {   // T is a multiple of 4 * THREADS
        *reinterpret_cast<uint4 *>(m.keys + i) = uint4{kEmpty, kEmpty, kEmpty, kEmpty};
        *reinterpret_cast<int4 *>(m.minpos + i) = int4{0x7FFFFFFF, 0x7FFFFFFF, 0x7FFFFFFF, 0x7FFFFFFF};
    }
}

template <int THREADS, int ITEMS>
__device__ __forceinline__ void dedup_stage(const DedupLds<THREADS, ITEMS> &m, const int32_t (&ld)[ITEMS]) {
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) m.stage[threadIdx.x + THREADS * i] = ld[i];
}

// This thread's entries tid ITEMS .. tid ITEMS + ITEMS - 1 from the staged
// list (after a barrier that follows dedup_stage); stage holds -1 past k.
template <int THREADS, int ITEMS>
__device__ __forceinline__ void dedup_read_staged(const DedupLds<THREADS, ITEMS> &m, int32_t (&v)[ITEMS]) {
    const int tid = threadIdx.x;
    if constexpr (ITEMS % 4 == 0) {
#pragma unroll
        for (int i = 0; i < ITEMS; i += 4) {
            const int4 w = *reinterpret_cast<const int4 *>(m.stage + tid * ITEMS + i);
            v[i] = w.x, v[i + 1] = w.y, v[i + 2] = w.z, v[i + 3] = w.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) v[i] = m.stage[tid * ITEMS + i];
    }
}

// The same entries straight from the list, one vector load per four (or
// fewer) of them; k must be a multiple of ITEMS (a thread's entries are all
// in the list or all past it, then -1) and the list aligned to the vector.
template <int THREADS, int ITEMS>
__device__ __forceinline__ void dedup_load_direct(const int32_t *__restrict__ src, int32_t k, int32_t (&v)[ITEMS]) {
    const int j0 = threadIdx.x * ITEMS;
    const bool in = j0 < k;
    const int32_t *p = src + (in ? j0 : 0);
    if constexpr (ITEMS % 4 == 0) {
#pragma unroll
        for (int i = 0; i < ITEMS; i += 4) {
            int4 w = {-1, -1, -1, -1};
            if (in) w = *reinterpret_cast<const int4 *>(p + i);
            v[i] = w.x, v[i + 1] = w.y, v[i + 2] = w.z, v[i + 3] = w.w;
        }
    } else if constexpr (ITEMS == 2) {
        int2 w = {-1, -1};
        if (in) w = *reinterpret_cast<const int2 *>(p);
        v[0] = w.x, v[1] = w.y;
    } else {
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) v[i] = in ? p[i] : -1;
    }
}

// The dedup of a list whose entries v[] this thread holds (entries tid ITEMS
// + i, -1 past k), the table cleared and synchronized: writes the k outputs
// and the count.  Leaves the entries' table slots slot[] (meaningful where
// v[i] >= 0) for dedup_undo; every slot written with a key is one of them.
template <int THREADS, int ITEMS>
__device__ __forceinline__ void dedup_core(const DedupLds<THREADS, ITEMS> &m, int32_t k, int log2_table,
                                           int32_t *__restrict__ dst, int32_t *__restrict__ count,
                                           const int32_t (&v)[ITEMS], uint32_t (&slot)[ITEMS]) {
    const int T = 1 << log2_table;
    const int tid = threadIdx.x;
    // Insert: every item's first compare-and-swap is issued before any result
    // is looked at (unconditionally: an entry < 0 targets this thread's dummy
    // slot, so no branch separates the atomics), then the few collisions probe
    // onwards, then the non-returning minimum of the positions.
    bool pending[ITEMS];
#pragma unroll
    for (int i = 0; i < ITEMS; ++i)
        slot[i] = v[i] >= 0 ? dedup_hash((uint32_t)v[i], log2_table) : (uint32_t)(T + tid);
    uint32_t old[ITEMS];
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) old[i] = lds_cas(&m.keys[slot[i]], kEmpty, (uint32_t)v[i]);
    __builtin_amdgcn_sched_barrier(0);        // all of them issued before any result is read
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) pending[i] = v[i] >= 0 && old[i] != kEmpty && old[i] != (uint32_t)v[i];
    // collisions: every pending item of the wavefront probes one slot further
    // per round, all of a round's atomics issued together (only the pending
    // lanes take part), so the rounds number the longest probe, not the sum
    bool any = false;
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) any |= pending[i];
    while (__ballot(any) != 0) {
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) {
            if (pending[i]) {
                slot[i] = (slot[i] + 1) & (T - 1);
                old[i] = lds_cas(&m.keys[slot[i]], kEmpty, (uint32_t)v[i]);
            }
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
        if (v[i] >= 0) lds_min(&m.minpos[slot[i]], tid * ITEMS + i);
    __syncthreads();

    // kept entries and their places: entry j = tid ITEMS + i is kept iff its
    // position is its key's minimum; the kept entries of the wavefront's
    // earlier lanes (all of whose entries precede this lane's) are counted
    // from one ballot per item, the wavefronts' totals exchanged through LDS
    uint32_t keep = 0;
    int below = 0, wave_kept = 0;
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
        const bool k_i = v[i] >= 0 && m.minpos[slot[i]] == tid * ITEMS + i;
        keep |= k_i ? 1u << i : 0u;
        const uint64_t b = __ballot(k_i);
        below += (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
        wave_kept += (int)__popcll(b);
    }
    const int lane = tid & 63, wave = tid >> 6;
    if (lane == 0) m.wave_tot[wave] = wave_kept;
    __syncthreads();
    int base = 0, total = 0;
#pragma unroll
    for (int w = 0; w < THREADS / 64; ++w) {
        const int t = m.wave_tot[w];
        base += w < wave ? t : 0;
        total += t;
    }
    int pos = base + below;
#pragma unroll
    for (int i = 0; i < ITEMS; ++i)
        if (keep & (1u << i)) m.stage[pos++] = v[i];   // stage was fully read before the barrier above
    __syncthreads();

    // ITEMS stores per thread on every path (k <= THREADS * ITEMS; lanes past
    // k repeat entry k - 1's store, the same value to the same address): a
    // caller that waits for loads issued before them can then leave the
    // stores in flight, which a count that varies with the path would not
    if (k > 0) {
#pragma unroll
        for (int i = 0; i < ITEMS; ++i) {
            const int j = min(tid + THREADS * i, k - 1);
            dst[j] = j < total ? m.stage[j] : -1;
        }
    }
    if (tid == 0) *count = total;
}

// Returns the table to its cleared state after dedup_core, touching only the
// slots that hold keys (each is some thread's slot[i] with v[i] >= 0; the
// dummy slots are never read).  The caller synchronizes after dedup_core's
// last LDS read and before the next list's atomics.
template <int THREADS, int ITEMS>
__device__ __forceinline__ void dedup_undo(const DedupLds<THREADS, ITEMS> &m, const int32_t (&v)[ITEMS],
                                           const uint32_t (&slot)[ITEMS]) {
#pragma unroll
    for (int i = 0; i < ITEMS; ++i)
        if (v[i] >= 0) {
            m.keys[slot[i]] = kEmpty;
            m.minpos[slot[i]] = 0x7FFFFFFF;
        }
}

// Dedup of list `list` by a workgroup of THREADS lanes; lds holds
// dedup_lds_words(THREADS, ITEMS, log2_table) 32-bit words, 16-byte aligned.
template <int THREADS, int ITEMS, bool DIRECT = false>
__device__ __forceinline__ void dedup_list(const int32_t *__restrict__ idx, int32_t k, int64_t idx_row_stride,
                                           int32_t *__restrict__ out_idx, int32_t *__restrict__ out_count,
                                           int log2_table, int64_t list, uint32_t *lds) {
    const DedupLds<THREADS, ITEMS> m(lds, 1 << log2_table);
    int32_t v[ITEMS];
    if constexpr (DIRECT) {
        dedup_load_direct<THREADS, ITEMS>(idx + list * idx_row_stride, k, v);
        dedup_clear<THREADS, ITEMS>(m, 1 << log2_table);
        __syncthreads();
    } else {   // all of the list's loads in flight at once (k <= THREADS * ITEMS), coalesced
        int32_t ld[ITEMS];
        dedup_load<THREADS, ITEMS>(idx + list * idx_row_stride, k, ld);
        dedup_clear<THREADS, ITEMS>(m, 1 << log2_table);
        dedup_stage<THREADS, ITEMS>(m, ld);
        __syncthreads();
        dedup_read_staged<THREADS, ITEMS>(m, v);
    }
    uint32_t slot[ITEMS];
    dedup_core<THREADS, ITEMS>(m, k, log2_table, out_idx + list * (int64_t)k, out_count + list, v, slot);
}

}  // namespace kv4
