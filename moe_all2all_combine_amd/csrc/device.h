// Device-side building blocks shared by the gfx950 kernels: vector copies,
// signal operations, bounded waits and the workgroup-level release/acquire.
//
// Memory-ordering model (gfx950, agent scope).  Each XCD has its own L2; a
// store is visible to another XCD only after the writer's L2 has written the
// line back, and a reader on another XCD must not hit a stale line of its own
// L2.  The compiler's agent-scope fences do exactly that: a release fence is a
// full L2 write-back plus a wait for the wave's own stores, an acquire fence
// invalidates the non-coherent lines of L1/L2.  A fence only waits for the
// memory operations of its own wave, so a workgroup that stored a tile with
// all its waves publishes it as:  every wave fences (release) -> workgroup
// barrier -> one lane updates the signal.  The consumer side mirrors it: one
// lane spins with relaxed loads -> barrier -> every wave fences (acquire).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace ra2a {

__device__ __forceinline__ uint64_t rtc_now() { return __builtin_amdgcn_s_memrealtime(); }

__device__ __forceinline__ void fence_release_agent() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
}
__device__ __forceinline__ void fence_acquire_agent() {
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

__device__ __forceinline__ uint64_t sig_load(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Signal update, relaxed: callers order it after their data with a release
// fence (see the header comment).  Both operations are read-modify-write
// atomics, which are coherent device-wide on their own.
__device__ __forceinline__ void sig_update(uint64_t* p, uint64_t v, int op) {
    if (op == kSigSet)
        (void)__hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        (void)__hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ bool cmp_holds(uint64_t x, int op, uint64_t v) {
    switch (op) {
        case kCmpEq: return x == v;
        case kCmpNe: return x != v;
        case kCmpGt: return x > v;
        case kCmpGe: return x >= v;
        case kCmpLt: return x < v;
        default: return x <= v;  // kCmpLe
    }
}

// Bounded spin by one lane: relaxed polling with s_sleep back-off.  Gives up
// (returns false) when the wait exceeds `timeout` ticks of the 100 MHz device
// real-time clock -- then it also raises the error word so every other waiter
// of the launch gives up promptly -- or when another waiter already did.
__device__ __forceinline__ bool spin_until(const uint64_t* p, int op, uint64_t v,
                                           uint64_t timeout, uint32_t* err) {
    uint64_t x = sig_load(p);
    if (cmp_holds(x, op, v)) return true;
    const uint64_t t0 = rtc_now();
    uint32_t n = 0;
    while (true) {
        __builtin_amdgcn_s_sleep(1);
        x = sig_load(p);
        if (cmp_holds(x, op, v)) return true;
        if ((++n & 31u) == 0) {
            if (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u)
                return false;
            if (rtc_now() - t0 > timeout) {
                __hip_atomic_fetch_or(err, kErrTimeout, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
                return false;
            }
        }
    }
}

// Workgroup-wide wait, device-wide flavour: lane 0 spins, everyone acquires.
// Returns false (uniformly across the workgroup) if the wait gave up.
__device__ __forceinline__ bool wg_wait(const uint64_t* p, int op, uint64_t v, uint64_t timeout,
                                        uint32_t* err, int* lds_flag) {
    if (threadIdx.x == 0) *lds_flag = spin_until(p, op, v, timeout, err) ? 1 : 0;
    __syncthreads();
    const bool ok = *lds_flag != 0;
    fence_acquire_agent();
    __syncthreads();  // lds_flag may be rewritten by the next wait
    return ok;
}

// Workgroup-wide release, device-wide flavour: every wave's stores become
// visible device-wide before any signal issued after this call by any lane.
__device__ __forceinline__ void wg_release() {
    fence_release_agent();
    __syncthreads();
}

// ---- synchronisation between workgroups of one XCD ---------------------------
//
// Workgroups on the same XCD share its L2; the vector L1 of each CU is write-
// through.  The signals themselves are device-scope atomics (read-modify-write
// updates, L1-bypassing polls), coherent on their own.  The data is ordered
// around them as follows.
//   release: every wave drains (s_waitcnt vmcnt(0): its stores have been
//            acknowledged by the L2), then the workgroup barrier, then wave 0
//            signals.  With producer and consumer on one XCD the data is now in
//            the L2 both read through, so nothing is written back from it --
//            that device-wide write-back is what the XCD-local protocol saves.
//            (SYNC == kSyncAgent adds it, for producers and consumers that may
//            sit on different XCDs.)
//   acquire: none.  Consumers read the published data with device-scope loads
//            (cache policy sc1), which are never served from the CU's L1 -- whose
//            lines may hold an earlier use of the same staging slot -- and so
//            read the L2 the producers' stores went to.  (The workgroup-scope
//            invalidate `buffer_inv sc0` would not do: outside threadgroup-split
//            dispatches it leaves the L1 alone; measured, a consumer then read
//            the slot's previous contents.)  SYNC == kSyncAgent instead has wave
//            0 run the device-scope acquire (`buffer_inv sc1`), dropping stale
//            L1 and L2 lines, before plain loads.
// The pipelined kernel guarantees the "same XCD" premise itself: a workgroup
// serves only stream groups its own XCD owns (XCC_ID register).

// This wave's memory operations have completed (stores acknowledged by the L2,
// loads returned).
__device__ __forceinline__ void wave_drain() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Workgroup-wide wait.  Lane 0 spins; with ACQUIRE, wave 0 then acquires for the
// whole workgroup (needed before reading data the signal publishes; not needed
// before only writing, e.g. after a ring hand-back).  Returns false, uniformly
// across the workgroup, if the wait gave up.
template <bool ACQUIRE>
__device__ __forceinline__ bool group_wait(const uint64_t* p, int op, uint64_t v, uint64_t timeout,
                                           uint32_t* err, int* lds_flag) {
    if (threadIdx.x == 0) {
        const bool ok = spin_until(p, op, v, timeout, err);
        if (ACQUIRE) fence_acquire_agent();
        *lds_flag = ok ? 1 : 0;
    }
    __syncthreads();
    const bool ok = *lds_flag != 0;
    __syncthreads();  // lds_flag may be rewritten by the next wait
    return ok;
}

// The same for `n` signals `step` bytes apart, all of which must hold.
template <bool ACQUIRE>
__device__ __forceinline__ bool group_wait_all(const uint64_t* p, int64_t step, int n, int op,
                                               uint64_t v, uint64_t timeout, uint32_t* err,
                                               int* lds_flag) {
    if (threadIdx.x == 0) {
        bool ok = true;
        for (int k = 0; k < n && ok; ++k)
            ok = spin_until(reinterpret_cast<const uint64_t*>(
                                reinterpret_cast<const uint8_t*>(p) + k * step),
                            op, v, timeout, err);
        if (ACQUIRE) fence_acquire_agent();
        *lds_flag = ok ? 1 : 0;
    }
    __syncthreads();
    const bool ok = *lds_flag != 0;
    __syncthreads();
    return ok;
}

// Workgroup-wide release: afterwards wave 0 may signal.  Every wave drains its
// own memory operations; with SYNC == kSyncAgent wave 0 then also writes the
// L2 back (one write-back covers every wave's stores, which the drains put in
// the L2).  Signals must be issued by wave 0 (threadIdx.x < 64).
template <int SYNC>
__device__ __forceinline__ void group_release() {
    wave_drain();
    __syncthreads();
    if (SYNC == kSyncAgent && threadIdx.x < 64) fence_release_agent();
}

__device__ __forceinline__ uint32_t xcc_id() {
    return __builtin_amdgcn_s_getreg(20 | (0 << 6) | (15 << 11)) & 0xFu;  // HW_REG_XCC_ID
}

// ---- vector copies ---------------------------------------------------------

// Native vector types (not HIP's struct wrappers), so copies stay in VGPRs.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int V> struct Vec;
template <> struct Vec<16> { using T = u32x4; };
template <> struct Vec<8> { using T = u32x2; };
template <> struct Vec<4> { using T = uint32_t; };
template <> struct Vec<2> { using T = uint16_t; };
template <> struct Vec<1> { using T = uint8_t; };

// Buffer loads through a resource descriptor: the cache-policy bits are explicit
// and the hardware range-checks every access against the descriptor's size
// (an out-of-range load returns 0 instead of touching other memory).
constexpr int kPolicySc1 = 16;  // device scope: never served from the CU's L1
constexpr int kPolicyNt = 2;    // non-temporal: streamed, evicted first
constexpr uint32_t kBufferDword3 = 0x00020000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             (int)kBufferDword3);
}

// The same for a wave-uniform base and size, stated to the compiler: the
// descriptor then lives in scalar registers.  (A descriptor the compiler cannot
// prove uniform sits in vector registers, and every buffer instruction using it
// is wrapped in a loop over its distinct values.)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_uniform(const void* base, uint32_t bytes) {
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
    return make_rsrc(reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo),
                     __builtin_amdgcn_readfirstlane(bytes));
}

template <int V, int POLICY> struct BufLoad;
template <int POLICY> struct BufLoad<16, POLICY> {
    static __device__ __forceinline__ u32x4 go(__amdgpu_buffer_rsrc_t r, uint32_t off) {
        return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, POLICY);
    }
};
template <int POLICY> struct BufLoad<8, POLICY> {
    static __device__ __forceinline__ u32x2 go(__amdgpu_buffer_rsrc_t r, uint32_t off) {
        return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, POLICY);
    }
};
template <int POLICY> struct BufLoad<4, POLICY> {
    static __device__ __forceinline__ uint32_t go(__amdgpu_buffer_rsrc_t r, uint32_t off) {
        return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, POLICY);
    }
};
template <int POLICY> struct BufLoad<2, POLICY> {
    static __device__ __forceinline__ uint16_t go(__amdgpu_buffer_rsrc_t r, uint32_t off) {
        return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, POLICY);
    }
};
template <int POLICY> struct BufLoad<1, POLICY> {
    static __device__ __forceinline__ uint8_t go(__amdgpu_buffer_rsrc_t r, uint32_t off) {
        return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, POLICY);
    }
};

// Buffer stores with cache policy POLICY.  kPolicyDevNt (device scope +
// non-temporal) is how the direct combine writes its output: a device-scope
// store is written through to the device's point of coherence -- it is what a
// relaxed device-scope atomic store compiles to on gfx950 (`sc1`, with no L2
// write-back around it) -- so once the wave has drained it (s_waitcnt
// vmcnt(0)) the data is visible to every XCD, and no L2 write-back
// (`buffer_wbl2`) is needed before the signal.  A reader still acquires
// (invalidates its own stale L1/L2 lines) after it sees the signal.
constexpr int kPolicyDevNt = kPolicySc1 | kPolicyNt;

template <int V, int POLICY> struct BufStore;
template <int POLICY> struct BufStore<16, POLICY> {
    static __device__ __forceinline__ void go(u32x4 v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
        __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, POLICY);
    }
};
template <int POLICY> struct BufStore<8, POLICY> {
    static __device__ __forceinline__ void go(u32x2 v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
        __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, POLICY);
    }
};
template <int POLICY> struct BufStore<4, POLICY> {
    static __device__ __forceinline__ void go(uint32_t v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
        __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, POLICY);
    }
};
template <int POLICY> struct BufStore<2, POLICY> {
    static __device__ __forceinline__ void go(uint16_t v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
        __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, POLICY);
    }
};
template <int POLICY> struct BufStore<1, POLICY> {
    static __device__ __forceinline__ void go(uint8_t v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
        __builtin_amdgcn_raw_buffer_store_b8(v, r, off, 0, POLICY);
    }
};

// Release of data written with device-scope stores (kPolicyDevNt): every wave
// drains its own stores -- each is then performed device-wide -- and the
// workgroup barrier orders them all before the signal wave 0 issues next.
__device__ __forceinline__ void group_release_written_through() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
}

template <typename T>
__device__ __forceinline__ T load_nt(const T* p) { return __builtin_nontemporal_load(p); }
template <typename T>
__device__ __forceinline__ void store_nt(T v, T* p) { __builtin_nontemporal_store(v, p); }

// Contiguous copy of `bytes` (a multiple of V) by threads [tid0, tid0 + nthr).
// Full rounds keep U vectors per thread in flight (all loads, then all
// stores, no bounds checks so the values stay in registers); the remainder
// goes one vector at a time.
// NT: non-temporal loads (streamed past the caches); NTS: the same for the
// stores (by default as NT).
template <int V, int U, bool NT = false, bool NTS = NT>
__device__ __forceinline__ void copy_flat(const uint8_t* __restrict__ src,
                                          uint8_t* __restrict__ dst, int64_t bytes, int64_t tid0,
                                          int64_t nthr) {
    using T = typename Vec<V>::T;
    const int64_t total = bytes / V;
    const T* s = reinterpret_cast<const T*>(src);
    T* d = reinterpret_cast<T*>(dst);
    int64_t idx = tid0;
    for (; idx + (U - 1) * nthr < total; idx += U * nthr) {
        T v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = NT ? load_nt(s + idx + u * nthr) : s[idx + u * nthr];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (NTS)
                store_nt(v[u], d + idx + u * nthr);
            else
                d[idx + u * nthr] = v[u];
        }
    }
    for (; idx < total; idx += nthr) {
        const T v = NT ? load_nt(s + idx) : s[idx];
        if (NTS)
            store_nt(v, d + idx);
        else
            d[idx] = v;
    }
}

// SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
// generators", OOPSLA 2014): the output for counter value x of a sequence
// seeded with `seed`.
__device__ __forceinline__ uint64_t splitmix64(uint64_t seed, uint64_t x) {
    uint64_t z = seed + (x + 1) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

}  // namespace ra2a
