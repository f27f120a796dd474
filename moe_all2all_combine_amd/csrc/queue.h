// Work-queue claims shared by the persistent kernels (combine, AllGather+GEMM).
//
// Each stream group g has a queue of tasks ordered so that every wait points
// to an earlier position; workgroups claim positions with one atomic each and
// run each task to completion, so the earliest unfinished task can always
// proceed (no deadlock at any residency).  Queue words (8-byte values on
// 128-byte slots, zeroed before every launch): per group a claim counter and a
// take-over counter, then a mask of fully claimed groups.
//
// Binding (OWNED): a group's tasks must run on one XCD (their data meets in one
// L2).  The home XCD (XCC_ID mod NG == g) claims directly from the claim
// counter; the returned word says whether another XCD took the group over
// first (bit 63, bits 32..39 = that XCD + 1).  Another XCD takes a group over
// only while its claim counter is still 0, then claims from the take-over
// counter.  Without binding any workgroup claims from any group.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace ra2a {

constexpr uint64_t kTaken = 1ull << 63;
constexpr uint64_t kOwnerMask = 0xFFull << 32;

// Claim state kept by thread 0 of a workgroup.
struct QueueClaim {
    uint64_t* ctr = nullptr;  // counter the current group's claims come from
    uint64_t known = 0;       // groups known to be fully claimed
    bool stale = true;        // `known` may be out of date
};

// Thread 0 only: the first position this workgroup gets in group g (visited as
// the gi-th group, gi = 0 being its home group), or -1 if it must not or need
// not serve group g.
template <bool OWNED>
__device__ __forceinline__ int64_t queue_first(uint64_t* qw, int g, int gi, uint32_t xcc,
                                               QueueClaim& qc) {
    uint64_t* const head = qw + (int64_t)(2 * g) * kSigStrideU64;
    uint64_t* const taker = head + kSigStrideU64;
    uint64_t* const drained = qw + (int64_t)(2 * kNumXcd) * kSigStrideU64;
    if (gi > 0 && qc.stale) {
        qc.known = __hip_atomic_load(drained, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        qc.stale = false;
    }
    if ((qc.known >> g) & 1ull) return -1;  // fully claimed
    if (!OWNED || gi == 0) {
        const uint64_t h = __hip_atomic_fetch_add(head, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        qc.ctr = head;
        return (h & kTaken) ? -1 : (int64_t)h;
    }
    const uint64_t mine = kTaken | ((uint64_t)(xcc + 1u) << 32);
    uint64_t cur = 0;
    __hip_atomic_compare_exchange_strong(head, &cur, mine, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    if (cur == 0ull || (cur & (kTaken | kOwnerMask)) == mine) {
        qc.ctr = taker;
        return (int64_t)__hip_atomic_fetch_add(taker, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return -1;
}

// Thread 0 only: the next claim from the current group.
__device__ __forceinline__ uint64_t queue_next(const QueueClaim& qc) {
    return __hip_atomic_fetch_add(qc.ctr, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Thread 0 only: a claim returned `pos` >= the queue's length.  The one claim
// landing exactly at the end marks the group fully claimed (no wait;
// same-address atomics serialise, so they are kept few).
__device__ __forceinline__ void queue_drained(uint64_t* qw, int g, int64_t pos, int64_t total,
                                              QueueClaim& qc) {
    if (pos == total)
        __hip_atomic_fetch_or(qw + (int64_t)(2 * kNumXcd) * kSigStrideU64, 1ull << g,
                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    qc.stale = true;
}

}  // namespace ra2a
