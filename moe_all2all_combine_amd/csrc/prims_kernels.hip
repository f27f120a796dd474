// gfx950 kernels of the one-sided primitives (HyperParallel RFC, sections 四 and 六):
// put, put_with_signal, signal_op and wait_for_signal.
#include <hip/hip_runtime.h>

#include "common.h"
#include "device.h"
#include "launch.h"

namespace ra2a {

namespace {

// Widest vector that every byte of [dst, dst+bytes) and [src, src+bytes) allows.
int vec_width(const void* dst, const void* src, int64_t bytes) {
    const uint64_t m = (uint64_t)(uintptr_t)dst | (uint64_t)(uintptr_t)src | (uint64_t)bytes;
    if ((m & 15u) == 0) return 16;
    if ((m & 7u) == 0) return 8;
    if ((m & 3u) == 0) return 4;
    if ((m & 1u) == 0) return 2;
    return 1;
}

// Puts at most this large run in one workgroup that also signals (one launch);
// larger ones use a wide copy launch followed by a one-lane signal launch.
constexpr int64_t kSmallPut = 256 * 1024;

}  // namespace

// A wide put: workgroup k copies segments k, k + grid, ... of kPutSeg * V bytes
// (8 vectors per lane, all in flight), streamed past the caches.
constexpr int kPutSeg = kThreads * 8;  // vectors per segment
template <int V>
__global__ void __launch_bounds__(kThreads) put_kernel(uint8_t* dst, const uint8_t* src,
                                                      int64_t bytes) {
    const int64_t seg = (int64_t)kPutSeg * V;
    for (int64_t o = (int64_t)blockIdx.x * seg; o < bytes; o += (int64_t)gridDim.x * seg) {
        const int64_t n = bytes - o < seg ? bytes - o : seg;
        copy_flat<V, 8, true>(src + o, dst + o, n, threadIdx.x, kThreads);
    }
}

// One workgroup: copy, fence (every wave), barrier, then one lane signals.
template <int V>
__global__ void __launch_bounds__(kThreads) put_signal_kernel(uint8_t* dst, const uint8_t* src,
                                                             int64_t bytes, uint64_t* sig,
                                                             uint64_t value, int op) {
    copy_flat<V, 8>(src, dst, bytes, threadIdx.x, kThreads);
    wg_release();
    if (threadIdx.x == 0) sig_update(sig, value, op);
}

// Ordered after the preceding launch on the stream (which has completed and
// whose writes are visible device-wide when this one starts).
__global__ void signal_kernel(uint64_t* sig, uint64_t value, int op) {
    if (threadIdx.x == 0) {
        fence_release_agent();
        sig_update(sig, value, op);
    }
}

__global__ void wait_kernel(const uint64_t* sig, int cmp, uint64_t value, uint64_t timeout,
                            uint32_t* err) {
    if (threadIdx.x == 0) {
        spin_until(sig, cmp, value, timeout, err);
        fence_acquire_agent();
    }
}

template <int V>
static hipError_t put_v(uint8_t* dst, const uint8_t* src, int64_t bytes, hipStream_t st) {
    const int64_t per_wg = (int64_t)kThreads * V * 8;
    int64_t grid = (bytes + per_wg - 1) / per_wg;
    if (grid > 2048) grid = 2048;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(put_kernel<V>, dim3((unsigned)grid), dim3(kThreads), 0, st, dst, src, bytes);
    return hipGetLastError();
}

hipError_t launch_put(uint8_t* dst, const uint8_t* src, int64_t bytes, hipStream_t st) {
    if (bytes <= 0) return hipSuccess;
    switch (vec_width(dst, src, bytes)) {
        case 16: return put_v<16>(dst, src, bytes, st);
        case 8: return put_v<8>(dst, src, bytes, st);
        case 4: return put_v<4>(dst, src, bytes, st);
        case 2: return put_v<2>(dst, src, bytes, st);
        default: return put_v<1>(dst, src, bytes, st);
    }
}

hipError_t launch_signal_op(uint64_t* sig, uint64_t value, int op, hipStream_t st) {
    hipLaunchKernelGGL(signal_kernel, dim3(1), dim3(64), 0, st, sig, value, op);
    return hipGetLastError();
}

hipError_t launch_put_with_signal(uint8_t* dst, const uint8_t* src, int64_t bytes, uint64_t* sig,
                                  uint64_t value, int op, hipStream_t st) {
    if (bytes > kSmallPut) {
        hipError_t e = launch_put(dst, src, bytes, st);
        if (e != hipSuccess) return e;
        return launch_signal_op(sig, value, op, st);
    }
    const dim3 g(1), b(kThreads);
    switch (vec_width(dst, src, bytes)) {
        case 16: hipLaunchKernelGGL(put_signal_kernel<16>, g, b, 0, st, dst, src, bytes, sig, value, op); break;
        case 8: hipLaunchKernelGGL(put_signal_kernel<8>, g, b, 0, st, dst, src, bytes, sig, value, op); break;
        case 4: hipLaunchKernelGGL(put_signal_kernel<4>, g, b, 0, st, dst, src, bytes, sig, value, op); break;
        case 2: hipLaunchKernelGGL(put_signal_kernel<2>, g, b, 0, st, dst, src, bytes, sig, value, op); break;
        default: hipLaunchKernelGGL(put_signal_kernel<1>, g, b, 0, st, dst, src, bytes, sig, value, op); break;
    }
    return hipGetLastError();
}

hipError_t launch_wait(const uint64_t* sig, int cmp, uint64_t value, uint64_t timeout,
                       uint32_t* err, hipStream_t st) {
    hipLaunchKernelGGL(wait_kernel, dim3(1), dim3(64), 0, st, sig, cmp, value, timeout, err);
    return hipGetLastError();
}

}  // namespace ra2a
