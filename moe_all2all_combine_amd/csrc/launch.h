// Host-side launchers of the gfx950 kernels (defined next to each kernel).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ag_gemm_geom.h"
#include "alltoallv_geom.h"
#include "gemm_rs_geom.h"
#include "common.h"

namespace ra2a {

hipError_t launch_signal_reset(uint8_t* base, int64_t stride, int W, int64_t sig_off,
                               int64_t nslots, hipStream_t st);
hipError_t launch_zero_u64(uint64_t* p, int64_t n, hipStream_t st);
hipError_t launch_pipelined(const PipeArgs& a, int V, int grid, hipStream_t st);
hipError_t pipelined_blocks_per_cu(int V, int sync, int direct, int* n);
hipError_t launch_xcc_probe(uint32_t* out, int n, hipStream_t st);
hipError_t launch_two_phase(const TwoPhaseArgs& a, int V, hipStream_t st);
hipError_t launch_ag_gemm(const AgGemmArgs& a, int grid, hipStream_t st);
hipError_t launch_gemm_rs(const GemmRsArgs& a, int grid, hipStream_t st);
hipError_t gemm_rs_blocks_per_cu(int sync, bool f32p, int* n);
hipError_t launch_alltoallv(const A2vArgs& a, int V, int grid, hipStream_t st);
hipError_t alltoallv_blocks_per_cu(int V, int* n);
hipError_t ag_gemm_blocks_per_cu(int sync, int* n);
hipError_t launch_transpose_b(const uint16_t* b, uint16_t* bt, int64_t K, int64_t N, hipStream_t st);

// One-sided primitives.
hipError_t launch_put(uint8_t* dst, const uint8_t* src, int64_t bytes, hipStream_t st);
hipError_t launch_put_with_signal(uint8_t* dst, const uint8_t* src, int64_t bytes, uint64_t* sig,
                                  uint64_t value, int op, hipStream_t st);
hipError_t launch_signal_op(uint64_t* sig, uint64_t value, int op, hipStream_t st);
hipError_t launch_wait(const uint64_t* sig, int cmp, uint64_t value, uint64_t timeout,
                       uint32_t* err, hipStream_t st);

}  // namespace ra2a
