// gfx950 kernel of the AllGather + GEMM overlap: one persistent launch whose
// workgroups take tasks from one work queue per XCD (queue.h):
//   * AllGather part: copy a few rows of shard w (slice w) into G (slice rank),
//     release, count the part; the tile's last part sets its signal to 1
//     (put_with_signal per tile, the HyperParallel RFC section 六 / 十);
//   * GEMM tile: wait until every tile covering its kGemmBM rows is signalled,
//     then C[kGemmBM x kGemmBN] = G[rows, :] @ B[:, cols] on the matrix cores (bf16 in,
//     fp32 accumulation, bf16 out rounded to nearest even) -- "Triton-distributed
//     Semantics", sections "Producer-Consumer Model" and "AllGather + GEMM
//     Overlapping": the consumer waits only for its own tile.
//
// Shard w's tasks form stream group w mod NG, bound to one XCD (XCC_ID), so the
// rows a GEMM tile reads were written into the L2 it reads through; the part's
// release is then a drain plus a barrier (device.h).  With agent_sync the
// release writes the L2 back and the GEMM tile acquires device-wide instead.
#include <hip/hip_runtime.h>

#include <utility>

#include "ag_gemm_geom.h"
#include "gemm_rs_geom.h"
#include "common.h"
#include "device.h"
#include "launch.h"
#include "queue.h"

namespace ra2a {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---- the matrix-core tile ----------------------------------------------------
//
// One output tile of kTileM x kTileN = 256 x 256 per workgroup of eight waves, two
// per SIMD; wave (wm, wn) = (wave / 4, wave mod 4) owns 128 rows x 64 columns as
// 8 x 4 blocks of v_mfma_f32_16x16x32_bf16.  The operands are given to the
// instruction swapped (B^T block first), so that lane l of block (x, y) holds
// rows 16 x + l % 16 and four consecutive columns 16 y + 4 (l / 16) .. + 3 of the
// wave's part: the epilogue writes 8 (bf16) or 16 (fp32) contiguous bytes.
// (Lane layout of the instruction: A operand row l % 16, k 8 (l / 16) .. + 7; B
// operand column l % 16, the same k; result column l % 16, rows 4 (l / 16) .. +3 --
// checked on the device with exact integer inputs before this tile was written.)
// Measured on the product alone, in one box call: 8192 x 4096 x 7168 in 0.418-0.423
// ms against 0.428-0.436 ms with four waves of 128 x 128 (one per SIMD), and
// 8192 x 4096 x 896 in 0.065-0.066 against 0.077-0.078 ms: with two waves per SIMD
// one wave's prologue, waits and epilogue overlap the other's matrix work.
constexpr int kTileM = kGemmBM;
constexpr int kTileN = kGemmBN;
constexpr int kGemmThreads = 512;  // eight waves
constexpr int kGemmWgPerCu = 1;
constexpr int kStageK = 64;        // k per pipeline stage: 128 bytes, one cache line per row
constexpr int kSlotA = kTileM * kStageK * 2;   // bytes of A in a stage slot
constexpr int kSlotB = kTileN * kStageK * 2;
constexpr int kSlot = kSlotA + kSlotB;         // 64 KiB; the LDS ring holds two
constexpr int kLoadsPerStage = 8;              // 1 KiB LDS loads per wave per stage (4 of A, 4 of B^T)
constexpr int kReadsPerStep = 12;              // 16-byte fragment reads per wave per k32 step (8 A, 4 B^T)
constexpr int kMfmaPerStep = 32;               // 8 x 4 blocks
constexpr int kEpiPitch = kTileN * 2 + 16;     // bf16 output tile staged in LDS, bytes per row
constexpr int kLdsBytes = kTileM * kEpiPitch;  // the larger of the two uses
static_assert(2 * kSlot <= kLdsBytes, "LDS array");
static_assert(kLdsBytes + 1024 <= 160 * 1024, "the LDS of a CU holds the workgroup");

// float -> bf16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// LDS stage layout of an operand: its 256 rows x 64 k, 128 bytes per row as eight
// 16-byte chunks; logical chunk c of row r sits at position c ^ ((r >> 1) & 7).
// A fragment read takes 16 consecutive rows (starting at a multiple of 16) at one
// chunk: the eight even rows then cover the eight positions once, and so do the
// eight odd ones, which lie in the other half of the 64 banks -- no conflict
// whether the LDS serves 16 or 8 lanes a clock (the counter reads 0.3 %).

// Offset sent for a chunk that must read as zero: past any buffer's range.
constexpr uint32_t kOutOfRange = 0xFFFFFFF0u;

// Per-lane terms of the stage loads, fixed for a tile: lane l lands at byte 16 l of
// a 1 KiB LDS block, i.e. row 8 P' + l / 8 of the wave's rows, position l % 8, and
// fetches the logical chunk stored there.
struct LoadLane {
    uint32_t row_off;  // (l / 8) * K * 2
    int chunk;         // (l % 8) ^ ((l / 8) >> 1): the logical chunk for an even part
};

__device__ __forceinline__ LoadLane load_lane(int64_t K) {
    const int l = (int)threadIdx.x & 63;
    LoadLane ll;
    ll.row_off = (uint32_t)(l >> 3) * (uint32_t)K * 2u;
    asm volatile("" : "+v"(ll.row_off));  // computed once, not folded back into every load
    ll.chunk = (l & 7) ^ (l >> 4);
    return ll;
}

// Load P (0 .. 7) of this wave's share of a stage (k0 .. k0 + 63): loads 0-3 bring
// A rows 32 w + 8 P .., loads 4-7 B^T rows 32 w + 8 (P - 4) .. into the slot (A,
// then B^T).  Row r = 32 w + 8 P + l / 8 has (r >> 1) & 7 = (l >> 4) ^ 4 (P & 1).
// Rows past the operand's buffer (the descriptor's range), k past K, and a stage
// past the last (`live` false) read as zero: no branch around the load.
template <int P>
__device__ __forceinline__ void stage_load_part(__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                                char* slot, int w, uint32_t K, uint32_t k0,
                                                const LoadLane& ll, bool live) {
    constexpr bool kA = P < 4;
    const int rbase = 32 * w + 8 * (kA ? P : P - 4);
    const int chunk = ll.chunk ^ (4 * (P & 1));
    const uint32_t k = k0 + 8u * (uint32_t)chunk;
    const uint32_t off = (live && k < K) ? (uint32_t)rbase * K * 2u + ll.row_off + k * 2u : kOutOfRange;
    char* const dst = slot + (kA ? 0 : kSlotA) + rbase * 128;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(kA ? ra : rb, (__attribute__((address_space(3))) void*)dst,
                                             16, off, 0, 0, 0);
}

template <int... Ps>
__device__ __forceinline__ void stage_load_seq(__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb, char* slot,
                                               int w, uint32_t K, uint32_t k0, const LoadLane& ll,
                                               std::integer_sequence<int, Ps...>) {
    (stage_load_part<Ps>(ra, rb, slot, w, K, k0, ll, true), ...);
}

// 16-byte LDS reads at addr + OFF (OFF an immediate).  Written as inline assembly
// on purpose: the compiler cannot tell these reads apart from the LDS slots still
// being filled by the direct loads of later stages, and before every LDS read it
// would wait for all of those loads (vmcnt(0)), serialising the pipeline.  The
// stage being read is complete for every wave (the stage barrier); the caller
// waits for the reads with lds_wait.
template <int OFF>
__device__ __forceinline__ bf16x8 lds_read16(uint32_t addr) {
    bf16x8 v;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
    return v;
}

// A wave's fragments of one k32 step: 8 A blocks (rows 16 x ..) and 4 B^T blocks.
struct Frags {
    bf16x8 a[8], b[4];
};

// Wait until this wave's LDS reads are in; the fragments are tied to the wait so
// that no use of them is scheduled above it.
__device__ __forceinline__ void lds_wait(Frags& f) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    asm volatile("" : "+v"(f.a[0]), "+v"(f.a[1]), "+v"(f.a[2]), "+v"(f.a[3]), "+v"(f.a[4]), "+v"(f.a[5]),
                      "+v"(f.a[6]), "+v"(f.a[7]));
    asm volatile("" : "+v"(f.b[0]), "+v"(f.b[1]), "+v"(f.b[2]), "+v"(f.b[3]));
}

// LDS byte address of a pointer into the LDS array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// Fragment read I (0-7: A block I, 8-11: B^T block I - 8); blocks are 16 rows =
// 2 KiB apart, and the lane's swizzled chunk is the same in every block.
template <int I>
__device__ __forceinline__ void read_frag(Frags& f, uint32_t a_addr, uint32_t b_addr) {
    if constexpr (I < 8)
        f.a[I] = lds_read16<I * 2048>(a_addr);
    else
        f.b[I - 8] = lds_read16<(I - 8) * 2048>(b_addr);
}

template <int... Is>
__device__ __forceinline__ void read_frags_seq(Frags& f, uint32_t a, uint32_t b, std::integer_sequence<int, Is...>) {
    (read_frag<Is>(f, a, b), ...);
}

__device__ __forceinline__ void sb() { __builtin_amdgcn_sched_barrier(0); }

template <int I>
__device__ __forceinline__ void mma_one(f32x4 (&acc)[8][4], const Frags& f) {
    constexpr int x = I / 4, y = I % 4;
    acc[x][y] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.b[y], f.a[x], acc[x][y], 0, 0, 0);
}

// A k32 step: its 32 MFMAs with the other work of the step between them -- the 12
// fragment reads of the next step after MFMAs 0 .. 11 (they land well before the
// step ends), and, in the second step of a stage, the 8 loads refilling the slot
// just freed after MFMAs 0, 2, .., 14: as early as the slot is free, which gives
// them the most time before the wait for them one step later (1.5-3 % faster than
// refills on the last 16 MFMAs, same box; the reads on MFMAs 0 .. 11 rather than
// on every second MFMA, another 0.5-1 %).
struct StepCtx {
    Frags* next;
    uint32_t na, nb;                      // the next step's fragment addresses
    __amdgpu_buffer_rsrc_t ra, rb;
    char* slot;                           // the slot to refill
    int w;
    uint32_t K, k0;                       // the stage it is refilled with
    const LoadLane* ll;
    bool live;
};

template <bool REFILL, int I, int J>
__device__ __forceinline__ void step_op(const StepCtx& c) {
    if constexpr (J < kReadsPerStep) {
        if constexpr (J == I) {
            read_frag<J>(*c.next, c.na, c.nb);
            sb();
        }
    } else if constexpr (REFILL) {
        if constexpr ((J - kReadsPerStep) * 2 == I) {
            stage_load_part<J - kReadsPerStep>(c.ra, c.rb, c.slot, c.w, c.K, c.k0, *c.ll, c.live);
            sb();
        }
    }
}
template <bool REFILL, int I, int... Js>
__device__ __forceinline__ void step_ops(const StepCtx& c, std::integer_sequence<int, Js...>) {
    (step_op<REFILL, I, Js>(c), ...);
}
template <bool REFILL, int... Is>
__device__ __forceinline__ void k32_step(f32x4 (&acc)[8][4], const Frags& f, const StepCtx& c,
                                         std::integer_sequence<int, Is...>) {
    ((mma_one<Is>(acc, f), sb(),
      step_ops<REFILL, Is>(c, std::make_integer_sequence<int, kReadsPerStep + kLoadsPerStage>{})),
     ...);
}

// Main loop of one kTileM x kTileN output tile: acc = the fp32 accumulators of
// C[i, n] = sum_k A[i, k] B^T[n, k] for the rows_valid rows of A at a_rows and the
// cols_valid rows of B^T at bt_rows (both K-contiguous bf16, K a multiple of 8);
// rows and columns past those counts accumulate zeros.  Lane l of wave (wm, wn)
// holds in acc[x][y] the rows 128 wm + 16 x + l % 16, columns 128 wn + 16 y +
// 4 (l / 16) .. + 3.  `lds` is the workgroup's LDS array (kLdsBytes); on return
// every wave is out of it and no load is in flight.
//
// Stores the caller issued before are not waited for first: the first stage's wait
// (vector memory operations complete in issue order) and barrier cover them, after
// which, if `pend` is set, wave 0 publishes them (with `agent`, an L2 write-back
// first) by setting the signal at `pend` to 1.
__device__ __forceinline__ void gemm_mainloop(f32x4 (&acc)[8][4], const uint16_t* a_rows, int rows_valid,
                                              const uint16_t* bt_rows, int cols_valid, int64_t K64,
                                              char* lds, uint64_t* pend = nullptr, bool agent = false) {
    // K opaque per tile: nothing derived from it is hoisted out of the persistent
    // task loop and kept alive across tiles.
    asm volatile("" : "+s"(K64));
    const uint32_t K = (uint32_t)K64;  // the host keeps 256 K 2 below 2^32
    const __amdgpu_buffer_rsrc_t ra = make_rsrc_uniform(a_rows, (uint32_t)rows_valid * K * 2u);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc_uniform(bt_rows, (uint32_t)cols_valid * K * 2u);
    const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int l = (int)threadIdx.x & 63;
    const int wm = w >> 2, wn = w & 3;
#pragma unroll
    for (int x = 0; x < 8; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int nk = (int)((K + kStageK - 1) / kStageK);
    const LoadLane ll = load_lane(K64);
    char* const slot0 = lds;
    char* const slot1 = lds + kSlot;
    // Stage s lives in slot s mod 2; both are loaded up front (the second only if
    // its stage exists), and stage 0 lands before the first reads.
    constexpr auto kParts = std::make_integer_sequence<int, kLoadsPerStage>{};
    stage_load_seq(ra, rb, slot0, w, K, 0, ll, kParts);
    if (nk > 1) {
        stage_load_seq(ra, rb, slot1, w, K, kStageK, ll, kParts);
        asm volatile("s_waitcnt vmcnt(%0)" ::"i"(kLoadsPerStage) : "memory");
    } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __builtin_amdgcn_s_barrier();
    if (pend != nullptr) {  // every wave's earlier stores are complete
        if (agent && threadIdx.x < 64) fence_release_agent();
        if (threadIdx.x == 0) sig_update(pend, 1ull, kSigSet);
    }
    // Fragment offsets inside a slot: row 128 wm + l % 16 (then + 16 x), logical chunk
    // l / 16 (+ 4 in the second k32 step: position ^ 4, byte ^ 64).
    const uint32_t sw = (uint32_t)((l >> 4) ^ ((l & 15) >> 1)) * 16u;
    const uint32_t oa = (uint32_t)((128 * wm + (l & 15)) * 128) + sw;
    const uint32_t ob = (uint32_t)kSlotA + (uint32_t)((64 * wn + (l & 15)) * 128) + sw;
    const uint32_t base0 = lds_addr(slot0);
    Frags f0, f1;
    read_frags_seq(f0, base0 + oa, base0 + ob, std::make_integer_sequence<int, kReadsPerStep>{});
    // Per stage s (two k32 steps):
    //   step 0: MFMAs of f0 = (s, k 0..31), reads f1 <- (s, k 32..63)
    //   wait for f1 (every read of stage s is in) and for stage s+1 (the only loads in
    //   flight), barrier: every wave is done with slot s mod 2
    //   step 1: MFMAs of f1, reads f0 <- (s+1, k 0..31), loads refilling slot s mod 2
    //           with stage s+2 (zeros past the last stage)
    // The last iteration reads f0 of a stage past the end (stale contents, unused);
    // those reads are drained after the loop, and the zero-filling loads too, before
    // the epilogue reuses the LDS.
    constexpr auto kSeq = std::make_integer_sequence<int, kMfmaPerStep>{};
    for (int s = 0; s < nk; ++s) {
        const uint32_t cs = base0 + (uint32_t)((s & 1) * kSlot);
        const uint32_t ns = base0 + (uint32_t)(((s + 1) & 1) * kSlot);
        char* const freed = (s & 1) ? slot1 : slot0;
        lds_wait(f0);
        sb();
        k32_step<false>(acc, f0, StepCtx{&f1, (cs + oa) ^ 64u, (cs + ob) ^ 64u, ra, rb, freed, w, K, 0, &ll, false},
                        kSeq);
        lds_wait(f1);
        if (s + 1 < nk) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // stage s+1 has landed
        __builtin_amdgcn_s_barrier();
        sb();
        k32_step<true>(acc, f1,
                       StepCtx{&f0, ns + oa, ns + ob, ra, rb, freed, w, K, (uint32_t)(s + 2) * kStageK, &ll,
                               s + 2 < nk},
                       kSeq);
    }
    lds_wait(f0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no load may still write the LDS
    __builtin_amdgcn_s_barrier();  // every wave is out of the ring
}

// Epilogue: the tile's rows_valid x cols_valid corner of acc, rounded to bf16
// (nearest even), stored at c (row stride ldc elements) through the LDS; with
// NTOUT the 16-byte pieces are stored non-temporally.
template <bool NTOUT>
__device__ __forceinline__ void epi_bf16(const f32x4 (&acc)[8][4], int rows_valid, int cols_valid, void* c,
                                         int64_t ldc, char* lds) {
    asm volatile("" : "+s"(ldc));
    const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int l = (int)threadIdx.x & 63;
    const int wm = w >> 2, wn = w & 3;
    // (The empty asm makes the output pointer opaque here, so that the epilogue's
    // addresses are not hoisted above the main loop and kept alive across it.)
    uint64_t cbase = reinterpret_cast<uint64_t>(c);
    asm volatile("" : "+v"(cbase));
    // bf16: round into the LDS tile (8 bytes per lane and block), then write it
    // out as 16-byte row pieces
#pragma unroll
    for (int x = 0; x < 8; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) {
            const int row = 128 * wm + 16 * x + (l & 15);
            const int col = 64 * wn + 16 * y + 4 * (l >> 4);
            u32x2 v;
            v[0] = bf16_rne(acc[x][y][0]) | (bf16_rne(acc[x][y][1]) << 16);
            v[1] = bf16_rne(acc[x][y][2]) | (bf16_rne(acc[x][y][3]) << 16);
            *reinterpret_cast<u32x2*>(lds + row * kEpiPitch + col * 2) = v;
        }
    __syncthreads();
    // 16-byte pieces need a 16-byte aligned output and a row stride of whole pieces
    const bool vec = (cbase & 15u) == 0 && (ldc & 7) == 0;
    constexpr int kPieces = kTileM * kTileN / 8;
    for (int i = (int)threadIdx.x; i < kPieces; i += kGemmThreads) {
        const int row = i / (kTileN / 8);
        const int col0 = (i - row * (kTileN / 8)) * 8;
        if (row >= rows_valid || col0 >= cols_valid) continue;
        const u32x4 v = *reinterpret_cast<const u32x4*>(lds + row * kEpiPitch + col0 * 2);
        uint16_t* const dst = reinterpret_cast<uint16_t*>(cbase) + (int64_t)row * ldc + col0;
        if (vec && col0 + 8 <= cols_valid) {
            if (NTOUT)
                __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst));
            else
                *reinterpret_cast<u32x4*>(dst) = v;
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k)
                if (col0 + k < cols_valid) dst[k] = (uint16_t)(v[k >> 1] >> (16 * (k & 1)));
        }
    }
    __builtin_amdgcn_s_barrier();  // the LDS is free for the next tile
}

// One output tile, stored as bf16.
template <bool NTOUT>
__device__ __forceinline__ void gemm_tile(const uint16_t* a_rows, int rows_valid, const uint16_t* bt_rows,
                                          int cols_valid, int64_t K, void* c, int64_t ldc, char* lds) {
    f32x4 acc[8][4];
    gemm_mainloop(acc, a_rows, rows_valid, bt_rows, cols_valid, K, lds);
    epi_bf16<NTOUT>(acc, rows_valid, cols_valid, c, ldc, lds);
}

// B (K x N, row-major) -> B^T (N x K): each lane transposes one 8 x 8 block in
// registers; a wave covers 8 x 8 blocks so that both its loads (rows of B) and
// its stores (rows of B^T) are 128 contiguous bytes per group of 8 lanes.
__global__ void __launch_bounds__(256) transpose_b_kernel(const uint16_t* __restrict__ b,
                                                          uint16_t* __restrict__ bt, int64_t K,
                                                          int64_t N) {
    const int l = (int)threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t nwb = (N + 63) / 64;  // wave tiles along N
    const int64_t k0 = (wave / nwb) * 64 + 8 * (l & 7);
    const int64_t n0 = (wave % nwb) * 64 + 8 * (l >> 3);
    if (k0 >= K || n0 >= N) return;
    u32x4 in[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) in[kk] = *reinterpret_cast<const u32x4*>(b + (k0 + kk) * N + n0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        u32x4 lo, hi;  // columns n0 + 2j and n0 + 2j + 1
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            lo[q] = __builtin_amdgcn_perm(in[2 * q + 1][j], in[2 * q][j], 0x05040100u);
            hi[q] = __builtin_amdgcn_perm(in[2 * q + 1][j], in[2 * q][j], 0x07060302u);
        }
        *reinterpret_cast<u32x4*>(bt + (n0 + 2 * j) * K + k0) = lo;
        *reinterpret_cast<u32x4*>(bt + (n0 + 2 * j + 1) * K + k0) = hi;
    }
}

hipError_t launch_transpose_b(const uint16_t* b, uint16_t* bt, int64_t K, int64_t N, hipStream_t st) {
    const int64_t waves = ((K + 63) / 64) * ((N + 63) / 64);
    hipLaunchKernelGGL(transpose_b_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st, b, bt, K, N);
    return hipGetLastError();
}

template <int SYNC>
__global__ void __launch_bounds__(kGemmThreads, kGemmWgPerCu) ag_gemm_kernel(AgGemmArgs a) {
    __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];  // the ring, or the staged output tile
    __shared__ int lds_flag;
    __shared__ int64_t lds_pos[2];
    constexpr bool kOwned = SYNC == kSyncXcd;
    uint8_t* const mine = a.base + (int64_t)a.rank * a.stride;
    uint64_t* const sig = reinterpret_cast<uint64_t*>(mine + a.sig_off);
    uint64_t* const qw = sig + agg_queue_slot(a) * kSigStrideU64;
    uint16_t* const G = reinterpret_cast<uint16_t*>(mine + a.g_off);
    const uint32_t xcc = xcc_id();
    const int home = SYNC == kSyncXcd ? (int)(xcc % (uint32_t)a.NG) : (int)(blockIdx.x % a.NG);
    const int64_t total = a.ntasks_shard * a.spg;
    QueueClaim qc;
    int k = 0;
    for (int gi = 0; gi < a.NG; ++gi) {
        const int g = (home + gi) % a.NG;
        if (threadIdx.x == 0) lds_pos[k & 1] = queue_first<kOwned>(qw, g, gi, xcc, qc);
        __syncthreads();
        int64_t pos = (int64_t)__builtin_amdgcn_readfirstlane((int)lds_pos[k & 1]);
        ++k;
        if (pos < 0) continue;
        while (true) {
            // the group's queue: spg shards of ntasks_shard each (the last group may
            // have fewer real shards; their tasks are skipped)
            if (pos >= total) {
                if (threadIdx.x == 0) queue_drained(qw, g, pos, total, qc);
                break;
            }
            uint64_t nxt = 0;
            if (threadIdx.x == 0) nxt = queue_next(qc);
            const AgTask t = agg_task_of(a, g, pos);
            if (t.w < a.W) {
                if (!t.gemm) {
                    // AllGather part: rows [row0, row0 + rows) of shard w -> G
                    const int64_t bytes = t.rows * a.K * 2;
                    const uint8_t* src = a.base + (int64_t)t.w * a.stride + a.a_off + t.row0 * a.K * 2;
                    uint8_t* dst = reinterpret_cast<uint8_t*>(G + ((int64_t)t.w * a.m_local + t.row0) * a.K);
                    // shard rows are read once: non-temporal loads; G is read back by
                    // this XCD's GEMM tiles: ordinary stores (2-4 % faster in one box
                    // call than ordinary loads, and than non-temporal stores)
                    copy_flat<16, 8, true, false>(src, dst, bytes, threadIdx.x, kGemmThreads);
                    group_release<SYNC>();
                    if (threadIdx.x == 0) {
                        const uint64_t done = __hip_atomic_fetch_add(sig + agg_count_slot(a, t.w, t.tile) * kSigStrideU64,
                                                                     1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        if (done + 1 == (uint64_t)agg_parts_of_tile(a, t.tile))
                            sig_update(sig + agg_sig_slot(a, t.w, t.tile) * kSigStrideU64, 1ull, kSigSet);
                    }
                } else {
                    int first, last;
                    agg_block_tiles(a, t.mb, &first, &last);
                    if (!group_wait_all<SYNC == kSyncAgent>(sig + agg_sig_slot(a, t.w, first) * kSigStrideU64,
                                                            kSigStrideU64 * 8, last - first, kCmpEq, 1ull,
                                                            a.timeout, a.err, &lds_flag))
                        return;
                    const int64_t row0 = (int64_t)t.w * a.m_local + (int64_t)t.mb * kGemmBM;
                    int64_t rv = a.m_local - (int64_t)t.mb * kGemmBM;
                    const int rows_valid = rv < kGemmBM ? (int)rv : kGemmBM;
                    const int64_t n0 = (int64_t)t.nb * kGemmBN;
                    const int cols_valid = a.N - n0 < kGemmBN ? (int)(a.N - n0) : kGemmBN;
                    gemm_tile<false>(G + row0 * a.K, rows_valid, a.bt + n0 * a.K, cols_valid, a.K,
                                            a.c + row0 * a.N + n0, a.N, lds);
                }
            }
            if (threadIdx.x == 0) lds_pos[k & 1] = (int64_t)nxt;
            __syncthreads();
            pos = (int64_t)__builtin_amdgcn_readfirstlane((int)lds_pos[k & 1]);
            ++k;
        }
    }
}

// ---------------------------------------------------------------------------
// GEMM + ReduceScatter (gemm_rs_geom.h): one persistent launch over one work
// queue per XCD.  Destination j's tasks form group j mod NG, bound to one XCD
// like the AllGather's, so the partials the receiver's task reads were written
// into the L2 it reads through.

// A partial tile in the lanes' own order: thread t's 16-byte piece number b --
// block (x, y), b = 4 x + y, as fp32; or blocks (x, 2 p) and (x, 2 p + 1), b =
// 2 x + p, as bf16 rounded to nearest even -- at byte 8192 b + 16 t of the
// tile's slot (512 threads).  Stored non-temporally: each partial is read once, by the
// receiver's task.
constexpr int kRsPieceBytes = kGemmThreads * 16;

__device__ __forceinline__ u32x4 bits(f32x4 v) { return __builtin_bit_cast(u32x4, v); }

template <bool F32P>
__device__ __forceinline__ void rs_store_partial(const f32x4 (&acc)[8][4], __amdgpu_buffer_rsrc_t rp,
                                                 uint32_t slot) {
    const uint32_t off = slot + threadIdx.x * 16u;
    if constexpr (F32P) {
#pragma unroll
        for (int b = 0; b < 32; ++b)
            BufStore<16, kPolicyNt>::go(bits(acc[b >> 2][b & 3]), rp, off + (uint32_t)(b * kRsPieceBytes));
    } else {
#pragma unroll
        for (int b = 0; b < 16; ++b) {
            const f32x4 u = acc[b >> 1][2 * (b & 1)], v = acc[b >> 1][2 * (b & 1) + 1];
            const u32x4 o = {bf16_rne(u[0]) | (bf16_rne(u[1]) << 16), bf16_rne(u[2]) | (bf16_rne(u[3]) << 16),
                             bf16_rne(v[0]) | (bf16_rne(v[1]) << 16), bf16_rne(v[2]) | (bf16_rne(v[3]) << 16)};
            BufStore<16, kPolicyNt>::go(o, rp, off + (uint32_t)(b * kRsPieceBytes));
        }
    }
}

// The receiver's own partial as the sum takes it: its accumulators, or those
// rounded to bf16 like every other partial.
template <bool F32P>
__device__ __forceinline__ f32x4 rs_own(f32x4 v) {
    if constexpr (F32P) {
        return v;
    } else {
        return f32x4{__uint_as_float(bf16_rne(v[0]) << 16), __uint_as_float(bf16_rne(v[1]) << 16),
                     __uint_as_float(bf16_rne(v[2]) << 16), __uint_as_float(bf16_rne(v[3]) << 16)};
    }
}

// Half h of a bf16 piece: the four values of one block.
__device__ __forceinline__ f32x4 rs_unpack_bf16(u32x4 x, int h) {
    const uint32_t lo = x[2 * h], hi = x[2 * h + 1];
    return f32x4{__uint_as_float(lo << 16), __uint_as_float(lo & 0xFFFF0000u), __uint_as_float(hi << 16),
                 __uint_as_float(hi & 0xFFFF0000u)};
}

// The receiver's task: acc <- sum over r = 0..W-1, in that order, of the tile's
// partials in fp32, its own (acc, see rs_own) in place r == j; slot r at byte
// tile_off + r src_stride of the receive area.  The partials are read with
// device-scope non-temporal loads (never from the CU's L1); the loads of
// kFoldPieces pieces of up to kFoldSrc sources are in flight together (a source
// past W, or j itself, is sent out of range and reads zero without touching
// memory; a select, not a branch, drops it, so no load waits behind a test).
// (4 sources x 4 pieces measured 1.5-2.5 % faster than 8 x 2 and 8 x 1, in one box call)
constexpr int kFoldSrc = 4;
constexpr int kFoldPieces = 4;

// Pieces P0 .. P0 + kFoldPieces - 1 (a template parameter, so that every index
// into acc is a constant and acc stays in registers).
template <bool F32P, int P0>
__device__ __forceinline__ void rs_fold_group(f32x4 (&acc)[8][4], __amdgpu_buffer_rsrc_t rp, uint32_t tile_off,
                                              uint32_t src_stride, int j, int W) {
    constexpr int kBlk = F32P ? 1 : 2;  // blocks per piece
    using Load = BufLoad<16, kPolicySc1 | kPolicyNt>;
    const uint32_t t16 = threadIdx.x * 16u;
    f32x4 s[kFoldPieces * kBlk];
#pragma unroll
    for (int i = 0; i < kFoldPieces * kBlk; ++i) s[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int src0 = 0; src0 < W; src0 += kFoldSrc) {
        u32x4 x[kFoldSrc][kFoldPieces];
#pragma unroll
        for (int g = 0; g < kFoldSrc; ++g) {
            const int src = src0 + g;
            const bool load = src < W && src != j;
            const uint32_t base = tile_off + (uint32_t)src * src_stride + t16;
#pragma unroll
            for (int q = 0; q < kFoldPieces; ++q)
                x[g][q] = Load::go(rp, load ? base + (uint32_t)((P0 + q) * kRsPieceBytes) : kOutOfRange);
        }
#pragma unroll
        for (int g = 0; g < kFoldSrc; ++g) {
            const int src = src0 + g;
#pragma unroll
            for (int q = 0; q < kFoldPieces; ++q)
#pragma unroll
                for (int h = 0; h < kBlk; ++h) {
                    const int b = (P0 + q) * kBlk + h;  // block 4 x + y
                    const f32x4 v = src == j ? rs_own<F32P>(acc[b >> 2][b & 3])
                                             : (F32P ? __builtin_bit_cast(f32x4, x[g][q]) : rs_unpack_bf16(x[g][q], h));
                    f32x4& t = s[q * kBlk + h];
                    t = src < W ? t + v : t;
                }
        }
    }
#pragma unroll
    for (int q = 0; q < kFoldPieces; ++q)
#pragma unroll
        for (int h = 0; h < kBlk; ++h) {
            const int b = (P0 + q) * kBlk + h;
            acc[b >> 2][b & 3] = s[q * kBlk + h];
        }
}

template <bool F32P, int... Gs>
__device__ __forceinline__ void rs_fold_groups(f32x4 (&acc)[8][4], __amdgpu_buffer_rsrc_t rp, uint32_t tile_off,
                                               uint32_t src_stride, int j, int W, std::integer_sequence<int, Gs...>) {
    (rs_fold_group<F32P, Gs * kFoldPieces>(acc, rp, tile_off, src_stride, j, W), ...);
}

template <bool F32P>
__device__ __forceinline__ void rs_fold(f32x4 (&acc)[8][4], __amdgpu_buffer_rsrc_t rp, uint32_t tile_off,
                                        uint32_t src_stride, int j, int W) {
    constexpr int kPieces = F32P ? 32 : 16;
    rs_fold_groups<F32P>(acc, rp, tile_off, src_stride, j, W,
                         std::make_integer_sequence<int, kPieces / kFoldPieces>{});
}

template <int SYNC, bool F32P>
__global__ void __launch_bounds__(kGemmThreads, kGemmWgPerCu) gemm_rs_kernel(GemmRsArgs a) {
    __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
    __shared__ int lds_flag;
    __shared__ int64_t lds_pos[2];
    constexpr bool kOwned = SYNC == kSyncXcd;
    uint64_t* const qw = reinterpret_cast<uint64_t*>(a.base + a.sig_off) + grs_queue_slot(a) * kSigStrideU64;
    const uint32_t xcc = xcc_id();
    const int home = SYNC == kSyncXcd ? (int)(xcc % (uint32_t)a.NG) : (int)(blockIdx.x % a.NG);
    const int64_t total = a.ntasks_dest * a.dpg;
    // the receive area (W slots of ntiles partial tiles) is below 4 GiB (host check)
    const uint32_t src_stride = (uint32_t)grs_part_offset(a, 1, 0);
    const uint32_t area = (uint32_t)grs_part_offset(a, a.W, 0);
    QueueClaim qc;
    int k = 0;
    // The (tile, r) signal of the partial this workgroup stored last, not set yet: its
    // stores drain under the next task's first loads, whose wait covers them
    // (gemm_mainloop sets it), or at the latest before the workgroup leaves a queue.
    uint64_t* pend = nullptr;
    for (int gi = 0; gi < a.NG; ++gi) {
        const int g = (home + gi) % a.NG;
        if (threadIdx.x == 0) lds_pos[k & 1] = queue_first<kOwned>(qw, g, gi, xcc, qc);
        __syncthreads();
        int64_t pos = (int64_t)__builtin_amdgcn_readfirstlane((int)lds_pos[k & 1]);
        ++k;
        if (pos < 0) continue;
        while (true) {
            // the group's queue: dpg destinations of ntasks_dest each (the last
            // group may have fewer real destinations; their tasks are skipped)
            if (pos >= total) {
                if (pend != nullptr) {
                    group_release<SYNC>();
                    if (threadIdx.x == 0) sig_update(pend, 1ull, kSigSet);
                    pend = nullptr;
                }
                if (threadIdx.x == 0) queue_drained(qw, g, pos, total, qc);
                break;
            }
            uint64_t nxt = 0;
            if (threadIdx.x == 0) nxt = queue_next(qc);
            const RsTask t = grs_group_task(a, g, pos);
            if (t.j < a.W) {
                // rank r's partial of the tile: rows j*mj + mb*256 .. of x1_r, rows
                // nb*256 .. of x2_r^T
                uint8_t* const dst_slice = a.base + (int64_t)t.j * a.stride;
                uint64_t* const sig = reinterpret_cast<uint64_t*>(dst_slice + a.sig_off);
                int mb, nb;
                grs_tile(a, t.tile, &mb, &nb);
                const int64_t row0 = (int64_t)mb * kRsTileM, col0 = (int64_t)nb * kRsTileN;
                const int rows = a.mj - row0 < kRsTileM ? (int)(a.mj - row0) : kRsTileM;
                const int cols = a.N - col0 < kRsTileN ? (int)(a.N - col0) : kRsTileN;
                const uint8_t* const src_slice = a.base + (int64_t)t.r * a.stride;
                const uint16_t* x1 = reinterpret_cast<const uint16_t*>(src_slice + a.a_off) +
                                     ((int64_t)t.j * a.mj + row0) * a.K;
                const uint16_t* x2t = reinterpret_cast<const uint16_t*>(src_slice + a.bt_off) + col0 * a.K;
                f32x4 acc[8][4];
                gemm_mainloop(acc, x1, rows, x2t, cols, a.K, lds, pend, SYNC == kSyncAgent);
                pend = nullptr;
                const __amdgpu_buffer_rsrc_t rp = make_rsrc_uniform(dst_slice + a.p_off, area);
                if (t.r != t.j) {
                    // into slot r of j's receive area; the (tile, r) signal follows once
                    // the stores have drained
                    rs_store_partial<F32P>(acc, rp, (uint32_t)grs_part_offset(a, t.r, t.tile));
                    pend = sig + grs_sig_slot(a, t.tile, t.r) * kSigStrideU64;
                } else {
                    // the other sources' partials: signals (tile, 0 .. j-1), (tile, j+1 .. W-1)
                    uint64_t* const s0 = sig + grs_sig_slot(a, t.tile, 0) * kSigStrideU64;
                    if (!group_wait_all<SYNC == kSyncAgent>(s0, kSigStrideU64 * 8, t.j, kCmpEq, 1ull, a.timeout,
                                                            a.err, &lds_flag) ||
                        !group_wait_all<SYNC == kSyncAgent>(s0 + (int64_t)(t.j + 1) * kSigStrideU64,
                                                            kSigStrideU64 * 8, a.W - 1 - t.j, kCmpEq, 1ull,
                                                            a.timeout, a.err, &lds_flag))
                        return;
                    rs_fold<F32P>(acc, rp, (uint32_t)grs_part_offset(a, 0, t.tile), src_stride, t.j, a.W);
                    epi_bf16<true>(acc, rows, cols, dst_slice + a.out_off + (row0 * a.N + col0) * 2, a.N, lds);
                    // (tile, j): the tile of out_j is complete, once its stores have drained
                    pend = sig + grs_sig_slot(a, t.tile, t.j) * kSigStrideU64;
                }
            }
            if (threadIdx.x == 0) lds_pos[k & 1] = (int64_t)nxt;
            __syncthreads();
            pos = (int64_t)__builtin_amdgcn_readfirstlane((int)lds_pos[k & 1]);
            ++k;
        }
    }
}

static const void* gemm_rs_fn(int sync, bool f32p) {
    if (sync == kSyncXcd)
        return f32p ? reinterpret_cast<const void*>(&gemm_rs_kernel<kSyncXcd, true>)
                    : reinterpret_cast<const void*>(&gemm_rs_kernel<kSyncXcd, false>);
    return f32p ? reinterpret_cast<const void*>(&gemm_rs_kernel<kSyncAgent, true>)
                : reinterpret_cast<const void*>(&gemm_rs_kernel<kSyncAgent, false>);
}

hipError_t launch_gemm_rs(const GemmRsArgs& a, int grid, hipStream_t st) {
    void* args[] = {const_cast<GemmRsArgs*>(&a)};
    return hipLaunchKernel(gemm_rs_fn(a.sync, a.f32p != 0), dim3(grid), dim3(kGemmThreads), args, 0, st);
}

hipError_t gemm_rs_blocks_per_cu(int sync, bool f32p, int* n) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(n, gemm_rs_fn(sync, f32p), kGemmThreads, 0);
}

hipError_t launch_ag_gemm(const AgGemmArgs& a, int grid, hipStream_t st) {
    void* args[] = {const_cast<AgGemmArgs*>(&a)};
    const void* fn = a.sync == kSyncXcd ? reinterpret_cast<const void*>(&ag_gemm_kernel<kSyncXcd>)
                                        : reinterpret_cast<const void*>(&ag_gemm_kernel<kSyncAgent>);
    return hipLaunchKernel(fn, dim3(grid), dim3(kGemmThreads), args, 0, st);
}

hipError_t ag_gemm_blocks_per_cu(int sync, int* n) {
    const void* fn = sync == kSyncXcd ? reinterpret_cast<const void*>(&ag_gemm_kernel<kSyncXcd>)
                                      : reinterpret_cast<const void*>(&ag_gemm_kernel<kSyncAgent>);
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(n, fn, kGemmThreads, 0);
}

}  // namespace ra2a
