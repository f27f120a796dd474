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
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTileM = kGemmBM;   // output rows of a tile (rows of A)
constexpr int kTileN = kGemmBN;   // output columns of a tile (rows of B^T)
constexpr int kGemmWaves = kTileM / 32;  // waves (wm, wn), wm = wave / 2, wn = wave mod 2
constexpr int kGemmThreads = 64 * kGemmWaves;
constexpr int kGemmWgPerCu = 512 / kGemmThreads;  // two waves per SIMD in all
constexpr int kWaveRows = 64;      // each wave owns 64 x 128 outputs of the tile
constexpr int kWaveCols = 128;
static_assert(kWaveRows * (kGemmWaves / 2) == kTileM && kWaveCols * 2 == kTileN,
              "the waves tile the output tile");
constexpr int kBlkA = kWaveRows / 32;  // 32 x 32 MFMA blocks per wave along rows
constexpr int kBlkB = kWaveCols / 32;  // ... and along columns
// k per pipeline stage: 64 bf16 = 128 bytes of an operand row, one whole cache
// line, so that each LDS load instruction fetches 8 whole lines.  With 32-k
// stages an instruction fetched 16 half lines and the loads filled LDS at 21 B
// per clock per CU against 36 B with whole lines (measured): below the 32 B per
// clock the matrix cores need at their peak for a 256 x 256 tile.
constexpr int kStageK = 64;
constexpr int kChunks = kStageK / 8;       // 16-byte chunks per operand row of a stage
constexpr int kStages = 2;                 // LDS ring depth: one stage computed, one landing
constexpr int kStageA = kTileM * kStageK;  // bf16 of A per stage
constexpr int kStageB = kTileN * kStageK;  // bf16 of B^T per stage
constexpr int kSlotElems = kStageA + kStageB;
constexpr int kRowsA = kTileM / kGemmWaves;  // A rows each wave loads per stage
constexpr int kRowsB = kTileN / kGemmWaves;  // B^T rows each wave loads per stage
constexpr int kDmaRows = 64 / kChunks;       // rows per LDS load instruction (1 KiB)
constexpr int kDmaA = kRowsA / kDmaRows, kDmaB = kRowsB / kDmaRows;  // a wave's LDS loads per stage
constexpr int kDmaPerStage = kDmaA + kDmaB;
static_assert(kRowsA % kDmaRows == 0 && kRowsB % kDmaRows == 0, "whole LDS load instructions");
constexpr int kKSteps = kStageK / 16;      // k16 MFMA steps per stage
static_assert(kKSteps == 4, "the main loop runs four k16 quarters per stage");
// bf16 epilogue: the output tile staged in LDS, rows padded by 16 bytes so that the
// two rows one write instruction touches fall in different banks
constexpr int kEpiPitch = kTileN * 2 + 16;                   // bytes per staged row
constexpr int kLdsElems = (kStages * kSlotElems) > (kTileM * kEpiPitch / 2)
                              ? (kStages * kSlotElems)
                              : (kTileM * kEpiPitch / 2);    // uint16 elements of the LDS array
static_assert(2 * kLdsElems * kGemmWgPerCu + 1024 <= 160 * 1024, "the LDS of a CU holds its workgroups");
// fp32 epilogue: half the tile's rows at a time, rows padded by 32 bytes (the two
// rows one write instruction touches then fall in the two halves of the banks)
constexpr int kEpiRows32 = kTileM / 2;
constexpr int kEpiPitch32 = kTileN * 4 + 32;
static_assert(kEpiRows32 * kEpiPitch32 <= 2 * kLdsElems, "the fp32 half tile must fit the LDS array");
static_assert(kWaveRows <= kEpiRows32 && kEpiRows32 % kWaveRows == 0, "a wave's rows lie in one half");

// float -> bf16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// LDS stage layout of an operand: its tile rows x 64 k (128 bytes per row, eight
// 16-byte chunks).  Chunk c of row r is stored at position c ^ g(r),
// g(r) = (r ^ ((r >> 3) & 3)) & 7.  A fragment read takes 32 consecutive rows at
// one chunk (lanes 0-31) and the same rows at the next chunk (lanes 32-63).  With
// 64 banks serving 16 lanes a clock (the model the bank-conflict counter bore
// out for 64-byte rows) the even rows of any 16 then cover the 8 chunk positions
// once, and so do the odd rows; with 32 banks serving 8 lanes a clock, any 8
// consecutive rows cover them once.  g depends on r mod 32 only, so the blocks
// of a wave (rows + 32 x) sit at fixed offsets.
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r ^ ((r >> 3) & 3)) & 7); }

// Offset sent for a chunk that must read as zero: past any buffer's range.
constexpr uint32_t kOutOfRange = 0xFFFFFFF0u;

// One of the kDmaPerStage LDS loads of a stage (k0 .. k0 + 64): parts 0 .. kDmaA-1
// load this wave's A rows, the others its B^T rows, into the stage's slot (A
// first, then B^T).  Each wave instruction fills 1 KiB of LDS, lane l landing at
// byte 16 l: 8 rows x 8 chunks; the lane therefore fetches the logical chunk
// that belongs at its swizzled position.  Rows past the operand's buffer and k
// past K read as 0.
//
// Two ways to address the load, equal in result, chosen per kernel by measurement:
//  * SM (scalar M0): the wave index is read as a scalar, so the LDS destination
//    (M0) is scalar arithmetic, and row x K x 2 splits into a scalar part and
//    lane_rows = (l / kChunks) x K x 2, a per-lane term common to every load of the
//    tile (lane_rows_of), so no multiply is left in the loop; k is 32-bit (the
//    host rejects K with tile rows x K x 2 bytes at 4 GiB or more).  GEMM +
//    ReduceScatter (K = 896): fp32 partials 0.84 -> 0.79 ms, bf16 0.76 -> 0.74 ms;
//  * otherwise the destination comes from the vector wave index through a
//    readfirstlane per load and the offset from 64-bit arithmetic the compiler
//    strength-reduces: AllGather + GEMM (K = 7168) 0.49 against 0.51 ms with SM.
template <int P, bool SM>
__device__ __forceinline__ void stage_load_part(__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                                uint16_t* slot, int64_t K, int64_t k0, uint32_t lane_rows) {
    static_assert(P >= 0 && P < kDmaPerStage, "a stage has kDmaPerStage parts");
    constexpr bool kA = P < kDmaA;
    const int l = (int)threadIdx.x & 63;
    uint32_t off;
    int rbase;
    if constexpr (SM) {
        const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
        rbase = kA ? kRowsA * w + kDmaRows * P : kRowsB * w + kDmaRows * (P - kDmaA);
        const int row = rbase + l / kChunks;
        const int k = (int)k0 + 8 * swz(row, l % kChunks);
        off = k < (int)K ? (uint32_t)rbase * (uint32_t)K * 2u + lane_rows + (uint32_t)k * 2u : kOutOfRange;
    } else {
        const int w = (int)threadIdx.x >> 6;
        rbase = kA ? kRowsA * w + kDmaRows * P : kRowsB * w + kDmaRows * (P - kDmaA);
        const int row = rbase + l / kChunks;
        const int64_t k = k0 + 8 * swz(row, l % kChunks);
        off = k < K ? (uint32_t)(((int64_t)row * K + k) * 2) : kOutOfRange;
    }
    uint16_t* const dst = (kA ? slot : slot + kStageA) + rbase * kStageK;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(kA ? ra : rb, (__attribute__((address_space(3))) void*)dst,
                                             16, off, 0, 0, 0);
}

template <bool SM, int... Ps>
__device__ __forceinline__ void stage_load_seq(__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                               uint16_t* slot, int64_t K, int64_t k0, uint32_t lane_rows,
                                               std::integer_sequence<int, Ps...>) {
    (stage_load_part<Ps, SM>(ra, rb, slot, K, k0, lane_rows), ...);
}

// Every load of one stage into its slot.
template <bool SM>
__device__ __forceinline__ void stage_load(__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                           uint16_t* slot, int64_t K, int64_t k0, uint32_t lane_rows) {
    stage_load_seq<SM>(ra, rb, slot, K, k0, lane_rows, std::make_integer_sequence<int, kDmaPerStage>{});
}

// The per-lane row term of the stage loads' offsets, computed once per tile and
// made opaque so that the compiler cannot fold it back into a multiply per load.
__device__ __forceinline__ uint32_t lane_rows_of(int64_t K) {
    uint32_t v = (uint32_t)(((int)threadIdx.x & 63) / kChunks) * (uint32_t)K * 2u;
    asm volatile("" : "+v"(v));
    return v;
}

// Matrix-core work: wave (wm, wn) owns rows kWaveRows wm .. + kWaveRows and
// columns kWaveCols wn .. + kWaveCols of the tile as kBlkA x kBlkB blocks of
// 32 x 32.  A k16 step reads kBlkA A and kBlkB B fragments (16 bytes per lane)
// and issues kBlkA kBlkB MFMAs (v_mfma_f32_32x32x16_bf16: lane l supplies row /
// column l % 32, k 8 (l / 32) .. +8).
struct Frags {
    bf16x8 a[kBlkA], b[kBlkB];
};

// 16-byte LDS reads at addr + OFF (OFF an immediate).  Written as inline
// assembly on purpose: the compiler cannot tell these reads apart from the LDS
// slots still being filled by the direct loads of later stages, and before
// every LDS read it would wait for all of those loads (vmcnt(0)), which
// serialises the pipeline.  The stage being read is already complete for every
// wave (wait_stages_after + barrier); the caller waits for the reads with
// lds_wait.
template <int OFF>
__device__ __forceinline__ bf16x8 lds_read16(uint32_t addr) {
    bf16x8 v;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
    return v;
}

// Wait until at most N of this wave's LDS reads are outstanding; the fragments
// are tied to the wait so that no use of them is scheduled above it.
template <int KA, int KB> struct FragTie;
template <> struct FragTie<2, 4> {
    template <int N>
    static __device__ __forceinline__ void wait(bf16x8* a, bf16x8* b) {
        asm volatile("s_waitcnt lgkmcnt(%6)"
                     : "+v"(a[0]), "+v"(a[1]), "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3])
                     : "i"(N));
    }
};
template <> struct FragTie<4, 4> {
    template <int N>
    static __device__ __forceinline__ void wait(bf16x8* a, bf16x8* b) {
        asm volatile("s_waitcnt lgkmcnt(%8)"
                     : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(b[0]), "+v"(b[1]),
                       "+v"(b[2]), "+v"(b[3])
                     : "i"(N));
    }
};

template <int N>
__device__ __forceinline__ void lds_wait(Frags& f) {
    FragTie<kBlkA, kBlkB>::template wait<N>(f.a, f.b);
}

// LDS byte address of a stage slot's first element.
__device__ __forceinline__ uint32_t lds_addr(const uint16_t* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint16_t*)p;
}

// Lane byte offsets, inside an operand's stage slot, of the lane's fragment of
// block 0 for k16 step kk (0 .. 3): row row0 + (l mod 32), chunk swz(row, 2 kk + l / 32).
// The swizzle depends only on the row mod 32, so the other blocks (rows + 32 x)
// sit at fixed offsets of 32 x 64 bytes.
__device__ __forceinline__ uint32_t frag_offset(int row0, int kk) {
    const int l = (int)threadIdx.x & 63;
    const int row = row0 + (l & 31);
    return 2u * (uint32_t)(row * kStageK + 8 * swz(row, 2 * kk + (l >> 5)));
}

// Fragment I of read_frags alone (I < kBlkA: A blocks; then the B blocks).
template <int I>
__device__ __forceinline__ void read_frag(Frags& f, uint32_t a_addr, uint32_t b_addr) {
    constexpr int kBlk = 32 * kStageK * 2;  // bytes between fragment blocks
    if constexpr (I < kBlkA)
        f.a[I] = lds_read16<I * kBlk>(a_addr);
    else
        f.b[I - kBlkA] = lds_read16<(I - kBlkA) * kBlk>(b_addr);
}

template <int... Is>
__device__ __forceinline__ void read_frags_seq(Frags& f, uint32_t a_addr, uint32_t b_addr,
                                               std::integer_sequence<int, Is...>) {
    (read_frag<Is>(f, a_addr, b_addr), ...);
}

// Every fragment of one k16 step: kBlkA A blocks, then kBlkB B blocks.
__device__ __forceinline__ void read_frags(Frags& f, uint32_t a_addr, uint32_t b_addr) {
    read_frags_seq(f, a_addr, b_addr, std::make_integer_sequence<int, kBlkA + kBlkB>{});
}

// MFMA I of mma_frags alone (block x = I / kBlkB, y = I mod kBlkB).
template <int I>
__device__ __forceinline__ void mma_one(f32x16 (&acc)[kBlkA][kBlkB], const Frags& f) {
    constexpr int x = I / kBlkB, y = I % kBlkB;
    acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[x], f.b[y], acc[x][y], 0, 0, 0);
}

__device__ __forceinline__ void sb() { __builtin_amdgcn_sched_barrier(0); }

// The interleaving of a k16 step: kMfma MFMAs, and after MFMA i the memory
// operations j (of n in all) with j * kMfma / n == i, so they spread evenly and
// the earliest ones come first.
constexpr int kMfma = kBlkA * kBlkB;
constexpr int kReads = kBlkA + kBlkB;
constexpr int op_slot(int j, int n) { return j * kMfma / n; }

// A k16 step before the barrier: the MFMAs of one fragment set, with the reads of
// the next step's fragments (into the other set) between them.
struct PreCtx {
    Frags* fr;
    uint32_t a, b;
};
template <int I, int J>
__device__ __forceinline__ void pre_op(const PreCtx& c) {
    if constexpr (op_slot(J, kReads) == I) {
        read_frag<J>(*c.fr, c.a, c.b);
        sb();
    }
}
template <int I, int... Js>
__device__ __forceinline__ void pre_ops(const PreCtx& c, std::integer_sequence<int, Js...>) {
    (pre_op<I, Js>(c), ...);
}
template <int... Is>
__device__ __forceinline__ void mma_step(f32x16 (&acc)[kBlkA][kBlkB], const Frags& fm, const PreCtx& c,
                                         std::integer_sequence<int, Is...>) {
    ((mma_one<Is>(acc, fm), sb(), pre_ops<Is>(c, std::make_integer_sequence<int, kReads>{})), ...);
}

// The last k16 step of a stage, after the barrier: its MFMAs, with the reads of
// the next stage's first fragments and then (when `refill`) the loads refilling
// the freed slot between them.
struct PostCtx {
    Frags* fr;
    uint32_t a, b;
    __amdgpu_buffer_rsrc_t ra, rb;
    uint16_t* st;
    int64_t K, k0;
    bool refill;
    uint32_t lane_rows;
};
template <bool SM, int I, int J>
__device__ __forceinline__ void post_op(const PostCtx& c) {
    if constexpr (op_slot(J, kReads + kDmaPerStage) == I) {
        if constexpr (J < kReads) {
            read_frag<J>(*c.fr, c.a, c.b);
        } else {
            if (c.refill) stage_load_part<J - kReads, SM>(c.ra, c.rb, c.st, c.K, c.k0, c.lane_rows);
        }
        sb();
    }
}
template <bool SM, int I, int... Js>
__device__ __forceinline__ void post_ops(const PostCtx& c, std::integer_sequence<int, Js...>) {
    (post_op<SM, I, Js>(c), ...);
}
template <bool SM, int... Is>
__device__ __forceinline__ void mma_step_refill(f32x16 (&acc)[kBlkA][kBlkB], const Frags& fm, const PostCtx& c,
                                                std::integer_sequence<int, Is...>) {
    ((mma_one<Is>(acc, fm), sb(), post_ops<SM, Is>(c, std::make_integer_sequence<int, kReads + kDmaPerStage>{})),
     ...);
}

__device__ __forceinline__ void mma_frags(f32x16 (&acc)[kBlkA][kBlkB], const Frags& f) {
#pragma unroll
    for (int x = 0; x < kBlkA; ++x)
#pragma unroll
        for (int y = 0; y < kBlkB; ++y)
            acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[x], f.b[y], acc[x][y], 0, 0, 0);
}

// One kTileM x kTileN output tile: C[i, n] = sum_k A[i, k] B^T[n, k] for the
// rows_valid rows of A at a_rows and the cols_valid rows of B^T at bt_rows (both
// K-contiguous bf16), stored at c (row stride ldc elements) as bf16 rounded to
// nearest even, or (F32OUT) as the fp32 accumulators themselves; with NTOUT the
// output's 16-byte pieces are stored non-temporally (GEMM+ReduceScatter partials,
// read back only by reduce tasks much later: 3-5 % faster there, measured; the
// AllGather+GEMM output keeps ordinary stores, 1-3 % faster for it).  SM selects the
// stage loads' addressing (stage_load_part).
template <bool F32OUT, bool NTOUT, bool SM>
__device__ __forceinline__ void gemm_tile(const uint16_t* a_rows, int rows_valid,
                                          const uint16_t* bt_rows, int cols_valid, int64_t K,
                                          void* c, int64_t ldc, uint16_t* lds) {
    // K and ldc opaque per tile: nothing derived from them is hoisted out of the
    // persistent task loop and kept alive across tiles.
    asm volatile("" : "+s"(K), "+s"(ldc));
    const __amdgpu_buffer_rsrc_t ra = make_rsrc_uniform(a_rows, (uint32_t)((int64_t)rows_valid * K * 2));
    const __amdgpu_buffer_rsrc_t rb = make_rsrc_uniform(bt_rows, (uint32_t)((int64_t)cols_valid * K * 2));
    f32x16 acc[kBlkA][kBlkB];
#pragma unroll
    for (int x = 0; x < kBlkA; ++x)
#pragma unroll
        for (int y = 0; y < kBlkB; ++y) acc[x][y] = f32x16{};
    const int64_t nk = (K + kStageK - 1) / kStageK;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // only this tile's LDS loads in flight below
    // Stage s lives in slot s mod 2.  Both slots are loaded up front (the second
    // only if its stage exists); stage 0 lands before the first reads.
    const uint32_t lane_rows = SM ? lane_rows_of(K) : 0u;
    stage_load<SM>(ra, rb, lds, K, 0, lane_rows);
    if (nk > 1) {
        stage_load<SM>(ra, rb, lds + kSlotElems, K, kStageK, lane_rows);
        asm volatile("s_waitcnt vmcnt(%0)" ::"i"(kDmaPerStage) : "memory");
    } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __builtin_amdgcn_s_barrier();
    // Software pipeline over stages of four k16 steps, the fragments of step q+1
    // read into the other register set while the MFMAs of step q run:
    //   q0: MFMAs of f0 = (s, 0), reads of f1 = (s, 1)
    //   q1: MFMAs of f1,          reads of f0 = (s, 2)
    //   q2: MFMAs of f0,          reads of f1 = (s, 3)
    //   wait for f1 (every read of stage s is in) and for stage s+1 (the only
    //   LDS loads in flight), barrier
    //   q3: MFMAs of f1,          reads of f0 = (s+1, 0), then the loads
    //       refilling slot s mod 2 with stage s+2
    // so the LDS latency of each step hides under the previous step's MFMAs, and
    // the memory instructions issue while the matrix core works (one MFMA, then one
    // memory instruction: the MFMA runs on while the next instruction issues).  A
    // slot is refilled only after the barrier that follows every wave's wait for
    // its own reads of it; stage s+2 then has q3 of stage s and q0..q2 of stage
    // s+1 to land.  The last iteration reads f0 of a stage past the end (a slot's
    // stale contents, never used): those reads are drained after the loop.  Every
    // branch below is uniform and guards loads only, so the MFMA sequence is the
    // same on every path.
    auto slot = [&](int64_t s) { return lds + (s & 1) * kSlotElems; };
    const int wave = (int)threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    // Step q's fragments sit at step 0's offsets XOR (q << 5): the chunk index
    // 2 q + lane / 32, XORed with g(row), only moves in bits 1-2 with q, which are
    // bits 5-6 of the byte offset (rows are 128 bytes).
    static_assert(kStageK * 2 == 128, "rows of 128 bytes");
    const uint32_t oa = frag_offset(kWaveRows * wm, 0);
    const uint32_t ob = frag_offset(kWaveCols * wn, 0) + 2u * kStageA;
    constexpr auto kSeq = std::make_integer_sequence<int, kMfma>{};
    Frags f0, f1;
    read_frags(f0, lds_addr(slot(0)) + oa, lds_addr(slot(0)) + ob);
    for (int64_t s = 0; s < nk; ++s) {
        const uint32_t cs = lds_addr(slot(s));
        lds_wait<0>(f0);  // the only LDS reads in flight here are f0's
        sb();
        mma_step(acc, f0, PreCtx{&f1, cs + (oa ^ (1u << 5)), cs + (ob ^ (1u << 5))}, kSeq);
        lds_wait<0>(f1);
        sb();
        mma_step(acc, f1, PreCtx{&f0, cs + (oa ^ (2u << 5)), cs + (ob ^ (2u << 5))}, kSeq);
        lds_wait<0>(f0);
        sb();
        mma_step(acc, f0, PreCtx{&f1, cs + (oa ^ (3u << 5)), cs + (ob ^ (3u << 5))}, kSeq);
        lds_wait<0>(f1);  // every read of stage s is in: its slot may be refilled
        if (s + 1 < nk) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // stage s+1 has landed
        __builtin_amdgcn_s_barrier();
        sb();
        const uint32_t ns = lds_addr(slot(s + 1));
        mma_step_refill<SM>(
            acc, f1, PostCtx{&f0, ns + oa, ns + ob, ra, rb, slot(s), K, (s + 2) * kStageK, s + 2 < nk, lane_rows},
            kSeq);
    }
    lds_wait<0>(f0);  // the reads past the last stage land before their registers are reused
    // epilogue: accumulator register e of block (x, y) holds row 8 (e/4) + 4 (lane/32) + e%4,
    // column lane % 32 of the block.  (The empty asm makes the output pointer opaque
    // here, so that the compiler does not hoist the epilogue's addresses above the
    // loop and keep them alive across it.)
    uint64_t cbase = reinterpret_cast<uint64_t>(c);
    asm volatile("" : "+v"(cbase));
    const int lane = (int)threadIdx.x & 63;
    if constexpr (F32OUT) {
        // fp32: through LDS half a tile at a time (rows [128 h, 128 h + 128)), written
        // out as 16-byte row pieces.  Each wave's rows lie in one half; waves of the
        // other half only help with the stores.
        uint8_t* const t = reinterpret_cast<uint8_t*>(lds);
        const bool vec = (cbase & 15u) == 0 && (ldc & 3) == 0;
        constexpr int kPieces = kEpiRows32 * kTileN / 4;  // 4 floats per piece
        const int my_half = kWaveRows * wm / kEpiRows32;
        for (int h = 0; h < kTileM / kEpiRows32; ++h) {
            __builtin_amdgcn_s_barrier();  // the ring, or the previous half, is free
            if (my_half == h) {
#pragma unroll
                for (int x = 0; x < kBlkA; ++x)
#pragma unroll
                    for (int y = 0; y < kBlkB; ++y) {
                        const int col = kWaveCols * wn + 32 * y + (lane & 31);
#pragma unroll
                        for (int e = 0; e < 16; ++e) {
                            const int row = kWaveRows * wm + 32 * x + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                            *reinterpret_cast<float*>(t + (row - kEpiRows32 * h) * kEpiPitch32 + col * 4) =
                                acc[x][y][e];
                        }
                    }
            }
            __syncthreads();
            for (int i = (int)threadIdx.x; i < kPieces; i += kGemmThreads) {
                const int lrow = i / (kTileN / 4);
                const int col0 = (i - lrow * (kTileN / 4)) * 4;
                const int row = kEpiRows32 * h + lrow;
                if (row >= rows_valid || col0 >= cols_valid) continue;
                const u32x4 v = *reinterpret_cast<const u32x4*>(t + lrow * kEpiPitch32 + col0 * 4);
                float* const dst = reinterpret_cast<float*>(cbase) + (int64_t)row * ldc + col0;
                if (vec && col0 + 4 <= cols_valid) {
                    if (NTOUT)
                        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst));
                    else
                        *reinterpret_cast<u32x4*>(dst) = v;
                } else {
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        if (col0 + k < cols_valid) dst[k] = __uint_as_float(v[k]);
                }
            }
        }
    } else {
        // bf16: round into the LDS tile (row pitch kEpiPitch), then write it out as
        // 16-byte row pieces -- 16 stores per lane instead of 128 two-byte ones.
        // Every wave's reads of the ring are complete (its own waits above); the
        // barrier makes that true for all of them before the ring is overwritten.
        __builtin_amdgcn_s_barrier();
        uint8_t* const t = reinterpret_cast<uint8_t*>(lds);
#pragma unroll
        for (int x = 0; x < kBlkA; ++x)
#pragma unroll
            for (int y = 0; y < kBlkB; ++y) {
                const int col = kWaveCols * wn + 32 * y + (lane & 31);
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int row = kWaveRows * wm + 32 * x + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                    *reinterpret_cast<uint16_t*>(t + row * kEpiPitch + col * 2) =
                        (uint16_t)bf16_rne(acc[x][y][e]);
                }
            }
        __syncthreads();
        // 16-byte pieces need a 16-byte aligned output and a row stride of whole pieces
        const bool vec = (cbase & 15u) == 0 && (ldc & 7) == 0;
        constexpr int kPieces = kTileM * kTileN / 8;  // 8 bf16 per piece
        for (int i = (int)threadIdx.x; i < kPieces; i += kGemmThreads) {
            const int row = i / (kTileN / 8);
            const int col0 = (i - row * (kTileN / 8)) * 8;
            if (row >= rows_valid || col0 >= cols_valid) continue;
            const u32x4 v = *reinterpret_cast<const u32x4*>(t + row * kEpiPitch + col0 * 2);
            uint16_t* const dst = reinterpret_cast<uint16_t*>(cbase) + (int64_t)row * ldc + col0;
            if (vec && col0 + 8 <= cols_valid) {
                *reinterpret_cast<u32x4*>(dst) = v;
            } else {
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    if (col0 + k < cols_valid) dst[k] = (uint16_t)(v[k >> 1] >> (16 * (k & 1)));
            }
        }
    }
    __builtin_amdgcn_s_barrier();  // the LDS ring is free for the next tile
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
    __shared__ uint16_t lds[kLdsElems];  // 2 stages x (A, B^T), 128 KiB, or the staged output tile
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
                    copy_flat<16, 8>(src, dst, bytes, threadIdx.x, kGemmThreads);
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
                    gemm_tile<false, false, false>(G + row0 * a.K, rows_valid, a.bt + n0 * a.K, cols_valid, a.K,
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
// like the AllGather's, so the partials a reduce task reads were written into
// the L2 it reads through.

// Reduce task: out_j tile = sum over r = 0..W-1 (in that order) of the partials
// partial_j[r] of the tile (bf16, or with F32P fp32), added in fp32 and rounded
// to bf16 (nearest even).  The partials are read with device-scope loads (never
// from the CU's L1).  V columns per lane: V partial elements form one load.
constexpr int kRsGroup = 8;  // partial loads in flight per lane in a reduce task

template <bool F32P, int V>
__device__ __forceinline__ void rs_reduce_cols(const GemmRsArgs& a, uint8_t* slice, int64_t row0,
                                               int64_t col0, int rows, int cols) {
    constexpr int E = F32P ? 4 : 2;  // bytes per partial element
    // device scope (never the CU's L1) and non-temporal: each partial is read once,
    // and streaming it keeps the L2 for the GEMM tiles' operands (fp32 partials
    // 0.86 -> 0.785 ms at W = 8, m = 8192, K = 896, N = 4096, measured)
    using Load = BufLoad<V * E, kPolicySc1 | kPolicyNt>;
    const __amdgpu_buffer_rsrc_t rp =
        make_rsrc_uniform(slice + a.p_off, (uint32_t)((int64_t)a.W * a.mj * a.N * E));
    uint16_t* const out = reinterpret_cast<uint16_t*>(slice + a.out_off);
    const uint32_t plane = (uint32_t)(a.mj * a.N * E);  // bytes of one source's partial
    const int vc = cols / V;
    for (int i = threadIdx.x; i < rows * vc; i += kGemmThreads) {
        const int r = i / vc;
        const int c = (i - r * vc) * V;
        const int64_t el = (row0 + r) * a.N + col0 + c;
        const uint32_t off = (uint32_t)(el * E);
        float s[V];
#pragma unroll
        for (int v = 0; v < V; ++v) s[v] = 0.f;
        // the sources in groups of kRsGroup: every load of a group is issued before
        // the first add (a short group loads the last source again and skips the
        // add), then the adds run in rank order
        for (int src0 = 0; src0 < a.W; src0 += kRsGroup) {
            decltype(Load::go(rp, 0u)) x[kRsGroup];
#pragma unroll
            for (int g = 0; g < kRsGroup; ++g) {
                const int src = src0 + g < a.W ? src0 + g : a.W - 1;
                x[g] = Load::go(rp, off + (uint32_t)src * plane);
            }
#pragma unroll
            for (int g = 0; g < kRsGroup; ++g) {
                // a select, not a branch: every loaded value is used, so no load is
                // sunk behind a test and the group's loads stay in flight together
                const bool live = src0 + g < a.W;
                if constexpr (V == 1) {
                    const float t = F32P ? __uint_as_float((uint32_t)x[g]) : __uint_as_float((uint32_t)x[g] << 16);
                    s[0] = live ? s[0] + t : s[0];
                } else {
#pragma unroll
                    for (int v = 0; v < V; ++v) {
                        const float t = F32P ? __uint_as_float(x[g][v])
                                             : __uint_as_float(v & 1 ? x[g][v >> 1] & 0xFFFF0000u : x[g][v >> 1] << 16);
                        s[v] = live ? s[v] + t : s[v];
                    }
                }
            }
        }
        if constexpr (V == 1) {
            out[el] = (uint16_t)bf16_rne(s[0]);
        } else {
            // V bf16 results as V/4 8-byte stores (out is 8-byte aligned, V*2 bytes per lane)
#pragma unroll
            for (int q = 0; q < V / 4; ++q) {
                u32x2 o;
                o[0] = bf16_rne(s[4 * q]) | (bf16_rne(s[4 * q + 1]) << 16);
                o[1] = bf16_rne(s[4 * q + 2]) | (bf16_rne(s[4 * q + 3]) << 16);
                *reinterpret_cast<u32x2*>(out + el + 4 * q) = o;
            }
        }
    }
}

template <bool F32P>
__device__ __forceinline__ void rs_reduce_tile(const GemmRsArgs& a, int j, int tile) {
    int mb, nb;
    grs_tile(a, tile, &mb, &nb);
    const int64_t row0 = (int64_t)mb * kRsTileM, col0 = (int64_t)nb * kRsTileN;
    const int rows = a.mj - row0 < kRsTileM ? (int)(a.mj - row0) : kRsTileM;
    const int cols = a.N - col0 < kRsTileN ? (int)(a.N - col0) : kRsTileN;
    uint8_t* const slice = a.base + (int64_t)j * a.stride;
    // 16-byte loads where every row of a tile splits into whole vectors
    constexpr int V = F32P ? 4 : 8;
    if (a.N % V == 0)
        rs_reduce_cols<F32P, V>(a, slice, row0, col0, rows, cols);
    else
        rs_reduce_cols<F32P, 1>(a, slice, row0, col0, rows, cols);
}

template <int SYNC, bool F32P>
__global__ void __launch_bounds__(kGemmThreads, kGemmWgPerCu) gemm_rs_kernel(GemmRsArgs a) {
    __shared__ uint16_t lds[kLdsElems];
    __shared__ int lds_flag;
    __shared__ int64_t lds_pos[2];
    constexpr bool kOwned = SYNC == kSyncXcd;
    uint64_t* const qw = reinterpret_cast<uint64_t*>(a.base + a.sig_off) + grs_queue_slot(a) * kSigStrideU64;
    const uint32_t xcc = xcc_id();
    const int home = SYNC == kSyncXcd ? (int)(xcc % (uint32_t)a.NG) : (int)(blockIdx.x % a.NG);
    const int64_t total = a.ntasks_dest * a.dpg;
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
            // the group's queue: dpg destinations of ntasks_dest each (the last
            // group may have fewer real destinations; their tasks are skipped)
            if (pos >= total) {
                if (threadIdx.x == 0) queue_drained(qw, g, pos, total, qc);
                break;
            }
            uint64_t nxt = 0;
            if (threadIdx.x == 0) nxt = queue_next(qc);
            const RsTask t = grs_group_task(a, g, pos);
            if (t.j < a.W) {
                uint8_t* const dst_slice = a.base + (int64_t)t.j * a.stride;
                uint64_t* const sig = reinterpret_cast<uint64_t*>(dst_slice + a.sig_off);
                if (!t.reduce) {
                    // rank r's partial of the tile: rows j*mj + mb*256 .. of x1_r,
                    // rows nb*256 .. of x2_r^T, into slot r of j's receive area
                    int mb, nb;
                    grs_tile(a, t.tile, &mb, &nb);
                    const int64_t row0 = (int64_t)mb * kRsTileM, col0 = (int64_t)nb * kRsTileN;
                    const int rows = a.mj - row0 < kRsTileM ? (int)(a.mj - row0) : kRsTileM;
                    const int cols = a.N - col0 < kRsTileN ? (int)(a.N - col0) : kRsTileN;
                    const uint8_t* const src_slice = a.base + (int64_t)t.r * a.stride;
                    const uint16_t* x1 = reinterpret_cast<const uint16_t*>(src_slice + a.a_off) +
                                         ((int64_t)t.j * a.mj + row0) * a.K;
                    const uint16_t* x2t = reinterpret_cast<const uint16_t*>(src_slice + a.bt_off) +
                                          col0 * a.K;
                    uint8_t* const part = dst_slice + a.p_off +
                                          (((int64_t)t.r * a.mj + row0) * a.N + col0) * (F32P ? 4 : 2);
                    gemm_tile<F32P, true, true>(x1, rows, x2t, cols, a.K, part, a.N, lds);
                    group_release<SYNC>();
                    if (threadIdx.x == 0)
                        sig_update(sig + grs_sig_slot(a, t.tile, t.r) * kSigStrideU64, 1ull, kSigSet);
                } else {
                    if (!group_wait_all<SYNC == kSyncAgent>(sig + grs_sig_slot(a, t.tile, 0) * kSigStrideU64,
                                                            kSigStrideU64 * 8, a.W, kCmpEq, 1ull,
                                                            a.timeout, a.err, &lds_flag))
                        return;
                    rs_reduce_tile<F32P>(a, t.j, t.tile);
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
