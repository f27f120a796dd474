// Geometry of the variable-size AllToAll (push): the launch's work queue, the
// chunks of each (source, destination) segment and the signal slots.  Shared by
// the gfx950 kernel and the host-side plan checker.
//
// (HyperParallel RFC, section 十, "AllToAll (Push mode)".)  Rank r holds rows of
// row_bytes bytes, cut in destination order into segments of send_counts_r[j]
// rows; rank j receives the rank-order concatenation of the segments addressed
// to it.  The ranks first exchange metadata (who receives how much, and where
// each sender's rows go), then push the data; a destination's arrival signal
// counts completed senders up to W.
//
// One launch, one work queue (positions claimed in order from an atomic
// counter; every wait points backwards):
//   [0, W)             count task of sender r: put send_counts_r[j] into
//                      recv_counts_j[r] for every j, release, ADD 1 to j's count
//                      signal;
//   [W, 2W)            offset task of destination j: wait for its count signal
//                      to read W, prefix-sum recv_counts_j, and SET each sender
//                      r's offset slot for j to (first row of r's rows in j) + 1;
//   [2W, 2W + NC)      data chunks: sender r's segment for j (destinations in the
//                      rotation j = (r + t) mod W, t = 0 .. W-1) in chunks of
//                      `chunk` bytes (an empty segment is one empty chunk), each
//                      waiting for r's offset slot for j, copying, releasing and
//                      adding 1 to the segment's chunk counter; the segment's last
//                      chunk ADDs 1 to j's arrival signal;
//   [2W + NC, 3W + NC) receive task of destination j: wait for the arrival
//                      signal to read W, then publish the total rows received.
// NC depends on the counts; every workgroup derives the chunk table from them.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define A2V_HD __host__ __device__ __forceinline__
#else
#define A2V_HD inline
#endif

namespace ra2a {

constexpr int kA2vMaxW = 32;  // the chunk table (W*W entries) lives in LDS

struct A2vArgs {
    uint8_t* base;       // heap base (slice 0)
    int64_t stride;      // slice stride, bytes
    int64_t in_off;      // symmetric offset of the input rows (in_r in slice r)
    int64_t cnt_off;     // symmetric offset of send_counts (int64[W] in slice r)
    int64_t out_off;     // symmetric offset of the output rows (out_j in slice j)
    int64_t rc_off;      // symmetric offset of recv_counts (int64[W + 1] in slice j)
    int64_t sig_off;     // symmetric offset of the signals (a2v_* slots)
    uint32_t* err;
    uint64_t timeout;
    int32_t W;
    int64_t row_bytes;   // bytes per row
    int64_t in_rows;     // rows each input holds (the sum of a rank's counts may not exceed it)
    int64_t out_rows;    // rows each output holds (what a rank receives may not exceed it)
    int64_t chunk;       // bytes per data chunk (a multiple of 16)
};

// Signal slots (128 bytes apart, word 0 used), per slice:
//   0            count signal (slice j): senders whose counts arrived (ends at W)
//   1 + j        offset slot for destination j (slice r): 0, then recv offset + 1
//   1 + W + r    chunk counter of source r's segment (slice j)
//   1 + 2W       arrival signal (slice j): senders whose segment is complete (ends at W)
//   2 + 2W       (slice 0 only) the queue's claim counter
A2V_HD int64_t a2v_count_slot() { return 0; }
A2V_HD int64_t a2v_offset_slot(int j) { return 1 + j; }
A2V_HD int64_t a2v_chunk_slot(int W, int r) { return 1 + W + r; }
A2V_HD int64_t a2v_arrival_slot(int W) { return 1 + 2 * (int64_t)W; }
A2V_HD int64_t a2v_queue_slot(int W) { return 2 + 2 * (int64_t)W; }
A2V_HD int64_t a2v_slots(int W) { return 3 + 2 * (int64_t)W; }

// Chunks of a segment of `rows` rows (at least one, so an empty segment still signals).
A2V_HD int64_t a2v_chunks(int64_t rows, int64_t row_bytes, int64_t chunk) {
    const int64_t bytes = rows > 0 ? rows * row_bytes : 0;
    return bytes > 0 ? (bytes + chunk - 1) / chunk : 1;
}

// Pair index of (sender r, step t): sender-major, t the rotation step.
A2V_HD int a2v_pair(int W, int r, int t) { return r * W + t; }
A2V_HD int a2v_dest(int W, int r, int t) { return (r + t) % W; }

struct A2vTask {
    int kind;      // 0 count, 1 offset, 2 chunk, 3 receive, -1 past the end
    int r, j;      // sender / destination (as the kind uses them)
    int64_t c;     // chunk index within its segment
};

// Task at queue position pos, given the exclusive prefix `first` of chunks over
// the W*W pairs (first[W*W] = NC).  Binary search over the pairs.
A2V_HD A2vTask a2v_task(int W, const int64_t* first, int64_t pos) {
    A2vTask t{-1, 0, 0, 0};
    const int64_t NC = first[W * W];
    if (pos < W) {
        t.kind = 0;
        t.r = (int)pos;
    } else if (pos < 2 * (int64_t)W) {
        t.kind = 1;
        t.j = (int)(pos - W);
    } else if (pos < 2 * (int64_t)W + NC) {
        const int64_t q = pos - 2 * (int64_t)W;
        int lo = 0, hi = W * W - 1;  // the last pair with first[p] <= q
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (first[mid] <= q)
                lo = mid;
            else
                hi = mid - 1;
        }
        t.kind = 2;
        t.r = lo / W;
        t.j = a2v_dest(W, t.r, lo - t.r * W);
        t.c = q - first[lo];
    } else if (pos < 3 * (int64_t)W + NC) {
        t.kind = 3;
        t.j = (int)(pos - 2 * (int64_t)W - NC);
    }
    return t;
}

A2V_HD int64_t a2v_total(int W, const int64_t* first) { return 3 * (int64_t)W + first[W * W]; }

// A sender whose counts are unusable (a negative count, or more rows in total
// than its input holds) sends nothing: all its counts read as 0.
A2V_HD bool a2v_rank_ok(int W, int64_t in_rows, const int64_t* row) {
    int64_t sum = 0;
    for (int j = 0; j < W; ++j) {
        const int64_t c = row[j];
        if (c < 0 || c > in_rows - sum) return false;
        sum += c;
    }
    return true;
}

// cnt[r*W + j] holds the raw counts; on return the usable ones.  The result
// says whether every sender's counts were usable.
A2V_HD bool a2v_sanitize(int W, int64_t in_rows, int64_t* cnt) {
    bool all_ok = true;
    for (int r = 0; r < W; ++r) {
        if (!a2v_rank_ok(W, in_rows, cnt + r * W)) {
            all_ok = false;
            for (int j = 0; j < W; ++j) cnt[r * W + j] = 0;
        }
    }
    return all_ok;
}

// First input row of sender r's segment for j (exclusive prefix over j).
A2V_HD int64_t a2v_send_offset(int W, const int64_t* cnt, int r, int j) {
    int64_t o = 0;
    for (int k = 0; k < j; ++k) o += cnt[r * W + k];
    return o;
}

// Byte range [lo, hi) of chunk c of a segment of `rows` rows.
A2V_HD void a2v_chunk_range(int64_t rows, int64_t row_bytes, int64_t chunk, int64_t c, int64_t* lo,
                            int64_t* hi) {
    const int64_t bytes = rows * row_bytes;
    *lo = c * chunk < bytes ? c * chunk : bytes;
    *hi = *lo + chunk < bytes ? *lo + chunk : bytes;
}

}  // namespace ra2a
