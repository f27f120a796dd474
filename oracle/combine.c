/*
 * CPU oracle for the Reverse All2All (EP-MoE combine) and its inverse, the forward
 * All2All (dispatch) -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg load
 * this file's library.  The GPU path never links, includes or calls it.
 *
 * Definition followed ("Reverse All2All (EP MoE Distributed Kernel)", section
 * "Reverse All2All Operator Semantics", and the MTE listing's producer/consumer
 * index arithmetic in section "Triton-Distributed Reverse All2All Operator"):
 *
 *   W ranks; rank r holds an input of shape (S*W, H, D); rank j receives an
 *   output of shape (S, H*W, D).  Input rows [j*S, (j+1)*S) of rank r belong to
 *   rank j, and rank r's heads land in output columns r*H .. r*H + H - 1:
 *
 *       out_j[s, r*H + h, d] = in_r[j*S + s, h, d]
 *
 *   for r, j in [0, W), s in [0, S), h in [0, H), d in [0, D).
 *
 * The copy is of raw elements (e bytes each), never of interpreted values, so
 * the result is unique and comparable byte for byte for every element type.
 * No blocking, no threading, no reordering: one loop per index of the
 * definition, written out element by element.
 */
#include <stdint.h>
#include <string.h>

#define OUT_INDEX(s, r, h, d) ((((s) * (H * W)) + (r) * H + (h)) * D + (d))
#define IN_INDEX(j, s, h, d) (((((j) * S + (s)) * H) + (h)) * D + (d))

/* out_j for one destination rank j, from the W source inputs in[0..W-1]. */
int oracle_combine_dest(const void *const *in, void *out_j, int64_t j, int64_t W,
                        int64_t S, int64_t H, int64_t D, int64_t e)
{
    if (W < 1 || S < 0 || H < 1 || D < 1 || j < 0 || j >= W) return -1;
    for (int64_t s = 0; s < S; ++s)
        for (int64_t r = 0; r < W; ++r)
            for (int64_t h = 0; h < H; ++h)
                for (int64_t d = 0; d < D; ++d) {
                    const int64_t o = OUT_INDEX(s, r, h, d);
                    const int64_t i = IN_INDEX(j, s, h, d);
                    switch (e) {
                    case 1: ((uint8_t *)out_j)[o] = ((const uint8_t *)in[r])[i]; break;
                    case 2: ((uint16_t *)out_j)[o] = ((const uint16_t *)in[r])[i]; break;
                    case 4: ((uint32_t *)out_j)[o] = ((const uint32_t *)in[r])[i]; break;
                    case 8: ((uint64_t *)out_j)[o] = ((const uint64_t *)in[r])[i]; break;
                    default: return -1;
                    }
                }
    return 0;
}

/* All W outputs. */
int oracle_combine(const void *const *in, void *const *out, int64_t W, int64_t S, int64_t H,
                   int64_t D, int64_t e)
{
    for (int64_t j = 0; j < W; ++j) {
        int rc = oracle_combine_dest(in, out[j], j, W, S, H, D, e);
        if (rc) return rc;
    }
    return 0;
}

/*
 * Forward All2All (dispatch), read as the exact inverse of the combine.  The
 * page's "EP MoE Scenario" sends tokens to the experts' ranks with the
 * dispatch and brings the expert outputs back with the combine, so combine
 * after dispatch returns every token to where it started.  (The page's shape
 * line for the dispatch has the same form as the combine's; its "dimension
 * swap" sentence and the round trip fix the direction.)  Rank j holds an input
 * of shape (S, H*W, D); rank r receives an output of shape (S*W, H, D):
 *
 *       out_r[j*S + s, h, d] = in_j[s, r*H + h, d]
 *
 * for r, j in [0, W), s in [0, S), h in [0, H), d in [0, D).
 */
int oracle_dispatch_dest(const void *const *in, void *out_r, int64_t r, int64_t W,
                         int64_t S, int64_t H, int64_t D, int64_t e)
{
    if (W < 1 || S < 0 || H < 1 || D < 1 || r < 0 || r >= W) return -1;
    for (int64_t j = 0; j < W; ++j)
        for (int64_t s = 0; s < S; ++s)
            for (int64_t h = 0; h < H; ++h)
                for (int64_t d = 0; d < D; ++d) {
                    const int64_t o = ((j * S + s) * H + h) * D + d;   /* out_r[j*S + s, h, d] */
                    const int64_t i = (s * (H * W) + r * H + h) * D + d; /* in_j[s, r*H + h, d] */
                    switch (e) {
                    case 1: ((uint8_t *)out_r)[o] = ((const uint8_t *)in[j])[i]; break;
                    case 2: ((uint16_t *)out_r)[o] = ((const uint16_t *)in[j])[i]; break;
                    case 4: ((uint32_t *)out_r)[o] = ((const uint32_t *)in[j])[i]; break;
                    case 8: ((uint64_t *)out_r)[o] = ((const uint64_t *)in[j])[i]; break;
                    default: return -1;
                    }
                }
    return 0;
}

/*
 * Where one output element comes from: for out_j[s, c, d] returns the source
 * rank r = c div H, the source row j*S + s and the source head c mod H.  Used
 * to check sampled outputs of workloads too large to combine on the host.
 */
void oracle_source_of(int64_t j, int64_t s, int64_t c, int64_t d, int64_t W, int64_t S,
                      int64_t H, int64_t D, int64_t *r, int64_t *row, int64_t *h)
{
    (void)W;
    (void)D;
    (void)d;
    *r = c / H;
    *h = c % H;
    *row = j * S + s;
}

/*
 * AllGather of row shards (HyperParallel RFC, section 十, AllGather and
 * fused_all_gather_matmul): rank w's shard A_w of m_local rows lands at rows
 * [w*m_local, (w+1)*m_local) of the gathered buffer.  row_bytes = K * e.
 */
void oracle_allgather(const void *const *shards, void *gathered, int64_t W, int64_t m_local,
                      int64_t row_bytes)
{
    for (int64_t w = 0; w < W; ++w)
        for (int64_t i = 0; i < m_local; ++i)
            memcpy((uint8_t *)gathered + (w * m_local + i) * row_bytes,
                   (const uint8_t *)shards[w] + i * row_bytes, (size_t)row_bytes);
}
