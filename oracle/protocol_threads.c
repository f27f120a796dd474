/* Threaded executor of the tile-signalled combine protocol -- TEST
 * INFRASTRUCTURE ONLY.  Only the test suite builds and runs it; the GPU path
 * never links or calls it.
 *
 * It runs the producer/consumer protocol with real host threads on C11 atomics,
 * so that ThreadSanitizer can watch the ordering it relies on:
 *
 *   producer (one thread per source r), for every S-block tile t and, within
 *   it, every destination j in the rotation j = (r + k) mod W (tile-major, the
 *   pages' task order; destination-major order deadlocks on a ring, since a
 *   producer would wait for credits that need other producers' later pieces):
 *     1. (ring of R slots) wait until slot t mod R of j has been handed back
 *        for its previous use: credit count >= t div R, acquire;
 *     2. write its piece, rows [t*B, (t+1)*B) of in_r addressed to j, into
 *        j's staging slot at column block r;
 *     3. publish with release order and signal j's tile: ADD 1 (push mode, the
 *        consumer waits for W) or SET 1 on the piece's own slot;
 *   consumer (one thread per destination j), for every tile t:
 *     1. wait until the tile's signal(s) reach the expected value, acquire
 *        (bounded: a wait that never ends is reported as a timeout);
 *     2. copy the staging slot into out_j rows [t*B, (t+1)*B), source-major;
 *     3. (ring) hand the slot back: credit count + 1, release.
 *
 * (The Reverse All2All page, "Reverse All2All (EP MoE Distributed Kernel)":
 * "MTE Implementation > Signal-Based Synchronization" and "Wait/Notify
 * Optimization > Dual Signal Memory Region Design"; the HyperParallel RFC,
 * section 5.1 "Push mode" and section six, put_with_signal.)  Credits are
 * counts of completed consumptions and tile signals are unique per tile, the
 * readings the protocol model takes.
 *
 * Result: out_j[s, r, x] = in_r[j*S + s, x] (the combine's definition, with the
 * H*D elements of a row as x), final signals W (ADD) or 1 (SET) everywhere, and
 * credits equal to each slot's number of uses.
 *
 * Negative controls (each must be caught, by ThreadSanitizer or by the checks):
 *   --signal-first   the producer signals (relaxed) before writing its piece;
 *   --no-reset       the signals start at their final values, as after a
 *                    launch whose signals were not zeroed;
 *   --drop-piece     source 0 never sends tile 0 to destination 0: the
 *                    consumer's wait times out.
 *
 * Usage: protocol_threads W S B X R add|set seed [control]
 *   B rows per tile, X elements per row, R ring slots (0: one slot per tile).
 * Exit status: 0 all checks pass, 1 a check failed, 2 a wait timed out,
 * 3 bad arguments.
 */
#define _POSIX_C_SOURCE 200809L
#include <pthread.h>
#include <sched.h>
#include <stdatomic.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>

static int W, S, B, X, R, T, use_add, control;
enum { CTRL_NONE, CTRL_SIGNAL_FIRST, CTRL_NO_RESET, CTRL_DROP_PIECE };
static uint64_t seed;
static uint32_t **in, **out, **stage;   /* in_r[W*S][X]; out_j[S][W][X]; stage_j[slots][B][W][X] */
static atomic_uint_least64_t **sig;     /* ADD: [j][t]; SET: [j][t*W + r] */
static atomic_uint_least64_t **credit;  /* [j][slot], ring only */
static atomic_int timed_out;
static double wait_limit_s = 5.0;  /* bounded waits: a wait this long is a timeout
                                      (PROTOCOL_WAIT_S overrides) */

static uint32_t in_value(int r, int row, int x) {
    return (uint32_t)r * 2654435761u ^ (uint32_t)row * 40503u ^ (uint32_t)x * 97u ^ 0x5bd1e995u;
}

/* per-thread xorshift64 for seeded delays */
static uint64_t next(uint64_t *s) {
    *s ^= *s << 13;
    *s ^= *s >> 7;
    *s ^= *s << 17;
    return *s;
}
static void delay(uint64_t *s) {
    const uint64_t d = next(s) % 64;
    if (d < 8) sched_yield();
    for (volatile uint64_t i = 0; i < d * 16; ++i) {
    }
}

static int slots(void) { return R > 0 ? R : T; }
static uint32_t *stage_at(int j, int slot, int b, int r) {
    return stage[j] + (((size_t)slot * B + b) * W + r) * X;
}

static double now_s(void) {
    struct timespec ts;
    clock_gettime(CLOCK_MONOTONIC, &ts);
    return (double)ts.tv_sec + 1e-9 * (double)ts.tv_nsec;
}

static int wait_at_least(atomic_uint_least64_t *p, uint64_t v) {
    const double t0 = now_s();
    for (long i = 0;; ++i) {
        if (atomic_load_explicit(p, memory_order_acquire) >= v) return 1;
        if (atomic_load_explicit(&timed_out, memory_order_relaxed)) return 0;
        if ((i & 255) == 255) {
            sched_yield();
            if (now_s() - t0 > wait_limit_s) {
                atomic_store(&timed_out, 1);
                return 0;
            }
        }
    }
}

static void *producer(void *arg) {
    const int r = (int)(intptr_t)arg;
    uint64_t rs = seed * 0x9E3779B97F4A7C15ull + (uint64_t)r * 0xD1B54A32D192ED03ull + 1;
    for (int t = 0; t < T; ++t) {
        for (int k = 0; k < W; ++k) {
            const int j = (r + k) % W;
            if (control == CTRL_DROP_PIECE && r == 0 && j == 0 && t == 0) continue;
            const int slot = R > 0 ? t % R : t;
            if (R > 0 && !wait_at_least(&credit[j][slot], (uint64_t)(t / R))) return NULL;
            delay(&rs);
            atomic_uint_least64_t *sp = use_add ? &sig[j][t] : &sig[j][(size_t)t * W + r];
            if (control == CTRL_SIGNAL_FIRST) {
                if (use_add)
                    atomic_fetch_add_explicit(sp, 1, memory_order_relaxed);
                else
                    atomic_store_explicit(sp, 1, memory_order_relaxed);
            }
            for (int b = 0; b < B; ++b) {
                const int row = j * S + t * B + b;
                memcpy(stage_at(j, slot, b, r), in[r] + (size_t)row * X, sizeof(uint32_t) * X);
            }
            delay(&rs);
            if (control != CTRL_SIGNAL_FIRST) {
                if (use_add)
                    atomic_fetch_add_explicit(sp, 1, memory_order_release);
                else
                    atomic_store_explicit(sp, 1, memory_order_release);
            }
        }
    }
    return NULL;
}

static void *consumer(void *arg) {
    const int j = (int)(intptr_t)arg;
    uint64_t rs = seed * 0xBF58476D1CE4E5B9ull + (uint64_t)j * 0x94D049BB133111EBull + 7;
    for (int t = 0; t < T; ++t) {
        const int slot = R > 0 ? t % R : t;
        if (use_add) {
            if (!wait_at_least(&sig[j][t], (uint64_t)W)) return NULL;
        } else {
            for (int r = 0; r < W; ++r)
                if (!wait_at_least(&sig[j][(size_t)t * W + r], 1)) return NULL;
        }
        delay(&rs);
        for (int b = 0; b < B; ++b)
            for (int r = 0; r < W; ++r)
                memcpy(out[j] + (((size_t)(t * B + b) * W + r) * X), stage_at(j, slot, b, r), sizeof(uint32_t) * X);
        if (R > 0) atomic_fetch_add_explicit(&credit[j][slot], 1, memory_order_release);
    }
    return NULL;
}

int main(int argc, char **argv) {
    if (argc < 8) {
        fprintf(stderr, "usage: %s W S B X R add|set seed [--signal-first|--no-reset|--drop-piece]\n", argv[0]);
        return 3;
    }
    W = atoi(argv[1]);
    S = atoi(argv[2]);
    B = atoi(argv[3]);
    X = atoi(argv[4]);
    R = atoi(argv[5]);
    use_add = strcmp(argv[6], "add") == 0;
    seed = strtoull(argv[7], NULL, 10);
    control = CTRL_NONE;
    if (argc > 8) {
        if (!strcmp(argv[8], "--signal-first")) control = CTRL_SIGNAL_FIRST;
        else if (!strcmp(argv[8], "--no-reset")) control = CTRL_NO_RESET;
        else if (!strcmp(argv[8], "--drop-piece")) control = CTRL_DROP_PIECE;
        else return 3;
    }
    if (W < 1 || W > 64 || S < 1 || B < 1 || S % B || X < 1 || R < 0 || (strcmp(argv[6], "add") && strcmp(argv[6], "set")))
        return 3;
    T = S / B;
    if (getenv("PROTOCOL_WAIT_S")) wait_limit_s = atof(getenv("PROTOCOL_WAIT_S"));
    const int nsig = use_add ? T : T * W;
    in = calloc(W, sizeof *in);
    out = calloc(W, sizeof *out);
    stage = calloc(W, sizeof *stage);
    sig = calloc(W, sizeof *sig);
    credit = calloc(W, sizeof *credit);
    for (int r = 0; r < W; ++r) {
        in[r] = malloc(sizeof(uint32_t) * (size_t)W * S * X);
        for (int row = 0; row < W * S; ++row)
            for (int x = 0; x < X; ++x) in[r][(size_t)row * X + x] = in_value(r, row, x);
        out[r] = calloc((size_t)S * W * X, sizeof(uint32_t));
        stage[r] = calloc((size_t)slots() * B * W * X, sizeof(uint32_t));
        sig[r] = malloc(sizeof(atomic_uint_least64_t) * nsig);
        for (int i = 0; i < nsig; ++i)
            atomic_init(&sig[r][i], control == CTRL_NO_RESET ? (use_add ? (uint64_t)W : 1u) : 0u);
        credit[r] = malloc(sizeof(atomic_uint_least64_t) * (R > 0 ? R : 1));
        for (int i = 0; i < (R > 0 ? R : 1); ++i) atomic_init(&credit[r][i], 0);
    }
    atomic_init(&timed_out, 0);
    pthread_t *th = malloc(sizeof(pthread_t) * 2 * W);
    for (int i = 0; i < W; ++i) {
        pthread_create(&th[i], NULL, consumer, (void *)(intptr_t)i);
        pthread_create(&th[W + i], NULL, producer, (void *)(intptr_t)i);
    }
    for (int i = 0; i < 2 * W; ++i) pthread_join(th[i], NULL);
    if (atomic_load(&timed_out)) {
        printf("timeout\n");
        return 2;
    }
    long bad = 0;
    for (int j = 0; j < W; ++j) {
        for (int s = 0; s < S; ++s)
            for (int r = 0; r < W; ++r)
                for (int x = 0; x < X; ++x)
                    bad += out[j][((size_t)s * W + r) * X + x] != in_value(r, j * S + s, x);
        for (int i = 0; i < nsig; ++i) bad += atomic_load(&sig[j][i]) != (use_add ? (uint64_t)W : 1u);
        if (R > 0)
            for (int i = 0; i < R; ++i) bad += atomic_load(&credit[j][i]) != (uint64_t)((T - i + R - 1) / R);
    }
    printf(bad ? "mismatch %ld\n" : "ok\n", bad);
    return bad ? 1 : 0;
}
