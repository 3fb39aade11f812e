/*
 * Driver that runs the C oracle (oracle/kda_oracle.c) under AddressSanitizer
 * and UndefinedBehaviorSanitizer (built by tests/test_oracle_sanitize.py with
 * gcc; CPU only).  Every buffer is allocated at its exact size, so any read or
 * write past an end is reported.  The cases cover the oracle's index
 * arithmetic: packed documents including empty and one-token ones, unequal
 * head sizes, chunk snapshots with ragged tails, every prologue flag, null
 * optional pointers, an empty call, rejected arguments, and two threads.
 * A known trajectory (the scalar hand case: S = 1, 0.25, -3) checks that the
 * instrumented build still computes the recurrence.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int kda_oracle_prefill(int64_t num_seqs, const int64_t *cu_seqlens, int64_t T, int64_t H,
                       int64_t dk, int64_t dv, const float *q, const float *k, const float *v,
                       const float *beta, const float *log_alpha, const double *initial_state,
                       double *final_state, double *o, int64_t chunk, double *chunk_states,
                       int nthreads, int flags);

static int failures = 0;
#define CHECK(c, msg)                                  \
    do {                                               \
        if (!(c)) {                                    \
            fprintf(stderr, "FAIL: %s\n", msg);        \
            ++failures;                                \
        }                                              \
    } while (0)

static float *fbuf(int64_t n, unsigned *seed, float lo, float hi)
{
    float *p = (float *)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
    for (int64_t i = 0; i < n; ++i) {
        *seed = *seed * 1664525u + 1013904223u;
        p[i] = lo + (hi - lo) * (float)(*seed >> 8) / (float)(1u << 24);
    }
    return p;
}

static void scalar_hand_case(void)
{
    /* (alpha, beta, k, v, q) per step from S0 = 0: (1/2, 1/2, 1, 2, 1),
     * (1/2, 1/2, 1, 0, 1), (1, 1, -1, 3, 1) -> S = 1, 0.25, -3 = o. */
    const int64_t cu[2] = {0, 3};
    float q[3] = {1, 1, 1}, k[3] = {1, 1, -1}, v[3] = {2, 0, 3}, b[3] = {0.5f, 0.5f, 1.0f};
    float la[3] = {(float)log(0.5), (float)log(0.5), 0.0f};
    double *o = (double *)malloc(sizeof(double) * 3), *fin = (double *)malloc(sizeof(double));
    int rc = kda_oracle_prefill(1, cu, 3, 1, 1, 1, q, k, v, b, la, NULL, fin, o, 0, NULL, 1, 0);
    CHECK(rc == 0, "scalar case rc");
    const double want[3] = {1.0, 0.25, -3.0};
    for (int t = 0; t < 3; ++t) CHECK(fabs(o[t] - want[t]) < 1e-6, "scalar case trajectory");
    CHECK(fabs(fin[0] + 3.0) < 1e-6, "scalar case final state");
    free(o);
    free(fin);
}

static void packed_case(int flags, int64_t chunk)
{
    const int64_t N = 5, H = 3, dk = 4, dv = 6;
    const int64_t lens[5] = {5, 0, 17, 1, 9};
    int64_t cu[6] = {0};
    for (int n = 0; n < N; ++n) cu[n + 1] = cu[n] + lens[n];
    const int64_t T = cu[N];
    unsigned seed = 12345u + (unsigned)flags * 7u + (unsigned)chunk;
    float *q = fbuf(T * H * dk, &seed, -1, 1), *k = fbuf(T * H * dk, &seed, -1, 1);
    float *v = fbuf(T * H * dv, &seed, -1, 1), *b = fbuf(T * H, &seed, 0, 1);
    float *la = fbuf(T * H * dk, &seed, -3, 0);
    double *init = (double *)malloc(sizeof(double) * (size_t)(N * H * dk * dv));
    for (int64_t i = 0; i < N * H * dk * dv; ++i) init[i] = 0.01 * (double)(i % 17) - 0.08;
    double *fin = (double *)malloc(sizeof(double) * (size_t)(N * H * dk * dv));
    double *o = (double *)malloc(sizeof(double) * (size_t)(T * H * dv));
    int64_t nch = 0;
    for (int n = 0; n < N; ++n) nch += (lens[n] + chunk - 1) / chunk;
    double *cs = (double *)malloc(sizeof(double) * (size_t)(nch * H * dk * dv));
    int rc = kda_oracle_prefill(N, cu, T, H, dk, dv, q, k, v, b, la, init, fin, o, chunk, cs, 2, flags);
    CHECK(rc == 0, "packed case rc");
    for (int64_t i = 0; i < T * H * dv; ++i) CHECK(isfinite(o[i]), "packed case output finite");
    /* the empty document keeps its initial state; each document's first
     * chunk snapshot is its initial state */
    for (int64_t i = 0; i < H * dk * dv; ++i) CHECK(fin[1 * H * dk * dv + i] == init[1 * H * dk * dv + i],
                                                   "empty document keeps its state");
    int64_t c0 = 0;
    for (int n = 0; n < N; ++n) {
        if (lens[n] > 0)
            for (int64_t i = 0; i < H * dk * dv; ++i)
                CHECK(cs[c0 * H * dk * dv + i] == init[n * H * dk * dv + i], "first snapshot = initial state");
        c0 += (lens[n] + chunk - 1) / chunk;
    }
    /* null optional outputs and no initial state */
    rc = kda_oracle_prefill(N, cu, T, H, dk, dv, q, k, v, b, la, NULL, NULL, o, 0, NULL, 1, flags);
    CHECK(rc == 0, "null optional pointers rc");
    free(q); free(k); free(v); free(b); free(la); free(init); free(fin); free(o); free(cs);
}

static void edge_cases(void)
{
    double o1[1];
    const int64_t cu_empty[3] = {0, 0, 0};
    /* two empty documents: nothing to read, final state = initial */
    double init[2 * 2 * 2] = {1, 2, 3, 4, 5, 6, 7, 8}, fin[8];
    float dummy[1] = {0};
    int rc = kda_oracle_prefill(2, cu_empty, 0, 1, 2, 2, dummy, dummy, dummy, dummy, dummy, init, fin, o1,
                                4, NULL, 1, 0);
    CHECK(rc == 0 && memcmp(init, fin, sizeof(fin)) == 0, "empty call keeps the state");
    const int64_t cu_bad[3] = {0, 3, 2};
    rc = kda_oracle_prefill(2, cu_bad, 2, 1, 2, 2, dummy, dummy, dummy, dummy, dummy, NULL, NULL, o1, 0, NULL,
                            1, 0);
    CHECK(rc == -1, "decreasing offsets are rejected");
    rc = kda_oracle_prefill(1, cu_empty, 0, 1, 2, 2, dummy, dummy, dummy, dummy, dummy, NULL, NULL, o1, 0, NULL,
                            1, 8);
    CHECK(rc == -1, "unknown prologue bit is rejected");
}

int main(void)
{
    scalar_hand_case();
    for (int flags = 0; flags < 8; ++flags) packed_case(flags, 4);
    packed_case(0, 1);
    packed_case(7, 16);
    edge_cases();
    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    printf("ORACLE_SANITIZE_PASS\n");
    return 0;
}
