/*
 * CPU oracle for the KDA gated delta-rule recurrence — plain C, fp64.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library; the product path never
 * does.  It shares no code, header or helper with the HIP path.
 *
 * Per sequence n and head h, with S a d_k x d_v matrix held in fp64:
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t
 *
 * The closed form and the order (I - beta k k^T) D (not D (I - beta k k^T))
 * follow "GLM-5.3-Flash Architecture Mastery" (course index, Course Outcomes
 * and Exit Criteria) and Module 11 — Correctness as Architecture Mastery,
 * §2 "The full correctness matrix", KDA row.  It is evaluated token by token
 * as five operations (the pages name five but do not print them; this is the
 * plainest expansion that multiplies out to the closed form):
 *
 *     decay    S'  = Diag(exp(log_alpha_t)) S_{t-1}
 *     predict  p   = S'^T k_t
 *     error    e   = v_t - p
 *     write    S_t = S' + beta_t k_t e^T
 *     read     o_t = S_t^T q_t
 *
 * Packed documents (cu_seqlens) never share state (Module 11, §2, row
 * "Padding / packing"); the state entering every chunk of a document can be
 * recorded for the chunk-boundary comparisons of Module 04 — KDA II, §4
 * "The correctness invariant".  The recording is a copy of the token-by-token
 * state; no chunked arithmetic happens here.
 *
 * Optional prologue (flags): the stages just before the recurrence in the
 * executed sublayer — Q/K normalisation, the decay gate producing alpha and
 * the write gate producing beta (Module 04 — KDA II, §3 "The sublayer is
 * bigger than the recurrence").  The pages give no formulas; the forms are
 * those the workload descriptions use for their inputs:
 *     flag 1  log_alpha holds x:  log alpha = -softplus(x) = -log(1 + e^x)
 *     flag 2  beta holds x:       beta = 1 / (1 + e^-x)
 *     flag 4  q, k -> x / sqrt(sum x^2 + 1e-6) over d_k, per (token, head)
 *
 * Inputs are fp32 arrays holding the values as given (bf16 inputs are
 * widened exactly by the caller).  Layouts (packed along T):
 *     q, k, log_alpha [T, H, dk]   v [T, H, dv]   beta [T, H]
 *     states          [N, H, dk, dv]              o [T, H, dv]
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define PRO_GATE_SOFTPLUS 1
#define PRO_BETA_SIGMOID 2
#define PRO_QK_L2NORM 4
#define QK_NORM_EPS 1e-6

/* log(1 + e^x) without overflow */
static double softplus(double x) { return (x > 0 ? x : 0.0) + log1p(exp(-fabs(x))); }

/* 1 / (1 + e^-x) without overflow */
static double sigmoid(double x)
{
    const double e = exp(-fabs(x));
    return x >= 0 ? 1.0 / (1.0 + e) : e / (1.0 + e);
}

/* dst = src / sqrt(sum src^2 + eps), or a plain widening copy */
static void load_vec(const float *src, double *dst, int64_t n, int normalise)
{
    double ss = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        dst[i] = (double)src[i];
        ss += dst[i] * dst[i];
    }
    if (normalise) {
        const double inv = 1.0 / sqrt(ss + QK_NORM_EPS);
        for (int64_t i = 0; i < n; ++i) dst[i] *= inv;
    }
}

/* One (sequence, head) pair, tokens [t0, t1).  S (dk*dv) holds the incoming
 * state and receives the outgoing one.  snaps (nullable): state entering
 * tokens t0, t0+chunk, ... written consecutively, each dk*dv, with stride
 * snap_stride between consecutive chunks.  scratch: 2 dv + 2 dk doubles. */
static void run_pair(int64_t t0, int64_t t1, int64_t h, int64_t H, int64_t dk, int64_t dv,
                     const float *q, const float *k, const float *v, const float *beta,
                     const float *log_alpha, double *S, double *o, int64_t chunk,
                     double *snaps, int64_t snap_stride, double *scratch, int flags)
{
    double *p = scratch;             /* [dv] */
    double *e = scratch + dv;        /* [dv] */
    double *qv = scratch + 2 * dv;   /* [dk] q_t after the prologue */
    double *kv = qv + dk;            /* [dk] k_t after the prologue */
    const int norm = (flags & PRO_QK_L2NORM) != 0;
    for (int64_t t = t0; t < t1; ++t) {
        if (snaps && chunk > 0 && (t - t0) % chunk == 0) {
            memcpy(snaps + ((t - t0) / chunk) * snap_stride, S, sizeof(double) * dk * dv);
        }
        const float *gt = log_alpha + (t * H + h) * dk;
        const float *vt = v + (t * H + h) * dv;
        load_vec(q + (t * H + h) * dk, qv, dk, norm);
        load_vec(k + (t * H + h) * dk, kv, dk, norm);
        double bt = (double)beta[t * H + h];
        if (flags & PRO_BETA_SIGMOID) bt = sigmoid(bt);

        /* decay: row i of S scaled by alpha_i */
        for (int64_t i = 0; i < dk; ++i) {
            const double g = (flags & PRO_GATE_SOFTPLUS) ? -softplus((double)gt[i]) : (double)gt[i];
            const double a = exp(g);
            for (int64_t j = 0; j < dv; ++j) S[i * dv + j] *= a;
        }
        /* predict: p = S'^T k */
        for (int64_t j = 0; j < dv; ++j) p[j] = 0.0;
        for (int64_t i = 0; i < dk; ++i) {
            const double ki = kv[i];
            for (int64_t j = 0; j < dv; ++j) p[j] += S[i * dv + j] * ki;
        }
        /* error: e = v - p */
        for (int64_t j = 0; j < dv; ++j) e[j] = (double)vt[j] - p[j];
        /* write: S += beta k e^T */
        for (int64_t i = 0; i < dk; ++i) {
            const double bk = bt * kv[i];
            for (int64_t j = 0; j < dv; ++j) S[i * dv + j] += bk * e[j];
        }
        /* read: o = S^T q */
        double *ot = o + (t * H + h) * dv;
        for (int64_t j = 0; j < dv; ++j) ot[j] = 0.0;
        for (int64_t i = 0; i < dk; ++i) {
            const double qi = qv[i];
            for (int64_t j = 0; j < dv; ++j) ot[j] += S[i * dv + j] * qi;
        }
    }
}

/*
 * Run the recurrence over num_seqs packed sequences.
 *   cu_seqlens    [num_seqs+1] token offsets (cu[0] = 0, non-decreasing, cu[N] = T)
 *   initial_state nullable => zeros; [N, H, dk, dv] fp64
 *   final_state   nullable;          [N, H, dk, dv] fp64
 *   o             [T, H, dv] fp64
 *   chunk, chunk_states: if chunk > 0 and chunk_states != NULL, the state
 *       entering each chunk of each document, documents in order, layout
 *       [sum_n ceil(len_n / chunk), H, dk, dv].
 *   nthreads      <= 0 => OpenMP default.
 *   flags         prologue bits (see the top of this file), 0 = none.
 * Returns 0, or -1 on invalid arguments, -2 on allocation failure.
 */
int kda_oracle_prefill(int64_t num_seqs, const int64_t *cu_seqlens, int64_t T, int64_t H,
                       int64_t dk, int64_t dv, const float *q, const float *k, const float *v,
                       const float *beta, const float *log_alpha, const double *initial_state,
                       double *final_state, double *o, int64_t chunk, double *chunk_states,
                       int nthreads, int flags)
{
    if (num_seqs < 0 || !cu_seqlens || H <= 0 || dk <= 0 || dv <= 0 || !o) return -1;
    if (flags & ~(PRO_GATE_SOFTPLUS | PRO_BETA_SIGMOID | PRO_QK_L2NORM)) return -1;
    if (cu_seqlens[0] != 0 || cu_seqlens[num_seqs] != T) return -1;
    for (int64_t n = 0; n < num_seqs; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;

    /* first chunk index of each document in chunk_states */
    int64_t *chunk_off = (int64_t *)malloc(sizeof(int64_t) * (size_t)(num_seqs + 1));
    if (!chunk_off) return -2;
    chunk_off[0] = 0;
    for (int64_t n = 0; n < num_seqs; ++n) {
        const int64_t len = cu_seqlens[n + 1] - cu_seqlens[n];
        chunk_off[n + 1] = chunk_off[n] + (chunk > 0 ? (len + chunk - 1) / chunk : 0);
    }
    const int64_t pairs = num_seqs * H;
    const int64_t sz = dk * dv;
    int err = 0;
#ifdef _OPENMP
    /* the thread count applies to this call only (no global side effect) */
    const int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel num_threads(nt)
#endif
    {
        double *S = (double *)malloc(sizeof(double) * (size_t)(sz + 2 * dv + 2 * dk));
        if (!S) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            err = -2;
        }
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t pr = 0; pr < pairs; ++pr) {
            if (!S) continue;
            const int64_t n = pr / H, h = pr % H;
            if (initial_state)
                memcpy(S, initial_state + pr * sz, sizeof(double) * sz);
            else
                memset(S, 0, sizeof(double) * sz);
            double *snaps = NULL;
            if (chunk > 0 && chunk_states) snaps = chunk_states + (chunk_off[n] * H + h) * sz;
            run_pair(cu_seqlens[n], cu_seqlens[n + 1], h, H, dk, dv, q, k, v, beta, log_alpha,
                     S, o, chunk, snaps, H * sz, S + sz, flags);
            if (final_state) memcpy(final_state + pr * sz, S, sizeof(double) * sz);
        }
        free(S);
    }
    free(chunk_off);
    return err;
}

int kda_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
