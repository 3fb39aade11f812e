/*
 * kda.h — C ABI of libkda: the KDA gated delta-rule recurrence on AMD
 * Instinct MI355X (gfx950).
 *
 * The operation (per sequence n and head h; S is d_k x d_v, fp32):
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t ,          alpha_t = exp(log_alpha_t) in (0, 1]^{d_k}
 *
 * Closed form and operator order: "GLM-5.3-Flash Architecture Mastery",
 * course index, Course Outcomes; Module 11 — Correctness as Architecture
 * Mastery, §2 "The full correctness matrix", KDA row.  Two entry points, one
 * per request phase (Module 04 — KDA II: Chunked Parallelism & the Full
 * Sublayer, §2 "Why decode and prefill need different kernels"):
 *
 *   kda_prefill_chunked  many tokens per sequence; chunk-parallel: every
 *                        chunk's composed transition is built independently
 *                        in structured (diagonal + low-rank) form, then the
 *                        chunks are applied in order (Module 04, §1 "The
 *                        recurrence has affine form").
 *   kda_decode_step      one token per sequence, fused recurrent step, the
 *                        state updated in place.
 *   kda_decode           m >= 1 tokens per sequence in one launch (multi-token
 *                        decode / speculative verification), the state read
 *                        once and written once, optionally the state after
 *                        every token for rollback (Module 11, §2 "The full
 *                        correctness matrix", row "Serving state").
 *
 *   kda_short_conv       the short causal convolution that precedes the
 *                        recurrence in the sublayer, with its rolling state.
 *   kda_backward         gradients of the recurrence (reverse mode through the
 *                        chunked form, from the prefill's chunk checkpoints).
 *
 * Both recurrence families can fuse the stages that run just before the
 * recurrence (KDA_PROLOGUE_* flags below).
 *
 * Conventions common to all entry points
 *   - Pointers marked DEVICE are device memory owned by the caller; the
 *     library never allocates, frees or synchronises.  Scratch memory for
 *     prefill is a caller-provided workspace sized by
 *     kda_prefill_workspace_bytes(), or, for kda_prefill_chunked_noalloc, a
 *     fixed array the library's code holds on each GPU.
 *   - Tensors are contiguous, row-major, with the layouts given below.
 *   - Every argument is validated on the host before the first launch; on an
 *     error nothing is launched and nothing is written.  After the launches
 *     a launch failure maps to KDA_ERR_HIP.  Execution is asynchronous on
 *     the given stream (a hipStream_t passed as void*; NULL = default).
 *   - No query scale is applied: callers pre-scale q.
 *   - log_alpha must be <= 0 and all inputs finite; other values are not
 *     checked and propagate (NaN in, NaN out).
 *   - Apart from the fixed scratch of kda_prefill_chunked_noalloc, the
 *     library holds no mutable global state: concurrent calls on different
 *     streams with disjoint outputs and workspaces are safe.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 3

typedef enum {
    KDA_OK = 0,
    KDA_ERR_NULL_ARG = 1,           /* a required pointer is NULL                 */
    KDA_ERR_BAD_SHAPE = 2,          /* sizes inconsistent or out of range         */
    KDA_ERR_UNSUPPORTED = 3,        /* valid but not implemented (dtype, d, C)    */
    KDA_ERR_WORKSPACE_TOO_SMALL = 4,
    KDA_ERR_HIP = 5,                /* a HIP launch failed                        */
    KDA_ERR_BAD_SEQLENS = 6,        /* host-visible cu_seqlens are malformed      */
    KDA_ERR_SCRATCH_LIMIT = 7,      /* needs more than the fixed scratch of
                                       kda_prefill_chunked_noalloc             */
    KDA_ERR_DEVICE_WAIT = 8         /* device-side only (*device_status): a
                                       hand-off between workgroups of the
                                       overlapped prefill failed; the call's
                                       results are undefined                  */
} kda_status;

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

/*
 * Prologue flags (the `prologue` field of the argument structs).  The
 * executed sublayer runs Q/K normalisation, a learned decay gate producing
 * alpha and a learned write gate producing beta just before the recurrence
 * (Module 04 — KDA II, §3 "The sublayer is bigger than the recurrence");
 * each flag fuses one of them into the kernels, so that the argument holds
 * the pre-activation x instead of the value:
 *   GATE_SOFTPLUS  log_alpha holds x; the kernels use log alpha = -softplus(x)
 *                  = -log(1 + e^x) (alpha = 1 / (1 + e^x)), computed in fp32.
 *   BETA_SIGMOID   beta holds x; beta = 1 / (1 + e^-x).
 *   QK_L2NORM      q and k are divided by sqrt(sum_c x_c^2 + 1e-6) over their
 *                  d_k channels, per (token, head), in fp32 (the inputs are
 *                  not rounded again after the division).
 * The pages name the stages without formulas; these are the forms the
 * workload descriptions apply to their inputs.  Unknown bits are
 * KDA_ERR_UNSUPPORTED.
 */
#define KDA_PROLOGUE_GATE_SOFTPLUS 1u
#define KDA_PROLOGUE_BETA_SIGMOID 2u
#define KDA_PROLOGUE_QK_L2NORM 4u
#define KDA_PROLOGUE_ALL 7u

/*
 * Prefill arguments.  Sequences are either the B rows of a batch
 * (cu_seqlens == NULL, num_seqs == B) or documents packed along T
 * (B == 1, cu_seqlens != NULL, num_seqs == len(cu_seqlens) - 1); documents
 * never share state (Module 11, §2, row "Padding / packing").
 *
 *   q, k        DEVICE [B, T, H, d_k]  in_dtype
 *   v           DEVICE [B, T, H, d_v]  in_dtype
 *   beta        DEVICE [B, T, H]       in_dtype, expected in [0, 1]
 *   log_alpha   DEVICE [B, T, H, d_k]  in_dtype, <= 0
 *   cu_seqlens  DEVICE int32 [num_seqs + 1]: 0 = cu[0] <= cu[1] <= ... <=
 *               cu[num_seqs] = T.  Checked on the device before any other
 *               kernel reads it: if malformed, no kernel writes o or any
 *               state and *device_status (if given) is set to
 *               KDA_ERR_BAD_SEQLENS.
 *   cu_seqlens_host  HOST, optional copy of cu_seqlens; when given it is
 *               validated on the host as well (KDA_ERR_BAD_SEQLENS).
 *   initial_state DEVICE fp32 [num_seqs, H, d_k, d_v], NULL = zeros.
 *   final_state DEVICE fp32 [num_seqs, H, d_k, d_v], NULL = not written.
 *               May alias initial_state (in-place continuation).
 *   chunk_states DEVICE fp32, NULL = not written: the state ENTERING every
 *               chunk, documents in order, [sum_n ceil(len_n / C), H, d_k, d_v]
 *               (the chunk-boundary states of Module 04, §4 "The correctness
 *               invariant").  Its size is bounded by
 *               kda_prefill_max_chunks() * H * d_k * d_v floats.
 *   o           DEVICE [B, T, H, d_v]  out_dtype (fp32 recommended: a bf16
 *               output alone costs ~2^-9 relative per element).
 *   device_status DEVICE int32, NULL = not reported; written 0 or an error.
 *   workspace   DEVICE, >= kda_prefill_workspace_bytes(args), 256-byte aligned.
 *   timing_events  HOST, nullable: pointer to 3 hipEvent_t created by the
 *               caller; recorded on hip_stream before the first kernel
 *               (the chunk table), between the per-chunk kernel and the scan
 *               kernel (after the single kernel on the fp32 vector-ALU path)
 *               and after the last kernel.  A profiling hook; costs nothing
 *               when NULL.
 *   prologue    KDA_PROLOGUE_* bits, 0 = q, k, beta, log_alpha used as given.
 *
 * Supported: d_k, d_v in {16, 32, 64, 128}; chunk_size in {16, 32, 64};
 * in_dtype f32 or bf16; out_dtype f32 or bf16.  Paths (all with fp32 state
 * and accumulation): bf16 inputs with d_k == d_v in {64, 128} run on bf16
 * matrix cores, reading q, k, v and log_alpha as 128-bit vectors (each
 * must be 16-byte aligned there, else KDA_ERR_UNSUPPORTED); every other
 * case (fp32 inputs for the 1e-5 contract, other
 * bf16 head sizes) runs on the fp32 matrix cores, with a workspace of about
 * 209 KB (d_k = 128) per (chunk, head) whatever the chunk size
 * (chunk_size 16 only while that stays within 4 GiB); larger chunk-16 calls
 * run in fp32 on the vector ALUs.
 *
 * On the bf16 matrix-core path, one sequence (num_seqs == 1) whose
 * inter-chunk scan needs at most 16 workgroups per XCD (ceil(H / 8) *
 * d_v / 16 <= 16) with chunk_size 64 runs, on a device with 256 CUs, as one
 * launch in which the scan consumes each chunk's intermediate block as soon
 * as it is written (Module 04 — KDA II, §2: the per-chunk work is parallel,
 * only the composition across chunks is sequential).  fp32 inputs with
 * d_k = 128 on the fp32 matrix-core path (any chunk size) overlap the same
 * way when one sequence's scan needs at most 16 workgroups per XCD.
 * Results are bitwise those of the two-kernel launch, which
 * KDA_PREFILL_OVERLAP=0 in the environment forces.  Its cross-workgroup waits are bounded (1 s, or
 * KDA_PREFILL_WAIT_TICKS ticks of the device's 100 MHz real-time counter
 * from the environment, for tests of this path): a hand-off that does not
 * complete sets *device_status to KDA_ERR_DEVICE_WAIT, every kernel still
 * runs to its end, and the call's results are undefined.
 */
typedef struct kda_prefill_args {
    int32_t B, T, H, d_k, d_v;
    int32_t num_seqs;
    int32_t chunk_size;
    int32_t in_dtype;              /* kda_dtype */
    int32_t out_dtype;             /* kda_dtype */
    const void *q, *k, *v, *beta, *log_alpha;
    const int32_t *cu_seqlens;
    const int32_t *cu_seqlens_host;
    const float *initial_state;
    float *final_state;
    float *chunk_states;
    void *o;
    int32_t *device_status;
    void *workspace;
    size_t workspace_bytes;
    void *timing_events;
    uint32_t prologue;
} kda_prefill_args;

/* Workspace bytes the call described by *a needs (0 if a is NULL or
 * invalid).  Pure host function; depends only on sizes and dtypes. */
size_t kda_prefill_workspace_bytes(const kda_prefill_args *a);

/* Upper bound on sum_n ceil(len_n / C): ceil(T / C) + num_seqs for packed
 * input, B * ceil(T / C) otherwise.  Pure host function. */
int64_t kda_prefill_max_chunks(const kda_prefill_args *a);

/* Chunked prefill over all sequences and heads.  Returns KDA_OK once the
 * kernels are enqueued on hip_stream. */
kda_status kda_prefill_chunked(const kda_prefill_args *a, void *hip_stream);

/*
 * Allocation-free variant of kda_prefill_chunked, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same operation, arguments, validation
 * and results as kda_prefill_chunked, except that the scratch comes from a
 * fixed device array inside the library instead of a->workspace (which is
 * ignored, with a->workspace_bytes):
 *   - the array holds KDA_NOALLOC_SCRATCH_BYTES on every GPU the library runs
 *     on, from the load of the library's code on that GPU until the process
 *     ends; its device address is looked up once per GPU, on the first call
 *     for that GPU (the GPU owning hip_stream, or the current one for NULL);
 *   - a call whose scratch need (kda_prefill_workspace_bytes) exceeds it
 *     returns KDA_ERR_SCRATCH_LIMIT before anything is launched;
 *   - nothing is allocated or freed (no hipMalloc, hipFree or allocating
 *     library routine);
 *   - every call on one GPU shares that GPU's array and finds the previous
 *     call's contents there (each call rewrites all it reads): calls that
 *     overlap in time on one GPU (on different streams, or from threads
 *     without ordering) race and give undefined results; calls ordered on
 *     one stream are safe.
 * The caller still provides every input and output buffer.
 */
#define KDA_NOALLOC_SCRATCH_BYTES (256u << 20)
kda_status kda_prefill_chunked_noalloc(const kda_prefill_args *a, void *hip_stream);

/*
 * One decode step for B independent sequences (one token each), fused:
 * the state is read once and written once per (sequence, head)
 * (Module 04, §2: decode uses a fused recurrent kernel).
 *
 *   q, k, log_alpha  DEVICE [B, H, d_k]  in_dtype
 *   v                DEVICE [B, H, d_v]  in_dtype
 *   beta             DEVICE [B, H]       in_dtype
 *   state            DEVICE fp32 [B, H, d_k, d_v], updated in place
 *   o                DEVICE [B, H, d_v]  out_dtype
 * Supported: d_k, d_v in {16, 32, 64, 128}; dtypes as for prefill.
 */
kda_status kda_decode_step(int32_t B, int32_t H, int32_t d_k, int32_t d_v,
                           int32_t in_dtype, int32_t out_dtype,
                           const void *q, const void *k, const void *v,
                           const void *beta, const void *log_alpha,
                           float *state, void *o, void *hip_stream);

/*
 * m >= 1 consecutive tokens for each of B independent sequences in one
 * launch: multi-token decode and speculative verification, where a rejected
 * suffix must be rolled back to the state after the last accepted token
 * (Module 11, §2 "The full correctness matrix", row "Serving state"; the
 * course index's module list, Module 08 "Vision, MTP, and Hybrid Serving
 * State", on why a rollback must restore the recurrent state).
 * Per (sequence, head) the state is read once, the m tokens are applied in
 * registers, and the results are written once.  With 2 <= m <= 4 and no
 * token_states the m tokens are applied in the chunked form of the
 * recurrence (Module 04 — KDA II, §1 "The recurrence has affine form"): one
 * pass of reductions over the state and a rank-m update, equal to applying
 * them one by one up to fp32 rounding; otherwise token by token with the
 * same fused step as kda_decode_step.
 *
 *   q, k, log_alpha  DEVICE [B, m, H, d_k]  in_dtype
 *   v                DEVICE [B, m, H, d_v]  in_dtype
 *   beta             DEVICE [B, m, H]       in_dtype
 *   initial_state    DEVICE fp32 [B, H, d_k, d_v]: the state before token 0.
 *   final_state      DEVICE fp32 [B, H, d_k, d_v], NULL = not written: the
 *                    state after token m - 1.  May alias initial_state (in
 *                    place); leave it NULL to keep initial_state for a
 *                    rollback to zero accepted tokens.
 *   token_states     DEVICE fp32 [B, m, H, d_k, d_v], NULL = not written:
 *                    the state after every token (m x the state traffic).
 *   o                DEVICE [B, m, H, d_v]  out_dtype; o[b, j] uses the
 *                    state after token j.
 *   prologue         KDA_PROLOGUE_* bits.
 * Supported: d_k, d_v in {16, 32, 64, 128}; 1 <= m; B * m * H < 2^31; the
 * three state pointers 16-byte aligned (the kernel moves state rows as
 * 128-bit vectors), else KDA_ERR_UNSUPPORTED.
 */
typedef struct kda_decode_args {
    int32_t B, H, d_k, d_v;
    int32_t n_tokens;
    int32_t in_dtype;              /* kda_dtype */
    int32_t out_dtype;             /* kda_dtype */
    uint32_t prologue;
    const void *q, *k, *v, *beta, *log_alpha;
    const float *initial_state;
    float *final_state;
    float *token_states;
    void *o;
} kda_decode_args;

kda_status kda_decode(const kda_decode_args *a, void *hip_stream);

/*
 * Short causal convolution with a rolling state: the small local mixing step
 * the executed sublayer applies to q, k and/or v before the recurrence
 * (Module 04 — KDA II, §3 "The sublayer is bigger than the recurrence").
 * Its state, the last W - 1 inputs of each sequence, is serving state that a
 * rollback restores (Module 11, §2, row "Serving state").  The pages give
 * neither its width nor its form; this is a depthwise causal filter:
 *
 *     y_t[c] = sum_{j=0}^{W-1} weight[c][j] * x_{t-W+1+j}[c]  (+ bias[c]),
 *     then y * sigmoid(y) if activation == KDA_CONV_SILU,
 *
 * taps ordered oldest input first; inputs before a sequence's first token
 * come from its initial state (zeros when NULL).  Prefill passes whole
 * sequences; decode passes B rows of m tokens with the state updated in
 * place (final_state == initial_state).
 *
 *   x             DEVICE [B, T, C]  in_dtype (C = channels, e.g. H * d)
 *   weight        DEVICE fp32 [C, W]
 *   bias          DEVICE fp32 [C], NULL = none
 *   cu_seqlens    DEVICE int32 [num_seqs + 1], NULL = the B rows are the
 *                 sequences; else B == 1 and documents are packed along T
 *                 (offsets are not validated: malformed offsets give
 *                 unspecified values, never an out-of-range access)
 *   initial_state DEVICE fp32 [num_seqs, C, W - 1], oldest input first,
 *                 NULL = zeros
 *   final_state   DEVICE fp32 [num_seqs, C, W - 1], NULL = not written: the
 *                 last W - 1 inputs of each sequence (from its initial state
 *                 where the sequence is shorter).  May alias initial_state.
 *   y             DEVICE [B, T, C]  out_dtype
 * Supported: 1 <= W <= 8; C a positive multiple of 8; B * T * C < 2^31;
 * x, y and the states 16-byte aligned.
 */
#define KDA_CONV_NONE 0
#define KDA_CONV_SILU 1
typedef struct kda_conv_args {
    int32_t B, T, C, W;
    int32_t num_seqs;
    int32_t in_dtype;              /* kda_dtype */
    int32_t out_dtype;             /* kda_dtype */
    int32_t activation;            /* KDA_CONV_NONE or KDA_CONV_SILU */
    const void *x;
    const float *weight;
    const float *bias;
    const int32_t *cu_seqlens;
    const float *initial_state;
    float *final_state;
    void *y;
} kda_conv_args;

kda_status kda_short_conv(const kda_conv_args *a, void *hip_stream);

/*
 * Backward pass: gradients of q, k, v, beta, log_alpha and the initial state
 * from the gradients of o and of the final state.  The pages call the affine
 * composition the argument for parallel training (course index, module
 * list, the Module 04 entry) but derive no backward; this is reverse-mode
 * differentiation, in fp32, of the chunked form (bf16 inputs: every chunk's
 * gradients from its structured matrices, the chunks coupled by a reverse
 * scan of the state gradient) or of the token operations (fp32 inputs, last
 * token first, states recomputed token by token).  Both start from
 * checkpoints: the state entering every chunk of chunk_size tokens, exactly
 * what kda_prefill_chunked writes to chunk_states when called with that
 * chunk_size on the same inputs and initial state.
 *
 *   chunk_size   the checkpoint spacing: 16, 32 or 64 for bf16 inputs (64
 *                recommended), 16 for fp32 inputs.
 *
 *   q, k, v, beta, log_alpha, cu_seqlens, B, T, H, d_k, d_v, num_seqs,
 *   in_dtype     as for kda_prefill_chunked (no prologue: the gradients are
 *                with respect to the recurrence's own inputs)
 *   checkpoints  DEVICE fp32 [sum_n ceil(len_n / chunk_size), H, d_k, d_v]
 *   d_o          DEVICE fp32 [B, T, H, d_v]
 *   d_final_state DEVICE fp32 [num_seqs, H, d_k, d_v], NULL = zeros
 *   dq, dk, dlog_alpha  DEVICE fp32 [B, T, H, d_k]    (written)
 *   dv           DEVICE fp32 [B, T, H, d_v]            (written)
 *   dbeta        DEVICE fp32 [B, T, H]                 (written)
 *   d_initial_state DEVICE fp32 [num_seqs, H, d_k, d_v], NULL = not written
 *   workspace    DEVICE, >= kda_backward_workspace_bytes(args), 256-aligned
 * With fp32 inputs dq, dk, dlog_alpha and dbeta are sums over the state's
 * column tiles taken with fp32 atomics: their rounding may differ from run to
 * run; the bf16 path is deterministic.
 * Supported: d_k, d_v in {16, 32, 64, 128}; in_dtype f32 or bf16; with bf16
 * inputs checkpoints and d_o must be 16-byte aligned (KDA_ERR_UNSUPPORTED
 * otherwise).
 * The first int32 word of the workspace holds the call's device status once
 * it has run (0, or KDA_ERR_BAD_SEQLENS for malformed cu_seqlens).
 */
typedef struct kda_backward_args {
    int32_t B, T, H, d_k, d_v;
    int32_t num_seqs;
    int32_t in_dtype;              /* kda_dtype */
    int32_t chunk_size;            /* checkpoint spacing */
    const void *q, *k, *v, *beta, *log_alpha;
    const int32_t *cu_seqlens;
    const float *checkpoints;
    const float *d_o;
    const float *d_final_state;
    float *dq, *dk, *dv, *dbeta, *dlog_alpha;
    float *d_initial_state;
    void *workspace;
    size_t workspace_bytes;
} kda_backward_args;

size_t kda_backward_workspace_bytes(const kda_backward_args *a);
kda_status kda_backward(const kda_backward_args *a, void *hip_stream);

/* Static description of a status code (never NULL). */
const char *kda_status_string(int32_t status);

/* KDA_ABI_VERSION of the loaded library. */
int32_t kda_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H */
