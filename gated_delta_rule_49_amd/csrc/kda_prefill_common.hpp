// Parameters and sequence/chunk bookkeeping shared by the prefill kernels.
#pragma once
#include "kda_common.hpp"

namespace kda {

struct PrefillParams {
    const void *q, *k, *v, *beta, *log_alpha;
    void *o;
    const float *initial_state;
    float *final_state;
    float *chunk_states;
    const int32_t *cu_seqlens;   // device, may be null (B rows of T tokens)
    const int32_t *chunk_off;    // device [N+1] first chunk of each sequence (workspace)
    const int4 *chunk_info;      // device [chunks] (token start lo, hi, length, sequence) (workspace)
    int32_t *status;             // device, workspace word: 0 = inputs valid
    int32_t *user_status;        // device, optional mirror of *status
    int32_t B, T, H, dk, dv, N, C;
    int32_t n_chunks_bound;      // grid bound on the total number of chunks
    uint32_t prologue;           // kPro* bits: which inputs are pre-activations
    int32_t *ready;              // device, nullable: role counters and per-(head, chunk) flags of the overlapped launch (workspace)
    uint64_t wait_ticks;         // bound of the overlapped launch's waits, in 100 MHz real-time ticks
};

// Token range of sequence n: tokens [start, start + len) of the flattened
// (B*T) token axis.
struct SeqRange {
    int64_t start;
    int32_t len;
};

__device__ __forceinline__ SeqRange seq_range(const PrefillParams &p, int n) {
    SeqRange r;
    if (p.cu_seqlens) {
        r.start = p.cu_seqlens[n];
        r.len = p.cu_seqlens[n + 1] - p.cu_seqlens[n];
    } else {
        r.start = static_cast<int64_t>(n) * p.T;
        r.len = p.T;
    }
    return r;
}

// global chunk index x -> sequence n (binary search in chunk_off[0..N])
__device__ __forceinline__ int chunk_to_seq(const int32_t *chunk_off, int N, int x) {
    int lo = 0, hi = N;  // invariant: chunk_off[lo] <= x < chunk_off[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (chunk_off[mid] <= x) lo = mid; else hi = mid;
    }
    return lo;
}

}  // namespace kda
