// Internal host-side launch interface between the C ABI (kda_api.hip) and
// the kernel translation units.  Arguments are already validated.
#pragma once
#include <hip/hip_runtime.h>
#include "kda_prefill_common.hpp"

namespace kda {

// Workspace layout (byte offsets from the workspace base, 256-aligned):
//   [0, 256)            status word (int32) + padding
//   [256, 256 + 4(N+1)) chunk_off table, rounded up to 256
//   then chunk_info, 16 bytes per chunk (up to the chunk bound), rounded up
//   then, matrix-core path only, the per-(chunk, head) intermediate blocks,
//   then, for the shapes of the overlapped launch, one int32 flag per (chunk, head).
constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline size_t chunk_off_bytes(int N) { return align_up(sizeof(int32_t) * (static_cast<size_t>(N) + 1)); }
inline size_t table_bytes(int N, int64_t n_chunks_bound) {
    return kAlign + chunk_off_bytes(N) + align_up(16 * static_cast<size_t>(n_chunks_bound));
}

// matrix-core path: bytes of intermediates per (chunk, head)
size_t mfma_block_bytes(int C, int D);
bool mfma_supported(int dk, int dv, int C);
// shapes the overlapped matrix-core launch takes (one sequence, few heads);
// after the blocks it needs 64 int32 role counters and one int32 flag per
// (chunk, head), cleared by the chunk-table kernel
bool mfma_overlap_shape(int N, int H, int D, int C);
__host__ __device__ inline size_t mfma_ready_words(int64_t n_chunks_bound, int H) {
    return 64 + static_cast<size_t>(n_chunks_bound) * H;
}
inline size_t mfma_ready_bytes(int64_t n_chunks_bound, int H) {
    return align_up(sizeof(int32_t) * mfma_ready_words(n_chunks_bound, H));
}

hipError_t launch_chunk_table(const PrefillParams &p, hipStream_t s);
hipError_t launch_prefill_f32(const PrefillParams &p, int in_dtype, int out_dtype, hipStream_t s);
// mid_event (nullable) is recorded between the intra-chunk and the scan kernel
hipError_t launch_prefill_mfma(const PrefillParams &p, void *blocks, int out_dtype, hipStream_t s,
                               hipEvent_t mid_event);
// short causal convolution (validated arguments)
struct ConvParams {
    const void *x;              // [B, T, C]
    const float *weight;        // [C, W]
    const float *bias;          // nullable [C]
    const int32_t *cu_seqlens;  // nullable [N + 1] (B == 1)
    const float *initial_state; // nullable [N, C, W - 1]
    float *final_state;         // nullable [N, C, W - 1], may alias initial_state
    void *y;                    // [B, T, C]
    int32_t B, T, C, W, N;
    int32_t silu;
};
hipError_t launch_short_conv(const ConvParams &p, int in_dtype, int out_dtype, hipStream_t s);

// backward pass (validated arguments)
struct BackwardParams {
    const void *q, *k, *v, *beta, *log_alpha;  // [B, T, H, d] / [B, T, H]
    const float *d_o;                          // [B, T, H, dv]
    const float *d_final;                      // nullable [N, H, dk, dv]
    const float *checkpoints;                  // [chunks of 16, H, dk, dv]
    float *gq, *gk, *gv, *gbeta, *gg;          // fp32 gradients of q, k, v, beta, log alpha
    float *d_initial;                          // nullable [N, H, dk, dv]
    const int32_t *cu_seqlens;                 // nullable
    const int32_t *chunk_off;                  // device [N + 1], 16-token chunks (workspace)
    const int32_t *status;                     // device, workspace word: 0 = inputs valid
    int32_t B, T, H, dk, dv, N;
};
hipError_t launch_backward(const BackwardParams &p, int in_dtype, hipStream_t s);

// chunked backward (bf16 inputs): per-(chunk, head) blocks and the dS
// entering every chunk from the right live in the workspace
struct CbParams {
    const void *q, *k, *v, *beta, *log_alpha;  // bf16 [B, T, H, d] / [B, T, H]
    const float *d_o;                          // [B, T, H, dv]
    const float *d_final;                      // nullable [N, H, dk, dv]
    const float *checkpoints;                  // [chunks, H, dk, dv] state entering each chunk
    float *blocks;                             // [chunks, H] prep blocks (workspace)
    float *dS_right;                           // [chunks, H, dk, dv] (workspace)
    float *gq, *gk, *gv, *gbeta, *gg;          // fp32 gradients
    float *d_initial;                          // nullable [N, H, dk, dv]
    const int32_t *chunk_off;                  // [N + 1]
    const int4 *chunk_info;                    // [chunks]
    const int32_t *status;
    int32_t N, H, dk, dv;
    uint32_t prologue;                         // kPro* bits (forward prep only)
};
size_t cb_block_bytes(int dk);
hipError_t launch_backward_chunked(const CbParams &p, int n_items, hipStream_t s);
// the chunk prep kernel in forward mode (K~, Q~, K^, g, beta, P, M per block);
// in_dtype 0 = fp32, 1 = bf16
hipError_t launch_chunk_prep_fwd(const CbParams &p, int n_items, int in_dtype, hipStream_t s);
// fp32 matrix-core prefill: chunk prep (with the prologue, if any), then
// the forward scan; blocks = n_chunks_bound x H prep blocks
bool f32mm_supported(int dk, int dv, int C, uint32_t prologue);
// shapes the overlapped fp32 prefill takes (one sequence, d_k = 128, at most
// 16 scan workgroups per XCD; fp32 inputs); its counters and flags take
// mfma_ready_bytes(chunks, H) after the blocks
bool f32mm_overlap_shape(int N, int H, int dk, int dv);
hipError_t launch_prefill_f32mm(const PrefillParams &p, float *blocks, int in_dtype, int out_dtype, hipStream_t s,
                                hipEvent_t mid);

// m tokens per sequence; state_out and token_states nullable, state_out may
// alias state_in
hipError_t launch_decode(int B, int H, int m, int dk, int dv, int in_dtype, int out_dtype, uint32_t prologue,
                         const void *q, const void *k, const void *v, const void *beta, const void *log_alpha,
                         const float *state_in, float *state_out, float *token_states, void *o, hipStream_t s);

}  // namespace kda
