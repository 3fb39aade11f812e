// The per-(chunk, head) block that the chunk prep kernel writes (fp32,
// row-major) and that the chunked backward and the fp32 matrix-core prefill
// read: the chunk's cumulative decay and the structured-form factors
//     K~ = k e^G, Q~ = q e^G, K^ = k e^{G_L - G}, g = e^{G_L},
//     Gh = strict-lower(k k^T e^{G_r - G_i}), P = lower(q k^T e^{G_r - G_i}),
//     M = (I + Diag(beta) Gh)^-1, W = M Diag(beta) K~
// (Module 04 — KDA II: Chunked Parallelism & the Full Sublayer, §1 "The
// recurrence has affine form").
#pragma once
#include <stddef.h>

namespace kda {

constexpr int CB_C = 64;  // maximum chunk length
// a diagonal 16-token block of the prep's Gram products is factorised around
// its midpoint while it decays by at most this many nats in every channel
constexpr float kCbDiagSpan = 80.f;

// per-(chunk, head) block of the prep kernel, fp32, row-major; consumers
// that need P^T or M^T read P or M with the indices swapped
template <int DK>
struct CbLay {
    static constexpr size_t G = 0;                       // [C][DK]  cumulative log decay
    static constexpr size_t KT = G + CB_C * DK;          // [C][DK]  k e^G
    static constexpr size_t QT = KT + CB_C * DK;         // [C][DK]  q e^G
    static constexpr size_t KB = QT + CB_C * DK;         // [C][DK]  k e^{G_L - G}
    static constexpr size_t W = KB + CB_C * DK;          // [C][DK]  T K~
    static constexpr size_t GH = W + CB_C * DK;          // [C][C]   k_r . k_i e^{..}, i < r
    static constexpr size_t P = GH + CB_C * CB_C;        // [C][C]   q_r . k_i e^{..}, i <= r
    static constexpr size_t M = P + CB_C * CB_C;         // [C][C]   (I + A)^-1
    static constexpr size_t GAM = M + CB_C * CB_C;       // [DK]     e^{G_L}
    static constexpr size_t BETA = GAM + DK;             // [C]
    static constexpr size_t FLOATS = (BETA + CB_C + 63) / 64 * 64;
};

// Blocks of the chunk prep in forward mode (read only by the forward fp32
// scan) hold K~, Q~ and M in the register order of the scan's
// v_mfma_f32_16x16x4f32 A operands, so that each wave reads a 16 x 16
// fragment as one contiguous 1 KB (16 bytes per lane); the other parts stay
// row-major.  Element (r, c) of a row-major matrix with ncb 16-column blocks
// sits in fragment (r / 16, c / 16), lane 16 ((c % 16) / 4) + r % 16, slot
// c % 4.
__host__ __device__ constexpr int frag_a(int r, int c, int ncb) {
    return (((r >> 4) * ncb + (c >> 4)) * 64 + 16 * ((c & 15) >> 2) + (r & 15)) * 4 + (c & 3);
}

}  // namespace kda
