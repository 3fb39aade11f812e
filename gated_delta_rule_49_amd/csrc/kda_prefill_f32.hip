// Chunked KDA prefill computed entirely in fp32 on the vector ALUs.
//
// This is the path for fp32 inputs (the 1e-5 contract needs true fp32
// arithmetic end to end) and for head sizes the matrix-core path does not
// cover.  It follows the same chunk decomposition as the matrix-core path:
// Module 04 — KDA II, §1 "The recurrence has affine form": each chunk's
// composed transition is independent of the incoming state and is kept in
// structured form (diagonal decay plus a rank-L correction), never as a dense
// d_k x d_k matrix.  For a chunk of L tokens with incoming state S, per-channel
// cumulative log-decay G_r = sum_{i<=r} log_alpha_i and
//     A_ri = beta_r sum_c k_r[c] k_i[c] exp(G_r[c] - G_i[c])   (i < r)
//     P_ri =        sum_c q_r[c] k_i[c] exp(G_r[c] - G_i[c])   (i <= r)
//     T    = (I + A)^-1 Diag(beta)
//     Delta = T (V - (k * exp(G)) S)          rows are the per-token errors
//     O     = (q * exp(G)) S + P Delta
//     S'    = Diag(exp(G_L)) S + (k * exp(G_L - G))^T Delta
// All exponents are <= 0 (pairs i <= r), so nothing overflows.  G is
// accumulated and held in fp64 and differences are taken in fp64 before one
// fp32 exp: a cumulative log-decay of magnitude ~50 held in fp32 would put
// ~1e-5 relative error on every decay factor, the size of the fp32 contract.
//
// One workgroup per (sequence, head, BV-column tile of the state): the
// columns of S evolve independently.  Everything a chunk needs sits in LDS.
#include "kda_launch.hpp"

namespace kda {

constexpr int F32_THREADS = 256;
constexpr int F32_BV = 16;

__host__ __device__ inline size_t f32_lds_floats(int C, int dk) {
    return 2 * static_cast<size_t>(C) * dk  // G (fp64)
           + static_cast<size_t>(C) * C     // A, then T, then P
           + static_cast<size_t>(dk) * F32_BV  // S tile
           + static_cast<size_t>(C) * F32_BV   // X, then Delta
           + 3 * static_cast<size_t>(C);       // beta, 1/|k|, 1/|q|
}

template <typename TI, typename TO>
__global__ void __launch_bounds__(F32_THREADS) prefill_f32_kernel(PrefillParams p) {
    if (*p.status != 0) return;
    extern __shared__ float lds[];
    const int C = p.C, dk = p.dk, dv = p.dv, H = p.H;
    const int nvt = dv / F32_BV;
    const int vt = blockIdx.x % nvt;
    const int h = (blockIdx.x / nvt) % H;
    const int n = blockIdx.x / (nvt * H);
    const int v0 = vt * F32_BV;
    const int tid = threadIdx.x;

    double *G = reinterpret_cast<double *>(lds);  // [C][dk]
    float *AT = lds + 2 * C * dk;   // [C][C]
    float *S = AT + C * C;          // [dk][BV]
    float *X = S + dk * F32_BV;     // [C][BV]
    float *bet = X + C * F32_BV;    // [C]
    float *nk = bet + C;            // [C] 1/|k_r| (1 without the q/k norm)
    float *nq = nk + C;             // [C] 1/|q_r|

    const TI *q = static_cast<const TI *>(p.q);
    const TI *k = static_cast<const TI *>(p.k);
    const TI *v = static_cast<const TI *>(p.v);
    const TI *beta = static_cast<const TI *>(p.beta);
    const TI *la = static_cast<const TI *>(p.log_alpha);
    TO *o = static_cast<TO *>(p.o);

    const SeqRange sr = seq_range(p, n);
    const int64_t state_off = (static_cast<int64_t>(n) * H + h) * dk * dv;
    for (int e = tid; e < dk * F32_BV; e += F32_THREADS) {
        const int c = e / F32_BV, j = e % F32_BV;
        S[e] = p.initial_state ? p.initial_state[state_off + static_cast<int64_t>(c) * dv + v0 + j] : 0.f;
    }
    const int nch = (sr.len + C - 1) / C;
    const int64_t cbase = p.chunk_off[n];
    __syncthreads();

    for (int ch = 0; ch < nch; ++ch) {
        const int64_t t0 = sr.start + static_cast<int64_t>(ch) * C;
        const int L = min(C, sr.len - ch * C);
        // token t, head h -> row offsets
        auto kv = [&](int64_t t) { return (t * H + h); };

        if (p.chunk_states) {
            float *cs = p.chunk_states + ((cbase + ch) * H + h) * static_cast<int64_t>(dk) * dv;
            for (int e = tid; e < dk * F32_BV; e += F32_THREADS) {
                const int c = e / F32_BV, j = e % F32_BV;
                cs[static_cast<int64_t>(c) * dv + v0 + j] = S[e];
            }
        }
        // 1. cumulative log-decay (fp64), beta, q/k norms; padded rows decay by 1.
        //    Prologue (pre-activations): log alpha = -softplus(x), beta =
        //    sigmoid(x), 1/|.| = 1/sqrt(sum x^2 + eps), in fp32.
        for (int c = tid; c < dk; c += F32_THREADS) {
            double acc = 0.0;
            for (int r = 0; r < C; ++r) {
                if (r < L) {
                    float g = io<TI>::ld(la, kv(t0 + r) * dk + c);
                    if (p.prologue & kProGate) g = -(fmaxf(g, 0.f) + log1pf(expf(-fabsf(g))));
                    acc += static_cast<double>(g);
                }
                G[r * dk + c] = acc;
            }
        }
        for (int r = tid; r < C; r += F32_THREADS) {
            float b = 0.f, ik = 1.f, iq = 1.f;
            if (r < L) {
                b = io<TI>::ld(beta, kv(t0 + r));
                if (p.prologue & kProBeta) b = 1.f / (1.f + expf(-b));
                if (p.prologue & kProQKNorm) {
                    float sk = 0.f, sq = 0.f;
                    for (int c = 0; c < dk; ++c) {
                        const float x = io<TI>::ld(k, kv(t0 + r) * dk + c), y = io<TI>::ld(q, kv(t0 + r) * dk + c);
                        sk += x * x;
                        sq += y * y;
                    }
                    ik = 1.f / sqrtf(sk + kQKNormEps);
                    iq = 1.f / sqrtf(sq + kQKNormEps);
                }
            }
            bet[r] = b;
            nk[r] = ik;
            nq[r] = iq;
        }
        __syncthreads();

        // 2. A (strictly lower, rows scaled by beta)
        for (int e = tid; e < C * C; e += F32_THREADS) {
            const int r = e / C, i = e % C;
            float acc = 0.f;
            if (i < r && r < L) {
                const int64_t kr = kv(t0 + r) * dk, ki = kv(t0 + i) * dk;
                for (int c = 0; c < dk; ++c)
                    acc += io<TI>::ld(k, kr + c) * io<TI>::ld(k, ki + c) *
                           expf(static_cast<float>(G[r * dk + c] - G[i * dk + c]));
                acc *= bet[r] * nk[r] * nk[i];
            }
            AT[e] = acc;
        }
        __syncthreads();

        // 3. T = (I + A)^-1 Diag(beta), row by row, overwriting A in place:
        //    T[r, :] = beta_r e_r - sum_{i<r} A[r, i] T[i, :]
        for (int r = 0; r < C; ++r) {
            float val = 0.f;
            const int j = tid;
            if (j < C) {
                val = (j == r) ? bet[r] : 0.f;
                for (int i = j; i < r; ++i) val -= AT[r * C + i] * AT[i * C + j];
            }
            __syncthreads();
            if (j < C) AT[r * C + j] = (j <= r) ? val : 0.f;
            __syncthreads();
        }

        // 4. X = V - (k * exp(G)) S
        for (int e = tid; e < C * F32_BV; e += F32_THREADS) {
            const int r = e / F32_BV, j = e % F32_BV;
            float acc = 0.f;
            if (r < L) {
                const int64_t kr = kv(t0 + r) * dk;
                for (int c = 0; c < dk; ++c)
                    acc += io<TI>::ld(k, kr + c) * expf(static_cast<float>(G[r * dk + c])) * S[c * F32_BV + j];
                acc = io<TI>::ld(v, kv(t0 + r) * dv + v0 + j) - acc * nk[r];
            }
            X[e] = acc;
        }
        __syncthreads();
        // 5. Delta = T X (in place through registers)
        float dreg[(64 * F32_BV + F32_THREADS - 1) / F32_THREADS];
        {
            int idx = 0;
            for (int e = tid; e < C * F32_BV; e += F32_THREADS, ++idx) {
                const int r = e / F32_BV, j = e % F32_BV;
                float acc = 0.f;
                for (int i = 0; i <= r; ++i) acc += AT[r * C + i] * X[i * F32_BV + j];
                dreg[idx] = acc;
            }
        }
        __syncthreads();
        {
            int idx = 0;
            for (int e = tid; e < C * F32_BV; e += F32_THREADS, ++idx) X[e] = dreg[idx];
        }
        __syncthreads();

        // 6. P (inclusive lower) into the A/T buffer
        for (int e = tid; e < C * C; e += F32_THREADS) {
            const int r = e / C, i = e % C;
            float acc = 0.f;
            if (i <= r && r < L) {
                const int64_t qr = kv(t0 + r) * dk, ki = kv(t0 + i) * dk;
                for (int c = 0; c < dk; ++c)
                    acc += io<TI>::ld(q, qr + c) * io<TI>::ld(k, ki + c) *
                           expf(static_cast<float>(G[r * dk + c] - G[i * dk + c]));
                acc *= nq[r] * nk[i];
            }
            AT[e] = acc;
        }
        __syncthreads();

        // 7. O = (q * exp(G)) S + P Delta
        for (int e = tid; e < C * F32_BV; e += F32_THREADS) {
            const int r = e / F32_BV, j = e % F32_BV;
            if (r < L) {
                const int64_t qr = kv(t0 + r) * dk;
                float acc = 0.f;
                for (int c = 0; c < dk; ++c)
                    acc += io<TI>::ld(q, qr + c) * expf(static_cast<float>(G[r * dk + c])) * S[c * F32_BV + j];
                acc *= nq[r];
                for (int i = 0; i <= r; ++i) acc += AT[r * C + i] * X[i * F32_BV + j];
                io<TO>::st(o, kv(t0 + r) * dv + v0 + j, acc);
            }
        }
        // 8. S' = Diag(exp(G_L)) S + (k * exp(G_L - G))^T Delta
        float sreg[(128 * F32_BV + F32_THREADS - 1) / F32_THREADS];
        {
            int idx = 0;
            for (int e = tid; e < dk * F32_BV; e += F32_THREADS, ++idx) {
                const int c = e / F32_BV, j = e % F32_BV;
                const double gl = G[(C - 1) * dk + c];
                float acc = expf(static_cast<float>(gl)) * S[e];
                for (int r = 0; r < L; ++r)
                    acc += io<TI>::ld(k, kv(t0 + r) * dk + c) * nk[r] * expf(static_cast<float>(gl - G[r * dk + c])) *
                           X[r * F32_BV + j];
                sreg[idx] = acc;
            }
        }
        __syncthreads();
        {
            int idx = 0;
            for (int e = tid; e < dk * F32_BV; e += F32_THREADS, ++idx) S[e] = sreg[idx];
        }
        __syncthreads();
    }
    if (p.final_state) {
        for (int e = tid; e < dk * F32_BV; e += F32_THREADS) {
            const int c = e / F32_BV, j = e % F32_BV;
            p.final_state[state_off + static_cast<int64_t>(c) * dv + v0 + j] = S[e];
        }
    }
}

}  // namespace kda

namespace kda {

namespace {
template <typename TI, typename TO>
hipError_t run_f32(const PrefillParams &p, hipStream_t s) {
    const size_t lds = f32_lds_floats(p.C, p.dk) * sizeof(float);
    auto kern = prefill_f32_kernel<TI, TO>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    const unsigned grid = static_cast<unsigned>(p.N) * p.H * (p.dv / F32_BV);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(F32_THREADS), lds, s, p);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_prefill_f32(const PrefillParams &p, int in_dtype, int out_dtype, hipStream_t s) {
    if (in_dtype == 0 && out_dtype == 0) return run_f32<float, float>(p, s);
    if (in_dtype == 0 && out_dtype == 1) return run_f32<float, bf16_t>(p, s);
    if (in_dtype == 1 && out_dtype == 0) return run_f32<bf16_t, float>(p, s);
    return run_f32<bf16_t, bf16_t>(p, s);
}

}  // namespace kda
