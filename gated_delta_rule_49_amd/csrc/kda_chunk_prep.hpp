// The chunk prep of the fp32-matrix-core paths (the bf16 backward and, in
// forward mode, the fp32-input prefill): per (chunk, head) the decays and the
// chunk's structured matrices, written to one block of the workspace.
#pragma once
#include <type_traits>

#include "kda_chunk_block.hpp"
#include "kda_launch.hpp"

namespace kda {

// ------------------------------------------------------------------ prep --
// The chunk prep of chunk x, head h (256 threads, static LDS).  FWD: only
// what the forward needs (K~, Q~, K^, g, beta, P, M): no G, Gh, P^T, M^T or
// W.
template <int DK, typename TI, bool FWD>
__device__ __forceinline__ void cb_prep_run(const CbParams &p, int x, int h) {
    using Y = CbLay<DK>;
    const int H = p.H;
    const int4 ci = p.chunk_info[x];
    const int64_t t0 = static_cast<int64_t>(static_cast<uint32_t>(ci.x)) | (static_cast<int64_t>(ci.y) << 32);
    const int L = ci.z;
    const int tid = threadIdx.x;
    float *blk = p.blocks + (static_cast<size_t>(x) * H + h) * Y::FLOATS;
    const TI *q = static_cast<const TI *>(p.q);
    const TI *k = static_cast<const TI *>(p.k);
    const TI *la = static_cast<const TI *>(p.log_alpha);
    const TI *beta = static_cast<const TI *>(p.beta);

    // fp32 inputs (the 1e-5 contract): the cumulative decay stays in fp64,
    // exponents are differences taken in fp64 and exponentials are the
    // correctly rounded expf (a cumulative log-decay of ~50 held in fp32 puts
    // ~4e-6 relative error on a decay factor); bf16 inputs: fp32 and the
    // hardware exp
    constexpr bool kExact = sizeof(TI) == 4;
    using GT = typename std::conditional<kExact, double, float>::type;
    auto ex = [](GT x) { return kExact ? expf(static_cast<float>(x)) : __expf(static_cast<float>(x)); };
    // q and k staged in LDS: the backward's bf16 inputs as their raw bits
    // (exact; nothing rescales them), otherwise fp32.  A = Diag(beta) Gh
    // shares q's storage: it is written once the Gram products have read q.
    // With bf16 q, k the block's LDS is 66.6 KB, so two workgroups fit per CU.
    constexpr bool kRaw = sizeof(TI) == 2 && !FWD;
    using QKT = typename std::conditional<kRaw, bf16_t, float>::type;
    constexpr int QKS = kRaw ? DK + 2 : DK + 1;   // row stride, in elements
    constexpr int QBYTES = CB_C * QKS * static_cast<int>(sizeof(QKT)), ABYTES = CB_C * (CB_C + 1) * 4;
    __shared__ __attribute__((aligned(16))) char sqa[QBYTES > ABYTES ? QBYTES : ABYTES];
    __shared__ QKT sk[CB_C][QKS];
    __shared__ GT sG[CB_C][DK + 1];
    __shared__ float sb[CB_C];
    QKT (*sq)[QKS] = reinterpret_cast<QKT (*)[QKS]>(sqa);
    float (*sA)[CB_C + 1] = reinterpret_cast<float (*)[CB_C + 1]>(sqa);
    auto ldq = [&](int r, int c) -> float {
        if constexpr (kRaw) return bf16_to_f32(sq[r][c]); else return sq[r][c];
    };
    auto ldk = [&](int r, int c) -> float {
        if constexpr (kRaw) return bf16_to_f32(sk[r][c]); else return sk[r][c];
    };

    // Prologue (forward only; the arguments hold pre-activations): log alpha
    // = -softplus(x), beta = sigmoid(x), q and k divided by their L2 norms
    // over d_k; in fp32, with the correctly rounded functions for fp32 inputs.
    const uint32_t pro = FWD ? p.prologue : 0u;
    auto stage = [&](int r, int c, float qv, float kv, float x, bool live) {
        if constexpr (kRaw) {
            sq[r][c] = f32_to_bf16(qv);   // qv, kv came from bf16: exact
            sk[r][c] = f32_to_bf16(kv);
        } else {
            sq[r][c] = qv;
            sk[r][c] = kv;
        }
        if (pro & kProGate)
            x = !live ? 0.f : kExact ? -(fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)))) : -softplus_f32(x);
        sG[r][c] = x;
    };
    // 16-byte loads (8 bf16 or 4 fp32 per request) when the three arrays
    // allow it, all of a thread's requests issued before any is used
    constexpr int VEC = 16 / sizeof(TI);
    constexpr int NVL = CB_C * DK / VEC / 256;  // requests per thread and array
    const bool vec = ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                       reinterpret_cast<uintptr_t>(la)) & 15) == 0;
    bool staged = false;
    if constexpr (NVL >= 1) {
        if (vec) {
            typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
            u32x4 rq[NVL], rk[NVL], ra[NVL];
#pragma unroll
            for (int u = 0; u < NVL; ++u) {
                const int e = (tid + 256 * u) * VEC, r = e / DK, c0 = e % DK;
                const int64_t off = ((t0 + min(r, L - 1)) * H + h) * DK + c0;   // rows >= L: zeroed below
                rq[u] = *reinterpret_cast<const u32x4 *>(q + off);
                rk[u] = *reinterpret_cast<const u32x4 *>(k + off);
                ra[u] = *reinterpret_cast<const u32x4 *>(la + off);
            }
#pragma unroll
            for (int u = 0; u < NVL; ++u) {
                const int e = (tid + 256 * u) * VEC, r = e / DK, c0 = e % DK;
                const bool live = r < L;
                const TI *qe = reinterpret_cast<const TI *>(&rq[u]);
                const TI *ke = reinterpret_cast<const TI *>(&rk[u]);
                const TI *ae = reinterpret_cast<const TI *>(&ra[u]);
#pragma unroll
                for (int j = 0; j < VEC; ++j)
                    stage(r, c0 + j, live ? io<TI>::ld(qe, j) : 0.f, live ? io<TI>::ld(ke, j) : 0.f,
                          live ? io<TI>::ld(ae, j) : 0.f, live);
            }
            staged = true;
        }
    }
    if (!staged) {
        for (int e = tid; e < CB_C * DK; e += 256) {
            const int r = e / DK, c = e % DK;
            const int64_t off = ((t0 + r) * H + h) * DK + c;
            const bool live = r < L;
            stage(r, c, live ? io<TI>::ld(q, off) : 0.f, live ? io<TI>::ld(k, off) : 0.f,
                  live ? io<TI>::ld(la, off) : 0.f, live);
        }
    }
    if (tid < CB_C) {
        float b = tid < L ? io<TI>::ld(beta, (t0 + tid) * H + h) : 0.f;
        if ((pro & kProBeta) && tid < L) b = kExact ? 1.f / (1.f + expf(-b)) : sigmoid_f32(b);
        sb[tid] = b;
    }
    __syncthreads();
    if constexpr (!kRaw) if (pro & kProQKNorm) {  // rows of q and k to unit L2 norm (eps as in the other kernels)
        __shared__ float s_inv[2][CB_C];
        if (tid < 2 * CB_C) {
            const int r = tid % CB_C;
            float sum = 0.f;
            for (int c = 0; c < DK; ++c) {
                const float x = tid < CB_C ? sq[r][c] : sk[r][c];
                sum += x * x;
            }
            s_inv[tid / CB_C][r] = 1.f / sqrtf(sum + kQKNormEps);
        }
        __syncthreads();
        for (int e = tid; e < CB_C * DK; e += 256) {
            const int r = e / DK, c = e % DK;
            sq[r][c] *= s_inv[0][r];
            sk[r][c] *= s_inv[1][r];
        }
        __syncthreads();
    }
    if (tid < DK) {  // cumulative decay, accumulated in fp64
        double acc = 0.0;
        for (int r = 0; r < CB_C; ++r) {
            acc += static_cast<double>(sG[r][tid]);
            sG[r][tid] = static_cast<GT>(acc);
        }
    }
    __syncthreads();
    // elementwise factors and the decay of the whole chunk, four
    // consecutive channels per thread (16-byte stores; in forward mode K~
    // and Q~ go to their fragment-order slots, frag_a)
    for (int e4 = tid; e4 < CB_C * DK / 4; e4 += 256) {
        const int e = 4 * e4, r = e / DK, c0 = e % DK;
        f32x4 gv, kt, qt, kb;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const GT G = sG[r][c0 + j];
            const float E = ex(G);
            gv[j] = static_cast<float>(G);
            kt[j] = ldk(r, c0 + j) * E;
            qt[j] = ldq(r, c0 + j) * E;
            kb[j] = ldk(r, c0 + j) * ex(sG[CB_C - 1][c0 + j] - G);
        }
        if (!FWD) *reinterpret_cast<f32x4 *>(blk + Y::G + e) = gv;
        *reinterpret_cast<f32x4 *>(blk + Y::KT + (FWD ? frag_a(r, c0, DK / 16) : e)) = kt;
        *reinterpret_cast<f32x4 *>(blk + Y::QT + (FWD ? frag_a(r, c0, DK / 16) : e)) = qt;
        *reinterpret_cast<f32x4 *>(blk + Y::KB + e) = kb;
    }
    for (int c = tid; c < DK; c += 256) blk[Y::GAM + c] = ex(sG[CB_C - 1][c]);
    if (tid < CB_C) blk[Y::BETA + tid] = sb[tid];
    // Gh and P in 16 x 16 blocks (R, I <= R) on the fp32 matrix cores: in
    // step s lane l (g = l / 16, n = l % 16) supplies row r = 16R + n and
    // column i = 16I + n of channel c = 16cb + 4g + s, and holds the pairs
    // (16R + 4g + u, 16I + n).  The decay e^{G_r - G_i} is split around a
    // reference: off the diagonal the row m = 16R - 1 between the blocks
    // (both factors <= 1, so an underflow only drops a term below fp32's
    // range); on a diagonal block the per-channel midpoint of the block's
    // own decay (both factors within e^{+-span/2}), or, when the block decays
    // by more than kCbDiagSpan in some channel, pair by pair on the vector
    // ALUs.  Wave w takes diagonal block w and the off-diagonal pairs w and
    // w + 4 of (1,0) (2,0) (2,1) (3,0) (3,1) (3,2).
    {
        const int lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int g = lane >> 4, n = lane & 15;
        // A's values stay in registers until every wave is done with q
        f32x4 av[3];
        int aR[3], aI[3];
        auto emit = [&](int t, int R, int I, const f32x4 &gh, const f32x4 &pp) {
            aR[t] = R;
            aI[t] = I;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int r = 16 * R + 4 * g + u, i = 16 * I + n;
                const bool in = r < L && i <= r;
                const float ghv = (in && i < r) ? gh[u] : 0.f, pv = in ? pp[u] : 0.f;
                blk[Y::P + r * CB_C + i] = pv;
                if (!FWD) blk[Y::GH + r * CB_C + i] = ghv;
                av[t][u] = ghv * sb[r];
            }
        };
#pragma unroll
        for (int t = 0; t < 3; ++t) aR[t] = -1;
        for (int t = 0; t < 3; ++t) {
            int R, I;
            if (t == 0) {
                R = I = wv;
            } else {
                const int q = wv + 4 * (t - 1);
                if (q >= 6) break;
                R = q < 1 ? 1 : q < 3 ? 2 : 3;
                I = q - R * (R - 1) / 2;
            }
            const int r = 16 * R + n, i = 16 * I + n;
            f32x4 gh = {0.f, 0.f, 0.f, 0.f}, pp = gh;
            if (R != I) {
                const int m = 16 * R - 1;
                for (int c0 = 0; c0 < DK; c0 += 16)
#pragma unroll
                    for (int s2 = 0; s2 < 4; ++s2) {
                        const int c = c0 + 4 * g + s2;
                        const float fr = ex(sG[r][c] - sG[m][c]), fc = ex(sG[m][c] - sG[i][c]);
                        const float bk = ldk(i, c) * fc;
                        gh = __builtin_amdgcn_mfma_f32_16x16x4f32(ldk(r, c) * fr, bk, gh, 0, 0, 0);
                        pp = __builtin_amdgcn_mfma_f32_16x16x4f32(ldq(r, c) * fr, bk, pp, 0, 0, 0);
                    }
                emit(t, R, I, gh, pp);
                continue;
            }
            // diagonal block: the steepest channel decides the method
            float span = 0.f;
            for (int c = lane; c < DK; c += 64)
                span = fmaxf(span, static_cast<float>((R > 0 ? sG[16 * R - 1][c] : GT(0)) - sG[16 * R + 15][c]));
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) span = fmaxf(span, __shfl_xor(span, o));
            if (span <= kCbDiagSpan) {
                for (int c0 = 0; c0 < DK; c0 += 16)
#pragma unroll
                    for (int s2 = 0; s2 < 4; ++s2) {
                        const int c = c0 + 4 * g + s2;
                        const GT mid = GT(0.5) * ((R > 0 ? sG[16 * R - 1][c] : GT(0)) + sG[16 * R + 15][c]);
                        const float fr = ex(sG[r][c] - mid), fc = ex(mid - sG[r][c]);
                        const float bk = ldk(r, c) * fc;   // columns are the same 16 tokens
                        gh = __builtin_amdgcn_mfma_f32_16x16x4f32(ldk(r, c) * fr, bk, gh, 0, 0, 0);
                        pp = __builtin_amdgcn_mfma_f32_16x16x4f32(ldq(r, c) * fr, bk, pp, 0, 0, 0);
                    }
            } else {
                // lane holds the pairs (16R + 4g + u, 16R + n) of the accumulator layout
                for (int c = 0; c < DK; ++c) {
                    const GT gi = sG[i][c];
                    const float ki = ldk(i, c);
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int ru = 16 * R + 4 * g + u;
                        const GT d = sG[ru][c] - gi;
                        const float f = ki * ex(d < GT(0) ? d : GT(0));
                        gh[u] += ldk(ru, c) * f;
                        pp[u] += ldq(ru, c) * f;
                    }
                }
            }
            emit(t, R, I, gh, pp);
        }
        __syncthreads();   // q is dead: A takes its storage
#pragma unroll
        for (int t = 0; t < 3; ++t) {
            if (aR[t] < 0) continue;
#pragma unroll
            for (int u = 0; u < 4; ++u) sA[16 * aR[t] + 4 * g + u][16 * aI[t] + n] = av[t][u];
        }
    }
    // blocks above the diagonal are zero
    for (int e = tid; e < CB_C * CB_C; e += 256) {
        const int r = e / CB_C, i = e % CB_C;
        if (i / 16 > r / 16) {
            sA[r][i] = 0.f;
            blk[Y::P + e] = 0.f;
            if (!FWD) blk[Y::GH + e] = 0.f;
        }
    }
    __syncthreads();
    // M = (I + A)^-1 by forward substitution,
    //     M[r][j] = [r == j] - sum_{i < r} A[r][i] M[i][j]
    // (M is lower triangular, so the terms i < j are zero by themselves).
    // One wave: lane j keeps column j of M in registers and reads the rows
    // of A as broadcasts; no barrier inside the recurrence.
    if (tid < CB_C) {
        float mc[CB_C];
#pragma unroll
        for (int r = 0; r < CB_C; ++r) {
            float s0 = 0.f, s1 = 0.f;
#pragma unroll
            for (int i = 0; i + 1 < r; i += 2) {
                s0 += sA[r][i] * mc[i];
                s1 += sA[r][i + 1] * mc[i + 1];
            }
            if (r & 1) s0 += sA[r][r - 1] * mc[r - 1];
            mc[r] = (r == tid ? 1.f : 0.f) - (s0 + s1);
        }
#pragma unroll
        for (int r = 0; r < CB_C; ++r) sA[r][tid] = mc[r];
    }
    if (FWD) {
        __syncthreads();
        // in fragment order, walking the destination (16-byte stores):
        // slot d4 of fragment (R, B) holds row 16R + lane % 16, columns
        // 16B + 4 (lane / 16) .. + 3
        for (int d4 = tid; d4 < CB_C * CB_C / 4; d4 += 256) {
            const int fr = d4 / 64, lane = d4 % 64;
            const int r = 16 * (fr / (CB_C / 16)) + lane % 16, c = 16 * (fr % (CB_C / 16)) + 4 * (lane / 16);
            const f32x4 mv = {sA[r][c], sA[r][c + 1], sA[r][c + 2], sA[r][c + 3]};
            *reinterpret_cast<f32x4 *>(blk + Y::M + 4 * d4) = mv;
        }
        return;
    }
    __syncthreads();
    for (int e = tid; e < CB_C * CB_C; e += 256) blk[Y::M + e] = sA[e / CB_C][e % CB_C];
    // W = T K~ = M Diag(beta) K~ on the fp32 matrix cores: 16 x 16 output
    // blocks (token block rb, key block cb) dealt round-robin to the four
    // waves, the contraction over the token blocks ib <= rb (M is lower
    // triangular).  In step s lane l (g = l / 16, n = l % 16) supplies
    // A[n][4g + s] = M[16rb + n][i] beta_i and B[4g + s][n] = K~[i][16cb + n]
    // with i = 16ib + 4g + s, and holds W[16rb + 4g + u][16cb + n].
    {
        constexpr int NKB = DK / 16;
        const int lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int g = lane >> 4, n = lane & 15;
        for (int b = wv; b < 4 * NKB; b += 4) {
            const int rb = b / NKB, cb = b % NKB;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int ib = 0; ib <= rb; ++ib)
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2) {
                    const int i = 16 * ib + 4 * g + s2;
                    const int c = 16 * cb + n;   // K~ = k e^G formed here
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(sA[16 * rb + n][i] * sb[i],
                                                               ldk(i, c) * ex(sG[i][c]), acc, 0, 0, 0);
                }
#pragma unroll
            for (int u = 0; u < 4; ++u) blk[Y::W + (16 * rb + 4 * g + u) * DK + 16 * cb + n] = acc[u];
        }
    }
}

}  // namespace kda
