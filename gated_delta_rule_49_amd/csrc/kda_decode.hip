// Fused KDA decode (Module 04 — KDA II, §2 "Why decode and prefill need
// different kernels": decode applies recurrent steps to a state already
// resident in memory), for m >= 1 consecutive tokens per sequence in one
// launch (multi-token decode / speculative verification: Module 11, §2, row
// "Serving state").
//
// Per (sequence b, head h) and token, with a = exp(log_alpha) and S the fp32
// state:
//     p = S^T (a * k),  r = S^T (a * q),  kappa = k . q
//     delta = beta (v - p)
//     o = r + kappa * delta               (= S_t^T q_t, post-update state)
//     S <- a * S + k delta^T              (= (I - beta k k^T) Diag(a) S + beta k v^T)
// With the q/k norm, k and q are 1/|k|, 1/|q| times the inputs: the sums
// over rows are taken on the inputs and scaled once.
// The state is HBM-bound: it is read once into registers, the m tokens are
// applied there, and it is written once (plus once per token when the
// per-token states are requested).  A workgroup of 512 threads works on one
// (b, h) state at a time: the column space of S is split across lanes in
// float4 groups (16-byte coalesced rows) and the row space across row
// groups; the d_k reductions run lane-to-lane inside a wave (__shfl_xor) and
// across waves through LDS.  Four kernels share this layout:
// decode1_kernel (one token, output state: persistent, prefetching each
// workgroup's next state), decodec_kernel (2 to 4 tokens without per-token
// states, applied as one small chunk: persistent likewise), decodem_kernel
// (m tokens with per-token states, m <= NT / max(d_k, d_v): persistent
// likewise) and decode_kernel (one workgroup per state: the remaining
// launches).
// The state is read and written with non-temporal accesses.  Measured on
// MI355X for B=256, H=32, d=128 (1.09 GB per step): 512 threads per state
// with non-temporal accesses 187 us per step; 256 threads 208 us (213 us
// with ordinary accesses); 1024 threads 221 us; splitting a state by columns
// over 4 workgroups of 256 threads 196 us; the persistent single-token
// kernel below (each workgroup prefetching its next state) 182 us.
#include "kda_launch.hpp"

namespace kda {

// threads per workgroup (at most)
constexpr int kDecodeThreads = 512;
// workgroups of the persistent single-token launch.  Measured for B=256,
// H=32, d=128 (148 VGPRs: one 512-thread workgroup resident per CU):
// 256 -> 187.7 us per step, 512 -> 182.6, 768 -> 185.9, 1024 -> 182.2,
// 2048 -> 186.1; one workgroup per state 187.7.
constexpr int kDecodeGrid = 512;

template <int DK, int DV>
struct DecodeShape {
    static constexpr int TPR = DV / 4;                      // threads per row
    static constexpr int RG = (DK < kDecodeThreads / TPR) ? DK : kDecodeThreads / TPR;  // row groups
    static constexpr int NT = TPR * RG;                     // threads
    static constexpr int RPT = DK / RG;                     // rows per thread
    static constexpr int NW = (NT + 63) / 64;               // waves
};

// Arguments of one launch: m consecutive tokens per sequence.
struct DecodeParams {
    const void *q, *k, *v, *beta, *log_alpha;  // [B, m, H, d] / [B, m, H]
    const float *state_in;                     // [B, H, DK, DV]
    float *state_out;                          // nullable; may alias state_in
    float *token_states;                       // nullable; [B, m, H, DK, DV]
    void *o;                                   // [B, m, H, DV]
    int H, m;
    uint32_t prologue;                         // kPro* bits
};

// MULTI = false: the single-token launch (m == 1, no per-token states), a
// straight-line kernel without the token loop.  MULTI = true stages the
// inputs of up to MG tokens at once, so that the token loop itself waits on
// no global load.
template <int DK, int DV, typename TI, typename TO, bool MULTI>
__global__ void __launch_bounds__((DecodeShape<DK, DV>::NT)) decode_kernel(DecodeParams p) {
    using Sh = DecodeShape<DK, DV>;
    constexpr int MG = MULTI ? 8 : 1;   // tokens staged per group
    const int bh = blockIdx.x;
    const int b = bh / p.H, h = bh % p.H;
    const int tid = threadIdx.x;
    const int c4 = tid % Sh::TPR;   // column group: columns 4*c4 .. 4*c4+3
    const int rg = tid / Sh::TPR;   // row group: rows rg + RG*i
    const int wave = tid / 64;
    const int lane = tid % 64;
    const TI *q = static_cast<const TI *>(p.q);
    const TI *k = static_cast<const TI *>(p.k);
    const TI *v = static_cast<const TI *>(p.v);
    const TI *beta = static_cast<const TI *>(p.beta);
    const TI *la = static_cast<const TI *>(p.log_alpha);
    TO *o = static_cast<TO *>(p.o);

    __shared__ float s_a[MG][DK], s_k[MG][DK], s_q[MG][DK], s_ak[MG][DK], s_aq[MG][DK];
    __shared__ float s_v[MG][DV], s_b[MG];
    __shared__ float s_kappa[MG], s_nk[MG], s_nq[MG];
    // wave partials of p and r, double-buffered over tokens so that one
    // barrier per token suffices
    __shared__ float s_red[MULTI ? 2 : 1][2][Sh::NW][DV];

    // this thread's rows of S (float4 each), held in registers for all m
    // tokens; element (row, 4 c4) of the (b, h) state
    const int64_t soff = static_cast<int64_t>(bh) * DK * DV + 4 * c4;
    auto at = [&](int i) { return static_cast<int64_t>(rg + Sh::RG * i) * DV; };
    f32x4 sv[Sh::RPT];
#pragma unroll
    for (int i = 0; i < Sh::RPT; ++i)
        sv[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p.state_in + soff + at(i)));

    const int m = MULTI ? p.m : 1;
    int par = 0;
    for (int t0 = 0; t0 < m; t0 += MG) {
        const int nt = MULTI ? min(MG, m - t0) : 1;
        const int64_t tok0 = (static_cast<int64_t>(b) * m + t0) * p.H + h;  // row of [B, m, H]
        if (t0 > 0) __syncthreads();  // the previous group's readers of s_* are done
        // stage the group's token vectors
        for (int idx = tid; idx < nt * DK; idx += Sh::NT) {
            const int t = idx / DK, i = idx % DK;
            const int64_t off = (tok0 + static_cast<int64_t>(t) * p.H) * DK + i;
            const float x = io<TI>::ld(la, off);
            // alpha = exp(log alpha); with the gate prologue exp(-softplus(x)) = 1 / (1 + e^x)
            const float a = (p.prologue & kProGate) ? sigmoid_f32(-x) : __expf(x);
            const float kk = io<TI>::ld(k, off);
            const float qq = io<TI>::ld(q, off);
            s_a[t][i] = a;
            s_k[t][i] = kk;
            s_q[t][i] = qq;
            s_ak[t][i] = a * kk;
            s_aq[t][i] = a * qq;
        }
        for (int idx = tid; idx < nt * DV; idx += Sh::NT) {
            const int t = idx / DV, j = idx % DV;
            s_v[t][j] = io<TI>::ld(v, (tok0 + static_cast<int64_t>(t) * p.H) * DV + j);
        }
        if (tid < nt) {
            float bt = io<TI>::ld(beta, tok0 + static_cast<int64_t>(tid) * p.H);
            if (p.prologue & kProBeta) bt = sigmoid_f32(bt);
            s_b[tid] = bt;
        }
        __syncthreads();
        // kappa = k.q and, with the norm, 1/|k| and 1/|q|: one wave per token
        for (int t = wave; t < nt; t += Sh::NW) {
            float kq = 0.f, k2 = 0.f, q2 = 0.f;
            for (int i = lane; i < DK; i += 64) {
                const float kk = s_k[t][i], qq = s_q[t][i];
                kq += kk * qq;
                k2 += kk * kk;
                q2 += qq * qq;
            }
#pragma unroll
            for (int msk = 32; msk >= 1; msk >>= 1) {
                kq += __shfl_xor(kq, msk);
                k2 += __shfl_xor(k2, msk);
                q2 += __shfl_xor(q2, msk);
            }
            if (lane == 0) {
                float nk = 1.f, nq = 1.f;
                if (p.prologue & kProQKNorm) {
                    nk = 1.f / __builtin_sqrtf(k2 + kQKNormEps);
                    nq = 1.f / __builtin_sqrtf(q2 + kQKNormEps);
                }
                s_nk[t] = nk;
                s_nq[t] = nq;
                s_kappa[t] = kq * nk * nq;
            }
        }
        __syncthreads();

        for (int t = 0; t < nt; ++t, par ^= MULTI ? 1 : 0) {
            const int64_t tok = tok0 + static_cast<int64_t>(t) * p.H;
            // partial p = S^T (a k), r = S^T (a q) over this thread's rows
            f32x4 pr = {0.f, 0.f, 0.f, 0.f}, rr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < Sh::RPT; ++i) {
                const int row = rg + Sh::RG * i;
                pr += sv[i] * s_ak[t][row];
                rr += sv[i] * s_aq[t][row];
            }
            // reduce across the row groups inside the wave (lane bits >= log2(TPR))
#pragma unroll
            for (int msk = Sh::TPR; msk < 64 && msk < Sh::NT; msk <<= 1) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    pr[j] += __shfl_xor(pr[j], msk);
                    rr[j] += __shfl_xor(rr[j], msk);
                }
            }
            if (lane < Sh::TPR) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    s_red[par][0][wave][4 * c4 + j] = pr[j];
                    s_red[par][1][wave][4 * c4 + j] = rr[j];
                }
            }
            __syncthreads();
            // every thread needs delta for its 4 columns: sum the wave partials
            f32x4 pt = {0.f, 0.f, 0.f, 0.f}, rt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int w = 0; w < Sh::NW; ++w) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    pt[j] += s_red[par][0][w][4 * c4 + j];
                    rt[j] += s_red[par][1][w][4 * c4 + j];
                }
            }
            const float nk = s_nk[t], nq = s_nq[t], bt = s_b[t];
            f32x4 delta;
#pragma unroll
            for (int j = 0; j < 4; ++j) delta[j] = bt * (s_v[t][4 * c4 + j] - pt[j] * nk);
            if (rg == 0) {
                const float kappa = s_kappa[t];
                const int64_t ooff = tok * DV + 4 * c4;
#pragma unroll
                for (int j = 0; j < 4; ++j) io<TO>::st(o, ooff + j, rt[j] * nq + kappa * delta[j]);
            }
#pragma unroll
            for (int i = 0; i < Sh::RPT; ++i) {
                const int row = rg + Sh::RG * i;
                const float a = s_a[t][row], kk = s_k[t][row] * nk;
                sv[i] = a * sv[i] + kk * delta;
            }
            if (MULTI && p.token_states) {
                float *ts = p.token_states + tok * DK * DV + 4 * c4;
#pragma unroll
                for (int i = 0; i < Sh::RPT; ++i)
                    __builtin_nontemporal_store(sv[i], reinterpret_cast<f32x4 *>(ts + at(i)));
            }
        }
    }
    if (p.state_out) {
#pragma unroll
        for (int i = 0; i < Sh::RPT; ++i)
            __builtin_nontemporal_store(sv[i], reinterpret_cast<f32x4 *>(p.state_out + soff + at(i)));
    }
}


// Single-token launch, persistent: workgroup w updates the states w, w + G,
// w + 2G, ... (G = gridDim.x) and requests the next state and its token
// vectors before it updates the current one, so that one state's transfer
// from HBM overlaps the previous state's update and write-back.  The token
// vectors are staged in one of two LDS buffers by state parity and every
// wave forms kappa and the norms itself: two LDS-only barriers per state.
template <typename TI>
struct DecodeTok {  // one thread's share of a token's vectors (raw, converted at use)
    TI a, k, q, v, b;
};

template <int DK, int DV, typename TI>
__device__ __forceinline__ void decode1_request(const DecodeParams &p, int bh, int tid,
                                                f32x4 (&sv)[DecodeShape<DK, DV>::RPT], DecodeTok<TI> &in) {
    using Sh = DecodeShape<DK, DV>;
    const int c4 = tid % Sh::TPR, rg = tid / Sh::TPR;
    // uniform base, 32-bit per-lane offsets (shared by all states of the walk)
    const float *src = p.state_in + static_cast<int64_t>(bh) * DK * DV;
    const uint32_t lo = static_cast<uint32_t>(rg * DV + 4 * c4);
#pragma unroll
    for (int i = 0; i < Sh::RPT; ++i)
        sv[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(src + (lo + static_cast<uint32_t>(Sh::RG * i * DV))));
    if (tid < DK) {
        const int64_t off = static_cast<int64_t>(bh) * DK + tid;
        in.a = static_cast<const TI *>(p.log_alpha)[off];
        in.k = static_cast<const TI *>(p.k)[off];
        in.q = static_cast<const TI *>(p.q)[off];
    }
    if (tid < DV) in.v = static_cast<const TI *>(p.v)[static_cast<int64_t>(bh) * DV + tid];
    if (tid == 0) in.b = static_cast<const TI *>(p.beta)[bh];
}

template <int DK, int DV, typename TI, typename TO, int PAR>
__device__ __forceinline__ void decode1_update(const DecodeParams &p, int bh, int tid,
                                               f32x4 (&sv)[DecodeShape<DK, DV>::RPT], const DecodeTok<TI> &in,
                                               float (&s_a)[2][DK], float (&s_k)[2][DK], float (&s_q)[2][DK],
                                               float (&s_v)[2][DV], float (&s_b)[2],
                                               float (&s_red)[2][DecodeShape<DK, DV>::NW][DV]) {
    using Sh = DecodeShape<DK, DV>;
    const int c4 = tid % Sh::TPR, rg = tid / Sh::TPR, wave = tid / 64, lane = tid % 64;
    if (tid < DK) {
        const float x = io<TI>::ld(&in.a, 0);
        s_a[PAR][tid] = (p.prologue & kProGate) ? sigmoid_f32(-x) : __expf(x);
        s_k[PAR][tid] = io<TI>::ld(&in.k, 0);
        s_q[PAR][tid] = io<TI>::ld(&in.q, 0);
    }
    if (tid < DV) s_v[PAR][tid] = io<TI>::ld(&in.v, 0);
    if (tid == 0) {
        float bt = io<TI>::ld(&in.b, 0);
        if (p.prologue & kProBeta) bt = sigmoid_f32(bt);
        s_b[PAR] = bt;
    }
    lds_barrier();
    // kappa = k.q and, with the norm, 1/|k| and 1/|q|, formed by every wave
    float kq = 0.f, k2 = 0.f, q2 = 0.f;
    for (int i = lane; i < DK; i += 64) {
        const float kk = s_k[PAR][i], qq = s_q[PAR][i];
        kq += kk * qq;
        k2 += kk * kk;
        q2 += qq * qq;
    }
#pragma unroll
    for (int msk = 32; msk >= 1; msk >>= 1) {
        kq += __shfl_xor(kq, msk);
        k2 += __shfl_xor(k2, msk);
        q2 += __shfl_xor(q2, msk);
    }
    float nk = 1.f, nq = 1.f;
    if (p.prologue & kProQKNorm) {
        nk = 1.f / __builtin_sqrtf(k2 + kQKNormEps);
        nq = 1.f / __builtin_sqrtf(q2 + kQKNormEps);
    }
    const float kappa = kq * nk * nq;
    // partial p = S^T (a k), r = S^T (a q) over this thread's rows
    f32x4 pr = {0.f, 0.f, 0.f, 0.f}, rr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < Sh::RPT; ++i) {
        const int row = rg + Sh::RG * i;
        const float a = s_a[PAR][row];
        pr += sv[i] * (a * s_k[PAR][row]);
        rr += sv[i] * (a * s_q[PAR][row]);
    }
#pragma unroll
    for (int msk = Sh::TPR; msk < 64 && msk < Sh::NT; msk <<= 1) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            pr[j] += __shfl_xor(pr[j], msk);
            rr[j] += __shfl_xor(rr[j], msk);
        }
    }
    if (lane < Sh::TPR) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            s_red[0][wave][4 * c4 + j] = pr[j];
            s_red[1][wave][4 * c4 + j] = rr[j];
        }
    }
    lds_barrier();
    f32x4 pt = {0.f, 0.f, 0.f, 0.f}, rt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < Sh::NW; ++w) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            pt[j] += s_red[0][w][4 * c4 + j];
            rt[j] += s_red[1][w][4 * c4 + j];
        }
    }
    const float bt = s_b[PAR];
    f32x4 delta;
#pragma unroll
    for (int j = 0; j < 4; ++j) delta[j] = bt * (s_v[PAR][4 * c4 + j] - pt[j] * nk);
    if (rg == 0) {
        TO *o = static_cast<TO *>(p.o);
        const int64_t ooff = static_cast<int64_t>(bh) * DV + 4 * c4;
#pragma unroll
        for (int j = 0; j < 4; ++j) io<TO>::st(o, ooff + j, rt[j] * nq + kappa * delta[j]);
    }
    float *dst = p.state_out + static_cast<int64_t>(bh) * DK * DV;
    const uint32_t lo = static_cast<uint32_t>(rg * DV + 4 * c4);
#pragma unroll
    for (int i = 0; i < Sh::RPT; ++i) {
        const int row = rg + Sh::RG * i;
        const float a = s_a[PAR][row], kk = s_k[PAR][row] * nk;
        __builtin_nontemporal_store(a * sv[i] + kk * delta,
                                    reinterpret_cast<f32x4 *>(dst + (lo + static_cast<uint32_t>(Sh::RG * i * DV))));
    }
}

template <int DK, int DV, typename TI, typename TO>
__global__ void __launch_bounds__((DecodeShape<DK, DV>::NT)) decode1_kernel(DecodeParams p, int BH) {
    using Sh = DecodeShape<DK, DV>;
    __shared__ float s_a[2][DK], s_k[2][DK], s_q[2][DK], s_v[2][DV], s_b[2];
    __shared__ float s_red[2][Sh::NW][DV];
    const int tid = threadIdx.x, G = gridDim.x;
    f32x4 svA[Sh::RPT], svB[Sh::RPT];
    DecodeTok<TI> inA{}, inB{};
    int bh = blockIdx.x;   // uniform: every wave takes the same branches
    if (bh >= BH) return;
    decode1_request<DK, DV, TI>(p, bh, tid, svA, inA);
    for (;;) {
        const int bh1 = bh + G;
        if (bh1 < BH) decode1_request<DK, DV, TI>(p, bh1, tid, svB, inB);
        decode1_update<DK, DV, TI, TO, 0>(p, bh, tid, svA, inA, s_a, s_k, s_q, s_v, s_b, s_red);
        if (bh1 >= BH) break;
        const int bh2 = bh1 + G;
        if (bh2 < BH) decode1_request<DK, DV, TI>(p, bh2, tid, svA, inA);
        decode1_update<DK, DV, TI, TO, 1>(p, bh1, tid, svB, inB, s_a, s_k, s_q, s_v, s_b, s_red);
        if (bh2 >= BH) break;
        bh = bh2;
    }
}


// Multi-token launch with the state after every token (speculative
// verification with rollback), m <= NT / max(DK, DV) tokens (4 at d = 128),
// persistent like decode1_kernel: the next state and the raw token vectors
// of its m tokens (one element per thread and vector) are requested before
// the current state's m tokens are applied.  Per state: one barrier after
// staging; wave t mod NW forms token t's k.q and norms, published by the
// barrier of token 0's partials; one barrier per token (partials
// double-buffered by token parity).  Measured for B=256, m=4, H=32, d=128
// (145 VGPRs: one workgroup resident per CU): 595 us per launch against
// 649 us for decode_kernel<..., true>; without the per-token states it is
// slower (387 against 254 us: with one resident workgroup the m token
// updates of successive states no longer overlap), so that case stays on
// decode_kernel.
template <int DK, int DV>
struct DecodeMShape {
    using Sh = DecodeShape<DK, DV>;
    static constexpr int MT = Sh::NT / (DK > DV ? DK : DV);   // tokens per state at most
};

template <int DK, int DV, typename TI>
__device__ __forceinline__ void decodem_request(const DecodeParams &p, int bh, int tid,
                                                f32x4 (&sv)[DecodeShape<DK, DV>::RPT], DecodeTok<TI> &in) {
    using Sh = DecodeShape<DK, DV>;
    const int c4 = tid % Sh::TPR, rg = tid / Sh::TPR;
    const float *src = p.state_in + static_cast<int64_t>(bh) * DK * DV;
    const uint32_t lo = static_cast<uint32_t>(rg * DV + 4 * c4);
#pragma unroll
    for (int i = 0; i < Sh::RPT; ++i)
        sv[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(src + (lo + static_cast<uint32_t>(Sh::RG * i * DV))));
    const int b = bh / p.H, h = bh % p.H;
    const int64_t tok0 = static_cast<int64_t>(b) * p.m * p.H + h;   // row of [B, m, H] of token 0
    if (tid < p.m * DK) {
        const int t = tid / DK, i = tid % DK;
        const int64_t off = (tok0 + static_cast<int64_t>(t) * p.H) * DK + i;
        in.a = static_cast<const TI *>(p.log_alpha)[off];
        in.k = static_cast<const TI *>(p.k)[off];
        in.q = static_cast<const TI *>(p.q)[off];
    }
    if (tid < p.m * DV) {
        const int t = tid / DV, j = tid % DV;
        in.v = static_cast<const TI *>(p.v)[(tok0 + static_cast<int64_t>(t) * p.H) * DV + j];
    }
    if (tid < p.m) in.b = static_cast<const TI *>(p.beta)[tok0 + static_cast<int64_t>(tid) * p.H];
}

template <int DK, int DV>
struct DecodeMShared {
    using Sh = DecodeShape<DK, DV>;
    static constexpr int MT = DecodeMShape<DK, DV>::MT;
    float a[2][MT][DK], k[2][MT][DK], q[2][MT][DK], v[2][MT][DV], b[2][MT];
    float kappa[MT], nk[MT], nq[MT];
    float red[2][2][Sh::NW][DV];
};

template <int DK, int DV, typename TI, typename TO, int PAR>
__device__ __forceinline__ void decodem_update(const DecodeParams &p, int bh, int tid,
                                               f32x4 (&sv)[DecodeShape<DK, DV>::RPT], const DecodeTok<TI> &in,
                                               DecodeMShared<DK, DV> &sm, int &par) {
    using Sh = DecodeShape<DK, DV>;
    const int c4 = tid % Sh::TPR, rg = tid / Sh::TPR, wave = tid / 64, lane = tid % 64;
    const int m = p.m;
    if (tid < m * DK) {
        const int t = tid / DK, i = tid % DK;
        const float x = io<TI>::ld(&in.a, 0);
        sm.a[PAR][t][i] = (p.prologue & kProGate) ? sigmoid_f32(-x) : __expf(x);
        sm.k[PAR][t][i] = io<TI>::ld(&in.k, 0);
        sm.q[PAR][t][i] = io<TI>::ld(&in.q, 0);
    }
    if (tid < m * DV) sm.v[PAR][tid / DV][tid % DV] = io<TI>::ld(&in.v, 0);
    if (tid < m) {
        float bt = io<TI>::ld(&in.b, 0);
        if (p.prologue & kProBeta) bt = sigmoid_f32(bt);
        sm.b[PAR][tid] = bt;
    }
    lds_barrier();
    // token t's kappa = k.q and, with the norm, 1/|k| and 1/|q|, on wave
    // t mod NW; read after the barrier of token 0's partials
    for (int t = wave; t < m; t += Sh::NW) {
        float kq = 0.f, k2 = 0.f, q2 = 0.f;
        for (int i = lane; i < DK; i += 64) {
            const float kk = sm.k[PAR][t][i], qq = sm.q[PAR][t][i];
            kq += kk * qq;
            k2 += kk * kk;
            q2 += qq * qq;
        }
#pragma unroll
        for (int msk = 32; msk >= 1; msk >>= 1) {
            kq += __shfl_xor(kq, msk);
            k2 += __shfl_xor(k2, msk);
            q2 += __shfl_xor(q2, msk);
        }
        if (lane == 0) {
            float nk = 1.f, nq = 1.f;
            if (p.prologue & kProQKNorm) {
                nk = 1.f / __builtin_sqrtf(k2 + kQKNormEps);
                nq = 1.f / __builtin_sqrtf(q2 + kQKNormEps);
            }
            sm.nk[t] = nk;
            sm.nq[t] = nq;
            sm.kappa[t] = kq * nk * nq;
        }
    }
    const int b = bh / p.H, h = bh % p.H;
    const int64_t tok0 = static_cast<int64_t>(b) * m * p.H + h;
    const uint32_t lo = static_cast<uint32_t>(rg * DV + 4 * c4);
    for (int t = 0; t < m; ++t, par ^= 1) {
        const int64_t tok = tok0 + static_cast<int64_t>(t) * p.H;
        f32x4 pr = {0.f, 0.f, 0.f, 0.f}, rr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < Sh::RPT; ++i) {
            const int row = rg + Sh::RG * i;
            const float a = sm.a[PAR][t][row];
            pr += sv[i] * (a * sm.k[PAR][t][row]);
            rr += sv[i] * (a * sm.q[PAR][t][row]);
        }
#pragma unroll
        for (int msk = Sh::TPR; msk < 64 && msk < Sh::NT; msk <<= 1) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                pr[j] += __shfl_xor(pr[j], msk);
                rr[j] += __shfl_xor(rr[j], msk);
            }
        }
        if (lane < Sh::TPR) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                sm.red[par][0][wave][4 * c4 + j] = pr[j];
                sm.red[par][1][wave][4 * c4 + j] = rr[j];
            }
        }
        lds_barrier();
        f32x4 pt = {0.f, 0.f, 0.f, 0.f}, rt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < Sh::NW; ++w) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                pt[j] += sm.red[par][0][w][4 * c4 + j];
                rt[j] += sm.red[par][1][w][4 * c4 + j];
            }
        }
        const float nk = sm.nk[t], nq = sm.nq[t], bt = sm.b[PAR][t];
        f32x4 delta;
#pragma unroll
        for (int j = 0; j < 4; ++j) delta[j] = bt * (sm.v[PAR][t][4 * c4 + j] - pt[j] * nk);
        if (rg == 0) {
            TO *o = static_cast<TO *>(p.o);
            const float kappa = sm.kappa[t];
            const int64_t ooff = tok * DV + 4 * c4;
#pragma unroll
            for (int j = 0; j < 4; ++j) io<TO>::st(o, ooff + j, rt[j] * nq + kappa * delta[j]);
        }
#pragma unroll
        for (int i = 0; i < Sh::RPT; ++i) {
            const int row = rg + Sh::RG * i;
            const float a = sm.a[PAR][t][row], kk = sm.k[PAR][t][row] * nk;
            sv[i] = a * sv[i] + kk * delta;
        }
        if (p.token_states) {
            float *ts = p.token_states + tok * DK * DV;
#pragma unroll
            for (int i = 0; i < Sh::RPT; ++i)
                __builtin_nontemporal_store(sv[i], reinterpret_cast<f32x4 *>(ts + (lo + static_cast<uint32_t>(Sh::RG * i * DV))));
        }
    }
    if (p.state_out) {
        float *dst = p.state_out + static_cast<int64_t>(bh) * DK * DV;
#pragma unroll
        for (int i = 0; i < Sh::RPT; ++i)
            __builtin_nontemporal_store(sv[i], reinterpret_cast<f32x4 *>(dst + (lo + static_cast<uint32_t>(Sh::RG * i * DV))));
    }
}

template <int DK, int DV, typename TI, typename TO>
__global__ void __launch_bounds__((DecodeShape<DK, DV>::NT)) decodem_kernel(DecodeParams p, int BH) {
    using Sh = DecodeShape<DK, DV>;
    __shared__ DecodeMShared<DK, DV> sm;
    const int tid = threadIdx.x, G = gridDim.x;
    f32x4 svA[Sh::RPT], svB[Sh::RPT];
    DecodeTok<TI> inA{}, inB{};
    int par = 0;
    int bh = blockIdx.x;   // uniform: every wave takes the same branches
    if (bh >= BH) return;
    decodem_request<DK, DV, TI>(p, bh, tid, svA, inA);
    for (;;) {
        const int bh1 = bh + G;
        if (bh1 < BH) decodem_request<DK, DV, TI>(p, bh1, tid, svB, inB);
        decodem_update<DK, DV, TI, TO, 0>(p, bh, tid, svA, inA, sm, par);
        if (bh1 >= BH) break;
        const int bh2 = bh1 + G;
        if (bh2 < BH) decodem_request<DK, DV, TI>(p, bh2, tid, svA, inA);
        decodem_update<DK, DV, TI, TO, 1>(p, bh1, tid, svB, inB, sm, par);
        if (bh2 >= BH) break;
        bh = bh2;
    }
}


// Multi-token launch as one small chunk, 2 <= m <= 4 tokens, persistent
// like decode1_kernel.  The chunked form of the recurrence (Module 04 —
// KDA II, §1 "The recurrence has affine form") restricted to the m tokens
// gives every token's delta vector from the state S0 they start from:
//     X_t = v_t - S0^T (khat_t * Gamma_t),   Gamma_t = a_0 * ... * a_t
//     (I + A) Delta = Diag(beta) X,   A_ti = beta_t sum_c khat_t khat_i a_{i+1}..a_t  (i < t)
//     o_t = S0^T (qhat_t * Gamma_t) + sum_{i<=t} P_ti Delta_i,
//           P_ti = sum_c qhat_t khat_i a_{i+1}..a_t  (i <= t)
// (khat, qhat: k and q with the optional norm; the decay products are
// taken per channel), and then
//     S_m = Gamma_{m-1} * S0 + sum_t (khat_t * a_{t+1}..a_{m-1}) Delta_t^T,
// or, when the state after every token is asked for, token by token
// S_{t+1} = a_t * S_t + khat_t Delta_t^T.
// Roles: threads [0, DV) own a column each (they solve for Delta and form
// the outputs once per column), threads [DV, DV + DK) own a row each (they
// turn a state's tokens into per-row factors and per-channel terms of the
// m^2 + m pair sums kk_ti, qk_ti, |k_t|^2, |q_t|^2).  The row work depends
// on the tokens only, so it is done one state ahead, while the column
// owners work: per state there is one pass of 2m reductions over the rows
// of S0, a barrier, the column work beside the next state's row work, a
// barrier, and the update of the state.  Measured for B=256, H=32, d=128
// (state only, 512 workgroups, one resident per CU): m = 2 in 188 us and
// m = 4 in 209 us per launch, against 216 and 251 us token by token on
// decode_kernel; 256 workgroups gave 193 and 205 us, 1024 gave 191 and
// 219 us.  With per-token states decodem_kernel stays faster (590 against
// 682 us at m = 4: the token-by-token sweep writes every state anyway).
template <int M>
struct DecodeCJobs {
    static constexpr int NKK = M * (M - 1) / 2, NQK = M * (M + 1) / 2, N = NKK + NQK + 2 * M;
    static constexpr int kk(int t, int i) { return t * (t - 1) / 2 + i; }         // i < t
    static constexpr int qk(int t, int i) { return NKK + t * (t + 1) / 2 + i; }   // i <= t
    static constexpr int k2(int t) { return NKK + NQK + t; }
    static constexpr int q2(int t) { return NKK + NQK + M + t; }
};

template <int DK, int DV>
struct DecodeCRoles {
    static constexpr int W0 = DV / 64, W1 = (DV + DK - 1) / 64;   // waves holding row owners
    static constexpr int NPART = W1 - W0 + 1;                      // partial pair sums per job
};

template <int DK, int DV, int M>
struct DecodeCShared {
    using Sh = DecodeShape<DK, DV>;
    // first: 16-byte aligned; DK and DV are multiples of 4
    float red[2][M][Sh::NW][DV];   // wave partials of S0^T Ktil_t (0) and S0^T Qtil_t (1)
    // by state parity: per-row factors of each token
    float kt[2][M][DK];    // k_t Gamma_t
    float qt[2][M][DK];    // q_t Gamma_t
    float kh[2][M][DK];    // k_t a_{t+1} .. a_{m-1}
    float a[2][M][DK], k[2][M][DK];
    float gm[2][DK];       // Gamma_{m-1}
    float pj[2][DecodeCJobs<M>::N][DecodeCRoles<DK, DV>::NPART];   // partial pair sums
    float dl[M][DV];       // nk_t Delta_t
};

// one thread's token values: a row owner's a_t, k_t, q_t of its row, a
// column owner's v_t and beta_t of its column (raw, converted at use)
template <int M, typename TI>
struct DecodeCTok {
    TI r[3 * M];
};

// thread (rg, c4) holds the RPT consecutive rows rg * RPT .. rg * RPT + RPT - 1
// of the state, so that its rows' factors are contiguous in LDS; each load
// instruction still covers whole 512-byte rows of the state.  bh_col names
// the state whose v and beta the column owners take, bh_row the state whose
// a, k, q the row owners take.  Every load is unconditional (indices
// clamped) so that the wait counts leave the request in flight.
template <int DK, int DV>
__device__ __forceinline__ void decodec_request_state(const DecodeParams &p, int bh, int tid,
                                                      f32x4 (&sv)[DecodeShape<DK, DV>::RPT]) {
    using Sh = DecodeShape<DK, DV>;
    const int c4 = tid % Sh::TPR, rg = tid / Sh::TPR;
    const float *src = p.state_in + static_cast<int64_t>(bh) * DK * DV;
    const uint32_t lo = static_cast<uint32_t>(rg * Sh::RPT * DV + 4 * c4);
#pragma unroll
    for (int i = 0; i < Sh::RPT; ++i)
        sv[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(src + (lo + static_cast<uint32_t>(i * DV))));
}
template <int DK, int DV, int M, typename TI>
__device__ __forceinline__ void decodec_request_tokens(const DecodeParams &p, int bh_col, int bh_row, int tid,
                                                       DecodeCTok<M, TI> &in) {
    // rows [B, m, H] of token 0 of the two states
    const int64_t tc = static_cast<int64_t>(bh_col / p.H) * M * p.H + bh_col % p.H;
    const int64_t tr = static_cast<int64_t>(bh_row / p.H) * M * p.H + bh_row % p.H;
    const bool col = tid < DV;
    const int j = col ? tid : 0;
    const int c = col ? 0 : (tid - DV < DK ? tid - DV : DK - 1);
    const TI *v = static_cast<const TI *>(p.v), *be = static_cast<const TI *>(p.beta);
    const TI *la = static_cast<const TI *>(p.log_alpha), *k = static_cast<const TI *>(p.k), *q = static_cast<const TI *>(p.q);
#pragma unroll
    for (int t = 0; t < M; ++t) {
        const int64_t rc = tc + static_cast<int64_t>(t) * p.H, rr = tr + static_cast<int64_t>(t) * p.H;
        in.r[t] = col ? v[rc * DV + j] : la[rr * DK + c];
        in.r[M + t] = col ? be[rc] : k[rr * DK + c];
        in.r[2 * M + t] = col ? be[rc] : q[rr * DK + c];
    }
}
template <int DK, int DV, int M, typename TI>
__device__ __forceinline__ void decodec_request(const DecodeParams &p, int bh, int bh_col, int bh_row, int tid,
                                                f32x4 (&sv)[DecodeShape<DK, DV>::RPT], DecodeCTok<M, TI> &in) {
    decodec_request_state<DK, DV>(p, bh, tid, sv);
    decodec_request_tokens<DK, DV, M, TI>(p, bh_col, bh_row, tid, in);
}

// this thread's RPT consecutive entries of a per-row LDS vector
template <int RPT>
__device__ __forceinline__ void lds_rows(const float *src, float (&dst)[RPT]) {
    if constexpr (RPT % 4 == 0) {
#pragma unroll
        for (int i = 0; i < RPT; i += 4) {
            const float4 x = *reinterpret_cast<const float4 *>(src + i);
            dst[i] = x.x; dst[i + 1] = x.y; dst[i + 2] = x.z; dst[i + 3] = x.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < RPT; ++i) dst[i] = src[i];
    }
}

// x[l] + x[l ^ 32] in every lane: one swap of the wave's halves (VALU, no LDS)
__device__ __forceinline__ float sum_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// x of the lane named by a DPP control within its row of 16 (quad permutes
// and row mirrors only, so every lane has a source)
template <int CTRL>
__device__ __forceinline__ float dpp_row(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
// the sum over the row groups of a wave (lanes that hold the same columns)
template <int TPR>
__device__ __forceinline__ float rowgroup_sum(float x) {
#pragma unroll
    for (int msk = TPR; msk < 32; msk <<= 1) x += __shfl_xor(x, msk);
    return TPR < 64 ? sum_halves(x) : x;
}

// Sums over the 64 lanes of N values at once (N a power of two, 4 <= N <= 32):
// a reduce-scatter butterfly.  Each step pairs every lane with a lane whose
// bit b differs; the lane with bit b clear keeps the lower half of its
// values, the other the upper half, and each adds its partner's copy of the
// half it keeps, so the values per lane halve.  Bits 5 and 4 pair lanes
// with the half and row swaps (v_permlane32_swap, v_permlane16_swap), bits
// 3, 2, 1 with DPP within rows of 16 (rotate by 8, half-row mirror, quad
// permute); bits left after the values run out are summed plainly.  Lane l
// ends with the total of value l >> (6 - log2 N) in x[0].
// (both halves are summed with the partner and the kept one selected after
// the sums, so that no array element is chosen by a run-time index)
template <int CTRL, int N>
__device__ __forceinline__ void bfly_dpp(float (&x)[N], int n, bool hi) {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
        if (i < n / 2) {
            const float lo = x[i] + dpp_row<CTRL>(x[i]);
            const float up = x[i + n / 2] + dpp_row<CTRL>(x[i + n / 2]);
            x[i] = hi ? up : lo;
        }
    }
}
template <int N>
__device__ __forceinline__ void wave_reduce_scatter(float (&x)[N], int lane) {
    static_assert(N >= 4 && N <= 32 && (N & (N - 1)) == 0, "4, 8, 16 or 32 values");
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {      // bit 5
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[i]), __float_as_uint(x[i + N / 2]), false, false);
        x[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {      // bit 4
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x[i]), __float_as_uint(x[i + N / 4]), false, false);
        x[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    constexpr int n3 = N / 4, n2 = N / 8, n1 = N / 16;   // values entering the bit 3, 2, 1 steps
    if constexpr (n3 >= 2) bfly_dpp<0x128, N>(x, n3, (lane >> 3) & 1);   // row_ror:8
    else x[0] += dpp_row<0x128>(x[0]);
    if constexpr (n2 >= 2) bfly_dpp<0x141, N>(x, n2, (lane >> 2) & 1);   // row_half_mirror
    else x[0] += dpp_row<0x141>(x[0]);
    if constexpr (n1 >= 2) bfly_dpp<0x4E, N>(x, n1, (lane >> 1) & 1);    // quad_perm [2, 3, 0, 1]
    else x[0] += dpp_row<0x4E>(x[0]);
    x[0] += dpp_row<0xB1>(x[0]);                                        // quad_perm [1, 0, 3, 2]
}

// the row owners' work for one state's tokens, into buffer P: per-row
// factors, and per wave the partial pair sums over its row owners' channels
template <int DK, int DV, typename TI, int M, int P>
__device__ __forceinline__ void decodec_stage(const DecodeParams &p, int tid, const DecodeCTok<M, TI> &in,
                                              DecodeCShared<DK, DV, M> &sm) {
    using R = DecodeCRoles<DK, DV>;
    using J = DecodeCJobs<M>;
    const int wave = tid / 64, lane = tid % 64;
    if (wave < R::W0 || wave > R::W1) return;   // uniform: no row owner in this wave
    const int c = tid - DV;
    const bool row = c >= 0 && c < DK;
    float av[M], kv[M], qv[M];
#pragma unroll
    for (int t = 0; t < M; ++t) {
        // lanes that own no row (column owners in small head shapes hold v
        // here) take a = 1 and k = q = 0: their terms are exactly zero
        const float x = io<TI>::ld(&in.r[t], 0);
        av[t] = !row ? 1.f : (p.prologue & kProGate) ? sigmoid_f32(-x) : __expf(x);
        kv[t] = row ? io<TI>::ld(&in.r[M + t], 0) : 0.f;
        qv[t] = row ? io<TI>::ld(&in.r[2 * M + t], 0) : 0.f;
    }
    if (row) {
        float g = 1.f;
#pragma unroll
        for (int t = 0; t < M; ++t) {
            g *= av[t];
            sm.a[P][t][c] = av[t];
            sm.k[P][t][c] = kv[t];
            sm.kt[P][t][c] = kv[t] * g;
            sm.qt[P][t][c] = qv[t] * g;
        }
        sm.gm[P][c] = g;
        float suf = 1.f;
#pragma unroll
        for (int t = M - 1; t >= 0; --t) {
            sm.kh[P][t][c] = kv[t] * suf;
            suf *= av[t];
        }
    }
    // this channel's terms of the pair sums (zero outside the row owners),
    // padded with zeros to a power of two
    constexpr int NP = J::N <= 4 ? 4 : J::N <= 8 ? 8 : J::N <= 16 ? 16 : 32;
    float term[NP];
#pragma unroll
    for (int jb = J::N; jb < NP; ++jb) term[jb] = 0.f;
#pragma unroll
    for (int i = 0; i < M; ++i) {
        float w = 1.f;
#pragma unroll
        for (int t = i; t < M; ++t) {
            if (t > i) {
                w *= av[t];
                term[J::kk(t, i)] = kv[t] * kv[i] * w;
            }
            term[J::qk(t, i)] = qv[t] * kv[i] * w;
        }
    }
#pragma unroll
    for (int t = 0; t < M; ++t) {
        term[J::k2(t)] = kv[t] * kv[t];
        term[J::q2(t)] = qv[t] * qv[t];
    }
    wave_reduce_scatter<NP>(term, lane);
    constexpr int SH = NP == 4 ? 4 : NP == 8 ? 3 : NP == 16 ? 2 : 1;   // 6 - log2 NP
    const int jb = lane >> SH;
    if ((lane & ((1 << SH) - 1)) == 0 && jb < J::N) sm.pj[P][jb][wave - R::W0] = term[0];
}

template <int DK, int DV, typename TI, typename TO, int M, int PAR>
__device__ __forceinline__ void decodec_update(const DecodeParams &p, int bh, int tid,
                                               f32x4 (&sv)[DecodeShape<DK, DV>::RPT], const DecodeCTok<M, TI> &in,
                                               DecodeCShared<DK, DV, M> &sm) {
    using Sh = DecodeShape<DK, DV>;
    using J = DecodeCJobs<M>;
    using R = DecodeCRoles<DK, DV>;
    const int c4 = tid % Sh::TPR, rg = tid / Sh::TPR, wave = tid / 64, lane = tid % 64;
    // partial S0^T Ktil_t and S0^T Qtil_t over this thread's rows
    const int r0 = rg * Sh::RPT;
#pragma unroll
    for (int t = 0; t < M; ++t) {
        float kr[Sh::RPT], qr[Sh::RPT];
        lds_rows<Sh::RPT>(&sm.kt[PAR][t][r0], kr);
        lds_rows<Sh::RPT>(&sm.qt[PAR][t][r0], qr);
        f32x4 x = sv[0] * kr[0], y = sv[0] * qr[0];
#pragma unroll
        for (int i = 1; i < Sh::RPT; ++i) {
            x += sv[i] * kr[i];
            y += sv[i] * qr[i];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[j] = rowgroup_sum<Sh::TPR>(x[j]);
            y[j] = rowgroup_sum<Sh::TPR>(y[j]);
        }
        if (lane < Sh::TPR) {
            *reinterpret_cast<f32x4 *>(&sm.red[0][t][wave][4 * c4]) = x;
            *reinterpret_cast<f32x4 *>(&sm.red[1][t][wave][4 * c4]) = y;
        }
    }
    lds_barrier();
    const int64_t tok0 = static_cast<int64_t>(bh / p.H) * M * p.H + bh % p.H;
    // column owners: Delta by forward substitution and the outputs, once per column
    if (tid < DV) {
        const int j = tid;
        const bool norm = (p.prologue & kProQKNorm) != 0;
        auto pair = [&](int jb) {
            float s = sm.pj[PAR][jb][0];
#pragma unroll
            for (int u = 1; u < R::NPART; ++u) s += sm.pj[PAR][jb][u];
            return s;
        };
        float nk[M], nq[M], x[M], y[M], dl[M];
#pragma unroll
        for (int t = 0; t < M; ++t) {
            nk[t] = nq[t] = 1.f;
            if (norm) {
                nk[t] = 1.f / __builtin_sqrtf(pair(J::k2(t)) + kQKNormEps);
                nq[t] = 1.f / __builtin_sqrtf(pair(J::q2(t)) + kQKNormEps);
            }
            x[t] = sm.red[0][t][0][j];
            y[t] = sm.red[1][t][0][j];
#pragma unroll
            for (int w = 1; w < Sh::NW; ++w) {
                x[t] += sm.red[0][t][w][j];
                y[t] += sm.red[1][t][w][j];
            }
        }
        TO *o = static_cast<TO *>(p.o);
#pragma unroll
        for (int t = 0; t < M; ++t) {
            float bt = io<TI>::ld(&in.r[M + t], 0);
            if (p.prologue & kProBeta) bt = sigmoid_f32(bt);
            float d = bt * (io<TI>::ld(&in.r[t], 0) - nk[t] * x[t]);
#pragma unroll
            for (int i = 0; i < t; ++i) d -= (bt * nk[t] * nk[i] * pair(J::kk(t, i))) * dl[i];
            dl[t] = d;
            float ot = nq[t] * y[t];
#pragma unroll
            for (int i = 0; i <= t; ++i) ot += (nq[t] * nk[i] * pair(J::qk(t, i))) * dl[i];
            io<TO>::st(o, (tok0 + static_cast<int64_t>(t) * p.H) * DV + j, ot);
            sm.dl[t][j] = nk[t] * d;
        }
    }
    // row owners meanwhile: the next state's factors and pair sums
    decodec_stage<DK, DV, TI, M, PAR ^ 1>(p, tid, in, sm);
    lds_barrier();
    f32x4 dl[M];
#pragma unroll
    for (int t = 0; t < M; ++t) dl[t] = *reinterpret_cast<const f32x4 *>(&sm.dl[t][4 * c4]);
    const uint32_t lo = static_cast<uint32_t>(r0 * DV + 4 * c4);
    if (p.token_states) {   // token by token: S_{t+1} = a_t S_t + k_t (nk_t Delta_t)^T
#pragma unroll
        for (int t = 0; t < M; ++t) {
            float *ts = p.token_states + (tok0 + static_cast<int64_t>(t) * p.H) * DK * DV;
            float ar[Sh::RPT], kr[Sh::RPT];
            lds_rows<Sh::RPT>(&sm.a[PAR][t][r0], ar);
            lds_rows<Sh::RPT>(&sm.k[PAR][t][r0], kr);
#pragma unroll
            for (int i = 0; i < Sh::RPT; ++i) {
                sv[i] = ar[i] * sv[i] + kr[i] * dl[t];
                __builtin_nontemporal_store(sv[i], reinterpret_cast<f32x4 *>(ts + (lo + static_cast<uint32_t>(i * DV))));
            }
        }
    } else {                // S_m = Gamma_{m-1} S0 + sum_t kh_t (nk_t Delta_t)^T
        float gr[Sh::RPT];
        lds_rows<Sh::RPT>(&sm.gm[PAR][r0], gr);
#pragma unroll
        for (int i = 0; i < Sh::RPT; ++i) sv[i] *= gr[i];
#pragma unroll
        for (int t = 0; t < M; ++t) {
            float kr[Sh::RPT];
            lds_rows<Sh::RPT>(&sm.kh[PAR][t][r0], kr);
#pragma unroll
            for (int i = 0; i < Sh::RPT; ++i) sv[i] += kr[i] * dl[t];
        }
    }
    if (p.state_out) {
        float *dst = p.state_out + static_cast<int64_t>(bh) * DK * DV;
#pragma unroll
        for (int i = 0; i < Sh::RPT; ++i)
            __builtin_nontemporal_store(sv[i], reinterpret_cast<f32x4 *>(dst + (lo + static_cast<uint32_t>(i * DV))));
    }
}

template <int DK, int DV, typename TI, typename TO, int M>
__global__ void __launch_bounds__((DecodeShape<DK, DV>::NT)) decodec_kernel(DecodeParams p, int BH) {
    using Sh = DecodeShape<DK, DV>;
    static_assert(M >= 2 && DK + DV <= Sh::NT, "a column owner per column and a row owner per row");
    __shared__ DecodeCShared<DK, DV, M> sm;
    const int tid = threadIdx.x, G = gridDim.x;
    f32x4 svA[Sh::RPT], svB[Sh::RPT];
    DecodeCTok<M, TI> inA{}, inB{};
    auto clamp = [&](int x) { return x < BH ? x : BH - 1; };
    int bh = blockIdx.x;   // uniform: every wave takes the same branches
    if (bh >= BH) return;
    // the first state's tokens staged before the walk; afterwards every
    // update stages the tokens of the state after it
    decodec_request<DK, DV, M, TI>(p, bh, bh, bh, tid, svA, inA);
    decodec_stage<DK, DV, TI, M, 0>(p, tid, inA, sm);
    decodec_request_tokens<DK, DV, M, TI>(p, bh, clamp(bh + G), tid, inA);
    lds_barrier();
    for (;;) {
        // inA: state bh, v and beta of bh, a, k, q of bh + G
        const int bh1 = bh + G;
        decodec_request<DK, DV, M, TI>(p, clamp(bh1), clamp(bh1), clamp(bh1 + G), tid, svB, inB);
        decodec_update<DK, DV, TI, TO, M, 0>(p, bh, tid, svA, inA, sm);
        if (bh1 >= BH) break;
        const int bh2 = bh1 + G;
        decodec_request<DK, DV, M, TI>(p, clamp(bh2), clamp(bh2), clamp(bh2 + G), tid, svA, inA);
        decodec_update<DK, DV, TI, TO, M, 1>(p, bh1, tid, svB, inB, sm);
        if (bh2 >= BH) break;
        bh = bh2;
    }
}

}  // namespace kda

namespace kda {

namespace {
template <int DK, int DV, typename TI, typename TO>
hipError_t run_decode(const DecodeParams &p, int B, hipStream_t s) {
    using Sh = DecodeShape<DK, DV>;
    const dim3 grid(static_cast<unsigned>(B) * p.H), block(Sh::NT);
    if (p.m == 1 && !p.token_states && p.state_out) {
        const int BH = B * p.H;
        const int G = BH < kDecodeGrid ? BH : kDecodeGrid;
        hipLaunchKernelGGL((decode1_kernel<DK, DV, TI, TO>), dim3(G), block, 0, s, p, BH);
    } else if (p.m >= 2 && p.m <= 4 && !p.token_states) {
        // one workgroup per CU at these register counts; 3 and 4 tokens per
        // launch ran faster with one persistent workgroup per CU, 2 tokens
        // with two rounds of them (B=256, H=32, d=128: m = 4 in 203 against
        // 207 us, m = 3 in 188 against 190 us, m = 2 in 190 against 200 us;
        // grids that are not a multiple of 256 leave a partial second round)
        const int BH = B * p.H;
        const int GM = p.m == 2 ? kDecodeGrid : kDecodeGrid / 2;
        const int G = BH < GM ? BH : GM;
        if (p.m == 2) hipLaunchKernelGGL((decodec_kernel<DK, DV, TI, TO, 2>), dim3(G), block, 0, s, p, BH);
        else if (p.m == 3) hipLaunchKernelGGL((decodec_kernel<DK, DV, TI, TO, 3>), dim3(G), block, 0, s, p, BH);
        else hipLaunchKernelGGL((decodec_kernel<DK, DV, TI, TO, 4>), dim3(G), block, 0, s, p, BH);
    } else if (p.token_states && p.m <= DecodeMShape<DK, DV>::MT) {
        const int BH = B * p.H;
        const int G = BH < kDecodeGrid ? BH : kDecodeGrid;
        hipLaunchKernelGGL((decodem_kernel<DK, DV, TI, TO>), dim3(G), block, 0, s, p, BH);
    } else if (p.m == 1 && !p.token_states)
        hipLaunchKernelGGL((decode_kernel<DK, DV, TI, TO, false>), grid, block, 0, s, p);
    else
        hipLaunchKernelGGL((decode_kernel<DK, DV, TI, TO, true>), grid, block, 0, s, p);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t run_decode_dt(const DecodeParams &p, int B, int in_dt, int out_dt, hipStream_t s) {
    if (in_dt == 0 && out_dt == 0) return run_decode<DK, DV, float, float>(p, B, s);
    if (in_dt == 0 && out_dt == 1) return run_decode<DK, DV, float, bf16_t>(p, B, s);
    if (in_dt == 1 && out_dt == 0) return run_decode<DK, DV, bf16_t, float>(p, B, s);
    return run_decode<DK, DV, bf16_t, bf16_t>(p, B, s);
}

template <int DK>
hipError_t run_decode_dv(const DecodeParams &p, int B, int dv, int in_dt, int out_dt, hipStream_t s) {
    switch (dv) {
        case 16: return run_decode_dt<DK, 16>(p, B, in_dt, out_dt, s);
        case 32: return run_decode_dt<DK, 32>(p, B, in_dt, out_dt, s);
        case 64: return run_decode_dt<DK, 64>(p, B, in_dt, out_dt, s);
        default: return run_decode_dt<DK, 128>(p, B, in_dt, out_dt, s);
    }
}
}  // namespace

hipError_t launch_decode(int B, int H, int m, int dk, int dv, int in_dtype, int out_dtype, uint32_t prologue,
                         const void *q, const void *k, const void *v, const void *beta, const void *log_alpha,
                         const float *state_in, float *state_out, float *token_states, void *o, hipStream_t s) {
    DecodeParams p{q, k, v, beta, log_alpha, state_in, state_out, token_states, o, H, m, prologue};
    switch (dk) {
        case 16: return run_decode_dv<16>(p, B, dv, in_dtype, out_dtype, s);
        case 32: return run_decode_dv<32>(p, B, dv, in_dtype, out_dtype, s);
        case 64: return run_decode_dv<64>(p, B, dv, in_dtype, out_dtype, s);
        default: return run_decode_dv<128>(p, B, dv, in_dtype, out_dtype, s);
    }
}

}  // namespace kda
