// Fused single-token KDA decode step (Module 04 — KDA II, §2 "Why decode and
// prefill need different kernels": decode applies one recurrent step to a
// state already resident in memory).
//
// Per (sequence b, head h), with a = exp(log_alpha) and S the fp32 state:
//     p = S^T (a * k),  r = S^T (a * q),  kappa = k . q
//     delta = beta (v - p)
//     o = r + kappa * delta               (= S_t^T q_t, post-update state)
//     S <- a * S + k delta^T              (= (I - beta k k^T) Diag(a) S + beta k v^T)
// The state is HBM-bound: it is read once into registers, reduced along d_k,
// and written once.  One workgroup per (b, h); the column space of S is
// split across lanes in float4 groups (16-byte coalesced rows) and the row
// space across row groups; the d_k reductions run lane-to-lane inside a wave
// (DPP/permute via __shfl_xor) and across waves through LDS.
#include "kda_launch.hpp"

namespace kda {

template <int DK, int DV>
struct DecodeShape {
    static constexpr int TPR = DV / 4;                      // threads per row
    static constexpr int RG = (DK < 256 / TPR) ? DK : 256 / TPR;  // row groups
    static constexpr int NT = TPR * RG;                     // threads
    static constexpr int RPT = DK / RG;                     // rows per thread
    static constexpr int NW = (NT + 63) / 64;               // waves
    static constexpr int RG_PER_WAVE = 64 / TPR;            // row groups in a wave
};

template <int DK, int DV, typename TI, typename TO>
__global__ void __launch_bounds__((DecodeShape<DK, DV>::NT))
decode_step_kernel(const TI *__restrict__ q, const TI *__restrict__ k, const TI *__restrict__ v,
                   const TI *__restrict__ beta, const TI *__restrict__ log_alpha,
                   float *__restrict__ state, TO *__restrict__ o, int H) {
    using Sh = DecodeShape<DK, DV>;
    const int bh = blockIdx.x;
    const int tid = threadIdx.x;
    const int c4 = tid % Sh::TPR;   // column group: columns 4*c4 .. 4*c4+3
    const int rg = tid / Sh::TPR;   // row group: rows rg + RG*i

    __shared__ float s_a[DK], s_k[DK], s_q[DK], s_ak[DK], s_aq[DK];
    __shared__ float s_red[2][Sh::NW > 1 ? Sh::NW : 1][DV];
    __shared__ float s_kappa;

    const int64_t vecoff = static_cast<int64_t>(bh) * DK;
    for (int i = tid; i < DK; i += Sh::NT) {
        const float a = __expf(io<TI>::ld(log_alpha, vecoff + i));
        const float kk = io<TI>::ld(k, vecoff + i);
        const float qq = io<TI>::ld(q, vecoff + i);
        s_a[i] = a;
        s_k[i] = kk;
        s_q[i] = qq;
        s_ak[i] = a * kk;
        s_aq[i] = a * qq;
    }
    __syncthreads();
    if (tid < 64) {
        float kq = 0.f;
        for (int i = tid; i < DK; i += 64) kq += s_k[i] * s_q[i];
        for (int m = 32; m >= 1; m >>= 1) kq += __shfl_xor(kq, m);
        if (tid == 0) s_kappa = kq;
    }

    // load this thread's rows of S (float4 each) and reduce p, r partials
    float4 *S4 = reinterpret_cast<float4 *>(state + static_cast<int64_t>(bh) * DK * DV);
    float4 sv[Sh::RPT];
    float p[4] = {0.f, 0.f, 0.f, 0.f}, r[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < Sh::RPT; ++i) {
        const int row = rg + Sh::RG * i;
        sv[i] = S4[row * (DV / 4) + c4];
    }
#pragma unroll
    for (int i = 0; i < Sh::RPT; ++i) {
        const int row = rg + Sh::RG * i;
        const float ak = s_ak[row], aq = s_aq[row];
        p[0] += sv[i].x * ak; p[1] += sv[i].y * ak; p[2] += sv[i].z * ak; p[3] += sv[i].w * ak;
        r[0] += sv[i].x * aq; r[1] += sv[i].y * aq; r[2] += sv[i].z * aq; r[3] += sv[i].w * aq;
    }
    // reduce across the row groups inside the wave (lane bits >= log2(TPR))
#pragma unroll
    for (int m = Sh::TPR; m < 64 && m < Sh::NT; m <<= 1) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            p[j] += __shfl_xor(p[j], m);
            r[j] += __shfl_xor(r[j], m);
        }
    }
    const int wave = tid / 64;
    const int lane = tid % 64;
    if (lane < Sh::TPR) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            s_red[0][wave][4 * c4 + j] = p[j];
            s_red[1][wave][4 * c4 + j] = r[j];
        }
    }
    __syncthreads();
    // every thread needs delta for its 4 columns: sum the wave partials
    float pt[4] = {0.f, 0.f, 0.f, 0.f}, rt[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < Sh::NW; ++w) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            pt[j] += s_red[0][w][4 * c4 + j];
            rt[j] += s_red[1][w][4 * c4 + j];
        }
    }
    const float b = io<TI>::ld(beta, bh);
    const int64_t voff = static_cast<int64_t>(bh) * DV + 4 * c4;
    float delta[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) delta[j] = b * (io<TI>::ld(v, voff + j) - pt[j]);
    if (rg == 0) {
        const float kappa = s_kappa;
#pragma unroll
        for (int j = 0; j < 4; ++j) io<TO>::st(o, voff + j, rt[j] + kappa * delta[j]);
    }
#pragma unroll
    for (int i = 0; i < Sh::RPT; ++i) {
        const int row = rg + Sh::RG * i;
        const float a = s_a[row], kk = s_k[row];
        float4 s = sv[i];
        s.x = a * s.x + kk * delta[0];
        s.y = a * s.y + kk * delta[1];
        s.z = a * s.z + kk * delta[2];
        s.w = a * s.w + kk * delta[3];
        S4[row * (DV / 4) + c4] = s;
    }
}

}  // namespace kda

namespace kda {

namespace {
template <int DK, int DV, typename TI, typename TO>
hipError_t run_decode(int B, int H, const void *q, const void *k, const void *v, const void *beta,
                      const void *la, float *state, void *o, hipStream_t s) {
    using Sh = DecodeShape<DK, DV>;
    hipLaunchKernelGGL((decode_step_kernel<DK, DV, TI, TO>), dim3(static_cast<unsigned>(B) * H),
                       dim3(Sh::NT), 0, s, static_cast<const TI *>(q), static_cast<const TI *>(k),
                       static_cast<const TI *>(v), static_cast<const TI *>(beta),
                       static_cast<const TI *>(la), state, static_cast<TO *>(o), H);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t run_decode_dt(int B, int H, int in_dt, int out_dt, const void *q, const void *k,
                         const void *v, const void *beta, const void *la, float *state, void *o,
                         hipStream_t s) {
    if (in_dt == 0 && out_dt == 0) return run_decode<DK, DV, float, float>(B, H, q, k, v, beta, la, state, o, s);
    if (in_dt == 0 && out_dt == 1) return run_decode<DK, DV, float, bf16_t>(B, H, q, k, v, beta, la, state, o, s);
    if (in_dt == 1 && out_dt == 0) return run_decode<DK, DV, bf16_t, float>(B, H, q, k, v, beta, la, state, o, s);
    return run_decode<DK, DV, bf16_t, bf16_t>(B, H, q, k, v, beta, la, state, o, s);
}

template <int DK>
hipError_t run_decode_dv(int B, int H, int dv, int in_dt, int out_dt, const void *q, const void *k,
                         const void *v, const void *beta, const void *la, float *state, void *o,
                         hipStream_t s) {
    switch (dv) {
        case 16: return run_decode_dt<DK, 16>(B, H, in_dt, out_dt, q, k, v, beta, la, state, o, s);
        case 32: return run_decode_dt<DK, 32>(B, H, in_dt, out_dt, q, k, v, beta, la, state, o, s);
        case 64: return run_decode_dt<DK, 64>(B, H, in_dt, out_dt, q, k, v, beta, la, state, o, s);
        default: return run_decode_dt<DK, 128>(B, H, in_dt, out_dt, q, k, v, beta, la, state, o, s);
    }
}
}  // namespace

hipError_t launch_decode(int B, int H, int dk, int dv, int in_dtype, int out_dtype, const void *q,
                         const void *k, const void *v, const void *beta, const void *log_alpha,
                         float *state, void *o, hipStream_t s) {
    switch (dk) {
        case 16: return run_decode_dv<16>(B, H, dv, in_dtype, out_dtype, q, k, v, beta, log_alpha, state, o, s);
        case 32: return run_decode_dv<32>(B, H, dv, in_dtype, out_dtype, q, k, v, beta, log_alpha, state, o, s);
        case 64: return run_decode_dv<64>(B, H, dv, in_dtype, out_dtype, q, k, v, beta, log_alpha, state, o, s);
        default: return run_decode_dv<128>(B, H, dv, in_dtype, out_dtype, q, k, v, beta, log_alpha, state, o, s);
    }
}

}  // namespace kda
