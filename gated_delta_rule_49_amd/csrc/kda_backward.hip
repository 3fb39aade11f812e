// Backward pass of the KDA recurrence: gradients of q, k, v, beta, log alpha
// and the initial state from the gradients of the outputs and final state.
// The pages call the affine composition the argument for parallel training
// (course index, module list, the Module 04 entry) without deriving a
// backward; this is reverse-mode differentiation of one token's operations
//     S' = Diag(a) S, p = S'^T k, e = v - p, S_t = S' + b k e^T, o = S_t^T q
// applied from the last token to the first:
//     dS += q do^T;  dq = S_t do;  u = dS^T k;  dv = b u;  db = u . e
//     dk = b dS e - S' (b u);  dS' = dS - k (b u)^T;  dlog a = a * rowsum(dS' * S)
//     dS <- Diag(a) dS'
//
// One workgroup per (sequence, head, 4-column tile of the state): the
// columns of S and dS evolve independently, so a tile carries its own dS;
// the row quantities (dq, dk, dlog a) and db are sums over all columns and
// are accumulated across the tiles with fp32 atomics (their summation order
// is not fixed).  Thread i owns row i of the tile (BWD_BV floats of dS in
// registers).  The states the backward needs are recomputed per 16-token
// segment, last segment first, from checkpoints (the states entering every
// 16-token chunk, as a chunked prefill with chunk size 16 writes them):
// the segment's inputs are staged in LDS at its start, its states and
// errors are stored in LDS on a forward sweep and consumed on the backward
// sweep.  Everything is fp32.  Waves meet with an LDS-only barrier, so the
// atomic adds of one token are still in flight while the next is computed.
#include "kda_launch.hpp"

namespace kda {

constexpr int BWD_BV = 4;    // state columns per workgroup
constexpr int BWD_SEG = 16;  // tokens per recomputed segment (= checkpoint spacing)

// v of the lane named by a DPP control (quad permutes and row mirrors: every
// lane has a source in its own row of 16, so no bound control is involved)
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Column sums of a BWD_BV-vector over the DK threads of the workgroup; every
// thread gets the totals.  Each row of 16 lanes is summed with four DPP
// steps (exchange within pairs, within quads, then half-row and row
// mirrors), which leaves the row's sum in all its lanes; the DK / 16 row sums
// meet in LDS.  red: LDS [2][DK / 16][8], used alternately so that one
// barrier per reduction suffices.
template <int DK>
__device__ __forceinline__ void col_sum(float (&x)[BWD_BV], float (*red)[DK / 16][BWD_BV], int &par, int tid) {
    constexpr int NROW = DK / 16;
#pragma unroll
    for (int j = 0; j < BWD_BV; ++j) {
        x[j] += dpp<0xB1>(x[j]);   // quad_perm [1, 0, 3, 2]
        x[j] += dpp<0x4E>(x[j]);   // quad_perm [2, 3, 0, 1]
        x[j] += dpp<0x141>(x[j]);  // row_half_mirror
        x[j] += dpp<0x140>(x[j]);  // row_mirror
    }
    if ((tid & 15) == 0)
#pragma unroll
        for (int j = 0; j < BWD_BV; ++j) red[par][tid >> 4][j] = x[j];
    lds_barrier();
#pragma unroll
    for (int j = 0; j < BWD_BV; ++j) {
        float s = 0.f;
#pragma unroll
        for (int r = 0; r < NROW; ++r) s += red[par][r][j];
        x[j] = s;
    }
    par ^= 1;
}

template <int DK, typename TI>
__global__ void __launch_bounds__(DK) backward_kernel(BackwardParams p) {
    if (*p.status != 0) return;
    const int nvt = p.dv / BWD_BV;
    const int vt = blockIdx.x % nvt;
    const int h = (blockIdx.x / nvt) % p.H;
    const int n = blockIdx.x / (nvt * p.H);
    const int j0 = vt * BWD_BV;
    const int i = threadIdx.x;
    const TI *q = static_cast<const TI *>(p.q);
    const TI *k = static_cast<const TI *>(p.k);
    const TI *v = static_cast<const TI *>(p.v);
    const TI *beta = static_cast<const TI *>(p.beta);
    const TI *la = static_cast<const TI *>(p.log_alpha);

    __shared__ float segS[BWD_SEG][DK][BWD_BV];   // S_{t-1} of the segment's tokens
    __shared__ float segE[BWD_SEG][BWD_BV];       // e_t
    // the segment's inputs, loaded together at its start (one memory
    // latency per segment instead of one per token and sweep)
    __shared__ float segA[BWD_SEG][DK], segK[BWD_SEG][DK], segQ[BWD_SEG][DK];
    __shared__ float segV[BWD_SEG][BWD_BV], segDo[BWD_SEG][BWD_BV], segB[BWD_SEG];
    __shared__ float red[2][DK / 16][BWD_BV];
    int par = 0;

    int64_t start;
    int len;
    if (p.cu_seqlens) {
        start = p.cu_seqlens[n];
        len = p.cu_seqlens[n + 1] - p.cu_seqlens[n];
    } else {
        start = static_cast<int64_t>(n) * p.T;
        len = p.T;
    }
    const int nseg = (len + BWD_SEG - 1) / BWD_SEG;
    const int64_t cbase = p.chunk_off[n];
    const int64_t sbase = (static_cast<int64_t>(n) * p.H + h) * DK * p.dv;

    float dS[BWD_BV];
#pragma unroll
    for (int j = 0; j < BWD_BV; ++j)
        dS[j] = p.d_final ? p.d_final[sbase + static_cast<int64_t>(i) * p.dv + j0 + j] : 0.f;

    for (int c = nseg - 1; c >= 0; --c) {
        const int64_t t0 = start + static_cast<int64_t>(c) * BWD_SEG;
        const int L = min(BWD_SEG, len - c * BWD_SEG);
        // stage the segment's inputs
#pragma unroll
        for (int r = 0; r < BWD_SEG; ++r) {
            if (r >= L) continue;
            const int64_t th = (t0 + r) * p.H + h;
            segA[r][i] = __expf(io<TI>::ld(la, th * DK + i));
            segK[r][i] = io<TI>::ld(k, th * DK + i);
            segQ[r][i] = io<TI>::ld(q, th * DK + i);
        }
        for (int e = i; e < L * BWD_BV; e += DK) {
            const int r = e / BWD_BV, j = e % BWD_BV;
            const int64_t th = (t0 + r) * p.H + h;
            segV[r][j] = io<TI>::ld(v, th * p.dv + j0 + j);
            segDo[r][j] = p.d_o[th * p.dv + j0 + j];
        }
        if (i < L) segB[i] = io<TI>::ld(beta, (t0 + i) * p.H + h);
        // forward sweep: recompute the segment's states from its checkpoint
        float S[BWD_BV];
        const float *ck = p.checkpoints + ((cbase + c) * p.H + h) * static_cast<int64_t>(DK) * p.dv;
#pragma unroll
        for (int j = 0; j < BWD_BV; ++j) S[j] = ck[static_cast<int64_t>(i) * p.dv + j0 + j];
        lds_barrier();
        for (int r = 0; r < L; ++r) {
            const float a = segA[r][i];
            const float ki = segK[r][i];
            const float b = segB[r];
            float pk[BWD_BV];
#pragma unroll
            for (int j = 0; j < BWD_BV; ++j) {
                segS[r][i][j] = S[j];
                S[j] *= a;
                pk[j] = S[j] * ki;
            }
            col_sum<DK>(pk, red, par, i);
#pragma unroll
            for (int j = 0; j < BWD_BV; ++j) {
                const float e = segV[r][j] - pk[j];
                if (i == 0) segE[r][j] = e;
                S[j] += b * ki * e;
            }
        }
        lds_barrier();
        // backward sweep
        for (int r = L - 1; r >= 0; --r) {
            const int64_t th = (t0 + r) * p.H + h;
            const float a = segA[r][i];
            const float ki = segK[r][i];
            const float qi = segQ[r][i];
            const float b = segB[r];
            float Sp[BWD_BV], e[BWD_BV], dov[BWD_BV], u[BWD_BV];
            float dqi = 0.f;
#pragma unroll
            for (int j = 0; j < BWD_BV; ++j) {
                Sp[j] = a * segS[r][i][j];
                e[j] = segE[r][j];
                dov[j] = segDo[r][j];
                const float St = Sp[j] + b * ki * e[j];
                dqi += St * dov[j];
                dS[j] += qi * dov[j];
                u[j] = ki * dS[j];
            }
            col_sum<DK>(u, red, par, i);
            float dki = 0.f, dga = 0.f, db = 0.f;
#pragma unroll
            for (int j = 0; j < BWD_BV; ++j) {
                const float dp = -b * u[j];
                dki += b * dS[j] * e[j] + Sp[j] * dp;
                const float dSp = dS[j] + ki * dp;
                dga += dSp * segS[r][i][j];
                dS[j] = a * dSp;
                db += u[j] * e[j];
            }
            atomicAdd(p.gq + th * DK + i, dqi);
            atomicAdd(p.gk + th * DK + i, dki);
            atomicAdd(p.gg + th * DK + i, a * dga);
            if (i == 0) {
                atomicAdd(p.gbeta + th, db);
#pragma unroll
                for (int j = 0; j < BWD_BV; ++j) p.gv[th * p.dv + j0 + j] = b * u[j];
            }
        }
        lds_barrier();  // segS / segE are rewritten by the next segment
    }
    if (p.d_initial)
#pragma unroll
        for (int j = 0; j < BWD_BV; ++j) p.d_initial[sbase + static_cast<int64_t>(i) * p.dv + j0 + j] = dS[j];
}

__global__ void zero_kernel(float *x, int64_t n) {
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < n;
         e += static_cast<int64_t>(gridDim.x) * blockDim.x)
        x[e] = 0.f;
}

namespace {
hipError_t zero(float *x, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
    hipLaunchKernelGGL(zero_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, x, n);
    return hipGetLastError();
}

template <int DK, typename TI>
hipError_t run_backward(const BackwardParams &p, hipStream_t s) {
    const unsigned grid = static_cast<unsigned>(p.N) * p.H * (p.dv / BWD_BV);
    hipLaunchKernelGGL((backward_kernel<DK, TI>), dim3(grid), dim3(DK), 0, s, p);
    return hipGetLastError();
}

template <typename TI>
hipError_t run_backward_dk(const BackwardParams &p, hipStream_t s) {
    switch (p.dk) {
        case 16: return run_backward<16, TI>(p, s);
        case 32: return run_backward<32, TI>(p, s);
        case 64: return run_backward<64, TI>(p, s);
        default: return run_backward<128, TI>(p, s);
    }
}
}  // namespace

hipError_t launch_backward(const BackwardParams &p, int in_dtype, hipStream_t s) {
    const int64_t tok = static_cast<int64_t>(p.B) * p.T * p.H;
    hipError_t e = zero(p.gq, tok * p.dk, s);
    if (e == hipSuccess) e = zero(p.gk, tok * p.dk, s);
    if (e == hipSuccess) e = zero(p.gg, tok * p.dk, s);
    if (e == hipSuccess) e = zero(p.gbeta, tok, s);
    if (e == hipSuccess) e = zero(p.gv, tok * p.dv, s);  // tokens outside every sequence stay 0
    if (e != hipSuccess) return e;
    return in_dtype == 0 ? run_backward_dk<float>(p, s) : run_backward_dk<bf16_t>(p, s);
}

}  // namespace kda
