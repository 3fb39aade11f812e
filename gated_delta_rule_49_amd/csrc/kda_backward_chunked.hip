// Chunked backward pass of the KDA recurrence (bf16 inputs): the gradients
// of one chunk follow from the chunk's structured form
//     X = V - K~ S,  Delta = T X,  O = Q~ S + P Delta,  S' = Diag(g) S + K^T Delta
// (K~ = k e^G, Q~ = q e^G, K^ = k e^{G_L - G}, g = e^{G_L}, A = Diag(beta)
// strict-lower(k k^T e^{G_r - G_i}), M = (I + A)^-1, T = M Diag(beta),
// P = lower(q k^T e^{G_r - G_i})) by reverse-mode differentiation of these
// matrix products; the chunks are coupled only through the state gradient,
//     dS = Diag(g) dS' + Q~^T dO - W^T (P^T dO + K^ dS'),   W = T K~,
// a scan over the chunks in reverse that needs no forward state.  The
// pages derive no backward (course index, module list, the Module 04 entry
// calls the affine composition the argument for parallel training).
//
// Three kernels, all fp32 on the vector ALUs:
//   prep  (chunk, head):  G, K~, Q~, K^, g, Gh = k k^T e^{..}, P, M, W -> a block
//   scan  (sequence, head, 16-column tile): dS' of every chunk, last first
//   grad  (chunk, head):  every gradient of the chunk's tokens from its
//         entering state (the forward checkpoint), dS', dO and the block.
// No atomics: each chunk-head writes its own tokens' gradients.
#include "kda_launch.hpp"

namespace kda {

constexpr int CB_C = 64;  // maximum chunk length

// per-(chunk, head) block of the prep kernel, fp32, row-major
template <int DK>
struct CbLay {
    static constexpr size_t G = 0;                       // [C][DK]  cumulative log decay
    static constexpr size_t KT = G + CB_C * DK;          // [DK][C]  (k e^G)^T
    static constexpr size_t QT = KT + CB_C * DK;         // [C][DK]  q e^G
    static constexpr size_t KB = QT + CB_C * DK;         // [DK][C]  (k e^{G_L - G})^T
    static constexpr size_t W = KB + CB_C * DK;          // [C][DK]  T K~
    static constexpr size_t GH = W + CB_C * DK;          // [C][C]   k_r . k_i e^{..}, i < r
    static constexpr size_t P = GH + CB_C * CB_C;        // [C][C]   q_r . k_i e^{..}, i <= r
    static constexpr size_t M = P + CB_C * CB_C;         // [C][C]   (I + A)^-1
    static constexpr size_t MT = M + CB_C * CB_C;        // [C][C]   its transpose
    static constexpr size_t GAM = MT + CB_C * CB_C;      // [DK]     e^{G_L}
    static constexpr size_t BETA = GAM + DK;             // [C]
    static constexpr size_t FLOATS = (BETA + CB_C + 63) / 64 * 64;
};

size_t cb_block_bytes(int dk) {
    switch (dk) {
        case 16: return CbLay<16>::FLOATS * 4;
        case 32: return CbLay<32>::FLOATS * 4;
        case 64: return CbLay<64>::FLOATS * 4;
        default: return CbLay<128>::FLOATS * 4;
    }
}

// ------------------------------------------------------------------ prep --
template <int DK, typename TI>
__global__ void __launch_bounds__(256) cb_prep_kernel(CbParams p) {
    if (*p.status != 0) return;
    using Y = CbLay<DK>;
    const int H = p.H;
    const int x = blockIdx.x / H, h = blockIdx.x % H;
    if (x >= p.chunk_off[p.N]) return;  // the grid covers a bound on the chunk count
    const int4 ci = p.chunk_info[x];
    const int64_t t0 = static_cast<int64_t>(static_cast<uint32_t>(ci.x)) | (static_cast<int64_t>(ci.y) << 32);
    const int L = ci.z;
    const int tid = threadIdx.x;
    float *blk = p.blocks + (static_cast<size_t>(x) * H + h) * Y::FLOATS;
    const TI *q = static_cast<const TI *>(p.q);
    const TI *k = static_cast<const TI *>(p.k);
    const TI *la = static_cast<const TI *>(p.log_alpha);
    const TI *beta = static_cast<const TI *>(p.beta);

    __shared__ float sq[CB_C][DK + 1], sk[CB_C][DK + 1], sG[CB_C][DK + 1];
    __shared__ float sA[CB_C][CB_C + 1];
    __shared__ float sb[CB_C];

    for (int e = tid; e < CB_C * DK; e += 256) {
        const int r = e / DK, c = e % DK;
        const int64_t off = ((t0 + r) * H + h) * DK + c;
        const bool live = r < L;
        sq[r][c] = live ? io<TI>::ld(q, off) : 0.f;
        sk[r][c] = live ? io<TI>::ld(k, off) : 0.f;
        sG[r][c] = live ? io<TI>::ld(la, off) : 0.f;
    }
    if (tid < CB_C) sb[tid] = tid < L ? io<TI>::ld(beta, (t0 + tid) * H + h) : 0.f;
    __syncthreads();
    if (tid < DK) {  // cumulative decay, accumulated in fp64
        double acc = 0.0;
        for (int r = 0; r < CB_C; ++r) {
            acc += static_cast<double>(sG[r][tid]);
            sG[r][tid] = static_cast<float>(acc);
        }
    }
    __syncthreads();
    // elementwise factors and the decay of the whole chunk
    for (int e = tid; e < CB_C * DK; e += 256) {
        const int r = e / DK, c = e % DK;
        const float G = sG[r][c];
        blk[Y::G + e] = G;
        blk[Y::QT + e] = sq[r][c] * __expf(G);
    }
    for (int e = tid; e < CB_C * DK; e += 256) {  // transposed: [channel][row]
        const int c = e / CB_C, r = e % CB_C;
        const float G = sG[r][c];
        blk[Y::KT + e] = sk[r][c] * __expf(G);
        blk[Y::KB + e] = sk[r][c] * __expf(sG[CB_C - 1][c] - G);
    }
    for (int c = tid; c < DK; c += 256) blk[Y::GAM + c] = __expf(sG[CB_C - 1][c]);
    if (tid < CB_C) blk[Y::BETA + tid] = sb[tid];
    // Gh and P on the lower triangle, 4 x 4 pair blocks per thread
    constexpr int NB = CB_C / 4;
    for (int bi = tid; bi < NB * (NB + 1) / 2; bi += 256) {
        int R = 0;
        while ((R + 1) * (R + 2) / 2 <= bi) ++R;
        const int I = bi - R * (R + 1) / 2;  // I <= R
        float gh[4][4] = {}, pp[4][4] = {};
        for (int c = 0; c < DK; ++c) {
            float kr[4], qr[4], gr[4], ki[4], gi[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                kr[a] = sk[4 * R + a][c]; qr[a] = sq[4 * R + a][c]; gr[a] = sG[4 * R + a][c];
                ki[a] = sk[4 * I + a][c]; gi[a] = sG[4 * I + a][c];
            }
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b2 = 0; b2 < 4; ++b2) {
                    const float e = __expf(fminf(gr[a] - gi[b2], 0.f));
                    gh[a][b2] += kr[a] * ki[b2] * e;
                    pp[a][b2] += qr[a] * ki[b2] * e;
                }
        }
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b2 = 0; b2 < 4; ++b2) {
                const int r = 4 * R + a, i = 4 * I + b2;
                const bool in = r < L && i <= r;
                blk[Y::GH + r * CB_C + i] = (in && i < r) ? gh[a][b2] : 0.f;
                blk[Y::P + r * CB_C + i] = in ? pp[a][b2] : 0.f;
                sA[r][i] = (in && i < r) ? gh[a][b2] * sb[r] : 0.f;
            }
    }
    // upper-triangle pairs of A are zero
    for (int e = tid; e < CB_C * CB_C; e += 256) {
        const int r = e / CB_C, i = e % CB_C;
        if (i / 4 > r / 4) {
            sA[r][i] = 0.f;
            blk[Y::GH + e] = 0.f;
            blk[Y::P + e] = 0.f;
        }
    }
    __syncthreads();
    // M = (I + A)^-1 by forward substitution, row by row, in place over A:
    // M[r, j] = [r == j] - sum_{j <= i < r} A[r, i] M[i, j]
    for (int r = 0; r < CB_C; ++r) {
        float val = 0.f;
        if (tid < CB_C) {
            const int j = tid;
            val = (j == r) ? 1.f : 0.f;
            for (int i = j; i < r; ++i) val -= sA[r][i] * sA[i][j];
        }
        __syncthreads();
        if (tid < CB_C) sA[r][tid] = (tid <= r) ? val : 0.f;
        __syncthreads();
    }
    for (int e = tid; e < CB_C * CB_C; e += 256) {
        blk[Y::M + e] = sA[e / CB_C][e % CB_C];
        blk[Y::MT + e] = sA[e % CB_C][e / CB_C];
    }
    // W = T K~ = M Diag(beta) K~
    for (int e = tid; e < CB_C * DK; e += 256) {
        const int r = e / DK, c = e % DK;
        float acc = 0.f;
        for (int i = 0; i <= r; ++i) acc += sA[r][i] * sb[i] * sk[i][c] * __expf(sG[i][c]);
        blk[Y::W + e] = acc;
    }
}

// ------------------------------------------------------------------ scan --
// dS entering chunk c from the right (dS'), for every chunk, last first:
//     dS = Diag(g) dS' + Q~^T dO - W^T (P^T dO + K^ dS')
// One workgroup per (sequence, head, 8-column tile), 256 threads; the
// chunk's Q~, W, K^ and P are staged in LDS.
constexpr int CB_SCAN_BV = 8;
template <int DK>
struct CbScanLds {
    static constexpr int C = CB_C, BV = CB_SCAN_BV;
    static constexpr int QT = 0, W = QT + C * DK, KB = W + C * DK, P = KB + C * DK;   // [C][DK] x2, [DK][C], [C][C]
    static constexpr int DS = P + C * C;          // [DK][BV]
    static constexpr int DO = DS + DK * BV;       // [C][BV]
    static constexpr int YY = DO + C * BV;        // [C][BV]
    static constexpr int GM = YY + C * BV;        // [DK]
    static constexpr int FLOATS = GM + DK;
};

template <int DK>
__global__ void __launch_bounds__(256) cb_scan_kernel(CbParams p) {
    if (*p.status != 0) return;
    using Y = CbLay<DK>;
    using Q = CbScanLds<DK>;
    constexpr int BV = CB_SCAN_BV, C = CB_C, NT = 256;
    const int H = p.H, dv = p.dv;
    const int nvt = dv / BV;
    const int vt = blockIdx.x % nvt, h = (blockIdx.x / nvt) % H, n = blockIdx.x / (nvt * H);
    const int j0 = vt * BV;
    const int tid = threadIdx.x;
    const int64_t cbase = p.chunk_off[n];
    const int nch = p.chunk_off[n + 1] - p.chunk_off[n];

    extern __shared__ float lds[];
    float *sQ = lds + Q::QT, *sW = lds + Q::W, *sK = lds + Q::KB, *sP = lds + Q::P;
    float *sdS = lds + Q::DS, *sdO = lds + Q::DO, *sY = lds + Q::YY, *sG = lds + Q::GM;
    const int64_t sbase = (static_cast<int64_t>(n) * H + h) * DK * dv;
    for (int e = tid; e < DK * BV; e += NT) {
        const int c = e / BV, j = e % BV;
        sdS[e] = p.d_final ? p.d_final[sbase + static_cast<int64_t>(c) * dv + j0 + j] : 0.f;
    }
    for (int ch = nch - 1; ch >= 0; --ch) {
        const int64_t x = cbase + ch;
        const int4 ci = p.chunk_info[x];
        const int64_t t0 = static_cast<int64_t>(static_cast<uint32_t>(ci.x)) | (static_cast<int64_t>(ci.y) << 32);
        const int L = ci.z;
        const float *blk = p.blocks + (static_cast<size_t>(x) * H + h) * Y::FLOATS;
        __syncthreads();  // sdS complete; the previous chunk's readers are done
        float *rec = p.dS_right + (x * H + h) * static_cast<int64_t>(DK) * dv;
        for (int e = tid; e < DK * BV; e += NT) {
            const int c = e / BV, j = e % BV;
            rec[static_cast<int64_t>(c) * dv + j0 + j] = sdS[e];
        }
        for (int e = tid; e < C * DK / 4; e += NT) {
            reinterpret_cast<float4 *>(sQ)[e] = reinterpret_cast<const float4 *>(blk + Y::QT)[e];
            reinterpret_cast<float4 *>(sW)[e] = reinterpret_cast<const float4 *>(blk + Y::W)[e];
            reinterpret_cast<float4 *>(sK)[e] = reinterpret_cast<const float4 *>(blk + Y::KB)[e];
        }
        for (int e = tid; e < C * C / 4; e += NT)
            reinterpret_cast<float4 *>(sP)[e] = reinterpret_cast<const float4 *>(blk + Y::P)[e];
        for (int e = tid; e < DK; e += NT) sG[e] = blk[Y::GAM + e];
        for (int e = tid; e < C * BV; e += NT) {
            const int r = e / BV, j = e % BV;
            sdO[e] = r < L ? p.d_o[((t0 + r) * H + h) * dv + j0 + j] : 0.f;
        }
        __syncthreads();
        // Y = P^T dO + K^ dS'   (C x BV, 2 per thread)
        for (int e = tid; e < C * BV; e += NT) {
            const int r = e / BV, j = e % BV;
            float acc = 0.f;
            for (int i = r; i < C; ++i) acc += sP[i * C + r] * sdO[i * BV + j];
#pragma unroll 8
            for (int c = 0; c < DK; ++c) acc += sK[c * C + r] * sdS[c * BV + j];
            sY[e] = acc;
        }
        __syncthreads();
        // dS <- Diag(g) dS' + Q~^T dO - W^T Y   (DK x BV)
        float nv[(DK * BV + NT - 1) / NT];
#pragma unroll
        for (int m = 0; m < (DK * BV + NT - 1) / NT; ++m) {
            const int e = tid + NT * m;
            if (e >= DK * BV) continue;
            const int c = e / BV, j = e % BV;
            float acc = sG[c] * sdS[e];
#pragma unroll 8
            for (int r = 0; r < C; ++r) acc += sQ[r * DK + c] * sdO[r * BV + j] - sW[r * DK + c] * sY[r * BV + j];
            nv[m] = acc;
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < (DK * BV + NT - 1) / NT; ++m) {
            const int e = tid + NT * m;
            if (e < DK * BV) sdS[e] = nv[m];
        }
    }
    __syncthreads();
    if (p.d_initial)
        for (int e = tid; e < DK * BV; e += NT) {
            const int c = e / BV, j = e % BV;
            p.d_initial[sbase + static_cast<int64_t>(c) * dv + j0 + j] = sdS[e];
        }
}

// ------------------------------------------------------------------ grad --
// All gradients of one (chunk, head), CB_GRAD_NT threads.  The value
// dimension is walked in 16-column tiles.  Thread t keeps in registers the
// accumulators of dQ~, dK~ and dK^ for the elements e = t + NT m of the
// C x DK arrays (all in channel t mod DK) and of dP and dT for the elements
// of the C x C arrays (all in column t mod C), so the tile values of that
// channel or column are read from LDS once per tile.  The tiles are stored
// column by column with padded strides, and K~, K^ and M are staged both
// ways round where needed, so that the lanes of a wave, which take
// consecutive rows or channels, read consecutive words or one broadcast
// word.  After the walk the same LDS regions hold dT / dA, Z, dP, the
// staged decays and inputs, and dG.
constexpr int CB_GRAD_NT = 512;
template <int DK>
struct CbGradLds {
    static constexpr int C = CB_C, BV = 16;
    static constexpr int LC = C + 4, LK = DK + 4;            // padded column strides of the tiles
    static constexpr int TILE = 2 * BV * LK + 5 * BV * LC;   // S, dS' | dO, X, Delta, dDelta, dX
    static constexpr int MAT = 2 * C * C + C;                // dT -> dA, Z, dbeta
    static constexpr int U = TILE > MAT ? TILE : MAT;
    static constexpr int R1 = 0;                             // K~^T | K^^T  -> G | k, q (bf16)
    static constexpr int R2 = R1 + 2 * C * DK;               // tiles        -> dT/dA | Z/dG hi | dbeta
    static constexpr int R3 = R2 + U;                        // M | M^T | P  -> dG lo | M^T | dP
    static constexpr int AG = R3 + 3 * C * C;                // dgamma [DK]
    static constexpr int SB = AG + DK;                       // beta [C]
    static constexpr int CS = SB + C;                        // sum_r dK^ K^ [DK]
    static constexpr int FLOATS = CS + DK;
};

template <int DK, typename TI>
__global__ void __launch_bounds__(CB_GRAD_NT) cb_grad_kernel(CbParams p) {
    if (*p.status != 0) return;
    using Y = CbLay<DK>;
    using Q = CbGradLds<DK>;
    constexpr int NT = CB_GRAD_NT, BV = Q::BV, C = CB_C, LC = Q::LC, LK = Q::LK;
    constexpr int NE = C * DK / NT, NC = C * C / NT;
    constexpr int RG = NT / C, JPT = BV / RG;  // column groups and columns per thread of the row passes
    static_assert(NT % DK == 0 && NT % C == 0 && BV % RG == 0 && C == 64, "thread mapping");
    const int H = p.H, dv = p.dv;
    const int x = blockIdx.x / H, h = blockIdx.x % H;
    if (x >= p.chunk_off[p.N]) return;  // the grid covers a bound on the chunk count
    const int4 ci = p.chunk_info[x];
    const int64_t t0 = static_cast<int64_t>(static_cast<uint32_t>(ci.x)) | (static_cast<int64_t>(ci.y) << 32);
    const int L = ci.z;
    const int tid = threadIdx.x;
    const int lr = tid % C, jg = tid / C;  // row and column group of the row passes
    const int ec = tid % DK;               // channel of the C x DK accumulators
    const float *blk = p.blocks + (static_cast<size_t>(x) * H + h) * Y::FLOATS;
    const float *S = p.checkpoints + (static_cast<int64_t>(x) * H + h) * DK * dv;
    const float *dSr = p.dS_right + (static_cast<int64_t>(x) * H + h) * DK * dv;
    const TI *v = static_cast<const TI *>(p.v);

    extern __shared__ float lds[];
    float *sKt = lds + Q::R1, *sKb = sKt + C * DK;  // [DK][C]
    float *tS = lds + Q::R2, *tR = tS + BV * LK;    // [BV][LK]
    float *tO = tR + BV * LK, *tX = tO + BV * LC, *tD = tX + BV * LC, *tE = tD + BV * LC, *tF = tE + BV * LC;
    float *sM = lds + Q::R3, *sMT = sM + C * C, *sP = sMT + C * C;  // [C][C]
    float *aG = lds + Q::AG, *sB = lds + Q::SB, *sCS = lds + Q::CS;

    for (int e = tid; e < C * DK / 4; e += NT) {
        reinterpret_cast<float4 *>(sKt)[e] = reinterpret_cast<const float4 *>(blk + Y::KT)[e];
        reinterpret_cast<float4 *>(sKb)[e] = reinterpret_cast<const float4 *>(blk + Y::KB)[e];
    }
    for (int e = tid; e < C * C / 4; e += NT) {
        reinterpret_cast<float4 *>(sM)[e] = reinterpret_cast<const float4 *>(blk + Y::M)[e];
        reinterpret_cast<float4 *>(sMT)[e] = reinterpret_cast<const float4 *>(blk + Y::MT)[e];
        reinterpret_cast<float4 *>(sP)[e] = reinterpret_cast<const float4 *>(blk + Y::P)[e];
    }
    for (int e = tid; e < C; e += NT) sB[e] = blk[Y::BETA + e];
    for (int e = tid; e < DK; e += NT) aG[e] = sCS[e] = 0.f;

    float rQ[NE], rK[NE], rB[NE], rP[NC], rT[NC];
#pragma unroll
    for (int m = 0; m < NE; ++m) rQ[m] = rK[m] = rB[m] = 0.f;
#pragma unroll
    for (int m = 0; m < NC; ++m) rP[m] = rT[m] = 0.f;

    for (int j0 = 0; j0 < dv; j0 += BV) {
        __syncthreads();
        for (int e = tid; e < DK * BV; e += NT) {
            const int c = e / BV, j = e % BV;
            tS[j * LK + c] = S[static_cast<int64_t>(c) * dv + j0 + j];
            tR[j * LK + c] = dSr[static_cast<int64_t>(c) * dv + j0 + j];
        }
        for (int e = tid; e < C * BV; e += NT) {
            const int r = e / BV, j = e % BV;
            const int64_t row = (t0 + r) * H + h;
            tO[j * LC + r] = r < L ? p.d_o[row * dv + j0 + j] : 0.f;
            tF[j * LC + r] = r < L ? io<TI>::ld(v, row * dv + j0 + j) : 0.f;  // V, for X
        }
        __syncthreads();
        {   // X = V - K~ S
            float a[JPT];
#pragma unroll
            for (int u = 0; u < JPT; ++u) a[u] = tF[(jg + RG * u) * LC + lr];
#pragma unroll 8
            for (int c = 0; c < DK; ++c) {
                const float kt = sKt[c * C + lr];
#pragma unroll
                for (int u = 0; u < JPT; ++u) a[u] -= kt * tS[(jg + RG * u) * LK + c];
            }
#pragma unroll
            for (int u = 0; u < JPT; ++u) tX[(jg + RG * u) * LC + lr] = lr < L ? a[u] : 0.f;
        }
        __syncthreads();
        {   // Delta = M Diag(beta) X,  dDelta = P^T dO + K^ dS'  (the zero triangles of M, P add nothing)
            float d[JPT], dd[JPT];
#pragma unroll
            for (int u = 0; u < JPT; ++u) d[u] = dd[u] = 0.f;
#pragma unroll 8
            for (int i = 0; i < C; ++i) {
                const float t = sMT[i * C + lr] * sB[i], pv = sP[i * C + lr];
#pragma unroll
                for (int u = 0; u < JPT; ++u) {
                    d[u] += t * tX[(jg + RG * u) * LC + i];
                    dd[u] += pv * tO[(jg + RG * u) * LC + i];
                }
            }
#pragma unroll 8
            for (int c = 0; c < DK; ++c) {
                const float kb = sKb[c * C + lr];
#pragma unroll
                for (int u = 0; u < JPT; ++u) dd[u] += kb * tR[(jg + RG * u) * LK + c];
            }
#pragma unroll
            for (int u = 0; u < JPT; ++u) {
                tD[(jg + RG * u) * LC + lr] = d[u];
                tE[(jg + RG * u) * LC + lr] = dd[u];
            }
        }
        __syncthreads();
        {   // dX = Diag(beta) M^T dDelta  (= dv)
            float f[JPT];
#pragma unroll
            for (int u = 0; u < JPT; ++u) f[u] = 0.f;
#pragma unroll 8
            for (int i = 0; i < C; ++i) {
                const float mv = sM[i * C + lr];
#pragma unroll
                for (int u = 0; u < JPT; ++u) f[u] += mv * tE[(jg + RG * u) * LC + i];
            }
            const float b = sB[lr];
#pragma unroll
            for (int u = 0; u < JPT; ++u) tF[(jg + RG * u) * LC + lr] = f[u] * b;
        }
        __syncthreads();
        for (int e = tid; e < C * BV; e += NT) {
            const int r = e / BV, j = e % BV;
            if (r < L) p.gv[((t0 + r) * H + h) * dv + j0 + j] = tF[j * LC + r];
        }
        // dQ~ = dO S^T, dK~ = -dX S^T, dK^ = Delta dS'^T (channel ec);
        // dP = dO Delta^T, dT = dDelta X^T (column lr)
#pragma unroll 1
        for (int j = 0; j < BV; ++j) {
            const float sv = tS[j * LK + ec], rv = tR[j * LK + ec];
            const float *oj = tO + j * LC, *fj = tF + j * LC, *dj = tD + j * LC, *ej = tE + j * LC;
#pragma unroll
            for (int m = 0; m < NE; ++m) {
                const int r = (tid + NT * m) / DK;
                rQ[m] += oj[r] * sv;
                rK[m] -= fj[r] * sv;
                rB[m] += dj[r] * rv;
            }
            const float dvv = dj[lr], xv = tX[j * LC + lr];
#pragma unroll
            for (int m = 0; m < NC; ++m) {
                const int r = (tid + NT * m) / C;
                rP[m] += oj[r] * dvv;
                rT[m] += ej[r] * xv;
            }
        }
        for (int c = tid; c < DK; c += NT) {
            float g_ = 0.f;
#pragma unroll
            for (int j = 0; j < BV; ++j) g_ += tR[j * LK + c] * tS[j * LK + c];
            aG[c] += g_;
        }
    }
    __syncthreads();
    // T = M Diag(beta): dbeta_i = sum_r M_ri dT_ri, dM = dT Diag(beta);
    // M = (I + A)^-1: dA = -(M^T dM M^T) on the strict lower triangle;
    // A = Diag(beta) Gh: dbeta_r += sum_i dA_ri Gh_ri, dGh = Diag(beta) dA.
    float *sT = lds + Q::R2, *Z = sT + C * C, *sDB = Z + C * C;
    float *sdP = sP;  // P is dead
#pragma unroll
    for (int m = 0; m < NC; ++m) {
        sT[tid + NT * m] = rT[m];
        sdP[tid + NT * m] = rP[m];
    }
    __syncthreads();
    for (int e = tid; e < C * C; e += NT) {
        const int r = e / C, i = e % C;   // Z = M^T dM
        float acc = 0.f;
        for (int a = r; a < C; ++a) acc += sM[a * C + r] * sT[a * C + i];
        Z[e] = acc * sB[i];
    }
    for (int i = tid; i < C; i += NT) {
        float acc = 0.f;
        for (int r = i; r < C; ++r) acc += sM[r * C + i] * sT[r * C + i];
        sDB[i] = acc;
    }
    __syncthreads();
    // one row of dA per wave: dA_ri = -sum_a Z_ra M_ia, its row sum against Gh
    // goes to dbeta_r, and dGh replaces dT in place (dT is dead)
    float *sDA = sT;
    for (int e = tid; e < C * C; e += NT) {
        const int r = e / C, i = e % C;
        float acc = 0.f;
        if (i < r)
            for (int a = 0; a <= i; ++a) acc -= Z[r * C + a] * sMT[a * C + i];
        float g = acc * blk[Y::GH + e];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) g += __shfl_xor(g, o);
        if (i == 0) sDB[r] += g;
        sDA[e] = acc * sB[r];
    }
    // stage the decays and the raw q, k (bf16) for the pair sums over R1
    float *sGc = lds + Q::R1;
    uint16_t *sk16 = reinterpret_cast<uint16_t *>(sGc + C * DK), *sq16 = sk16 + C * DK;
    for (int e = tid; e < C * DK; e += NT) {
        const int r = e / DK, c = e % DK;
        const int64_t off = ((t0 + r) * H + h) * DK + c;
        sGc[e] = blk[Y::G + e];
        sk16[e] = r < L ? static_cast<const uint16_t *>(p.k)[off] : 0;
        sq16[e] = r < L ? static_cast<const uint16_t *>(p.q)[off] : 0;
    }
    __syncthreads();
    if (tid < L) p.gbeta[(t0 + tid) * H + h] = sDB[tid];
    // pair sums over the decay factors, per (row r, channel c):
    //   rowA = sum_{i<r} dGh_ri k_i e^{G_r-G_i}    rowP = sum_{i<=r} dP_ri k_i e^{G_r-G_i}
    //   colA = sum_{i>r} dGh_ir k_i e^{G_i-G_r}    colP = sum_{i>=r} dP_ir q_i e^{G_i-G_r}
    //   dk = rowA + colA + colP + dK~ e^G + dK^ e^{G_L-G},  dq = rowP + dQ~ e^G,
    //   dG = k rowA + q rowP - k (colA + colP) + dK~ K~ + dQ~ Q~ - dK^ K^
    // dG rows [0, C/2) go to M's slot, rows [C/2, C) to Z's slot (both dead)
    auto dGat = [&](int r, int c) -> float & {
        return r < C / 2 ? sM[r * DK + c] : Z[(r - C / 2) * DK + c];
    };
    float csum = 0.f;  // this thread's share of sum_r dK^ K^ (channel ec)
#pragma unroll
    for (int m = 0; m < NE; ++m) {
        const int e = tid + NT * m, r = e / DK, c = e % DK;
        const float Gr = sGc[e];
        float rowA = 0.f, rowP = 0.f, colA = 0.f, colP = 0.f;
        for (int i = 0; i < L; ++i) {
            const float ki = bf16_to_f32(sk16[i * DK + c]);
            const float Gi = sGc[i * DK + c];
            if (i <= r) {
                const float f = __expf(Gr - Gi) * ki;
                rowA += sDA[r * C + i] * f;
                rowP += sdP[r * C + i] * f;
            }
            if (i >= r) {
                const float f = __expf(Gi - Gr);
                colA += sDA[i * C + r] * ki * f;
                colP += sdP[i * C + r] * bf16_to_f32(sq16[i * DK + c]) * f;
            }
        }
        const float kr = bf16_to_f32(sk16[e]), qr = bf16_to_f32(sq16[e]);
        const float E = __expf(Gr), eL = __expf(sGc[(C - 1) * DK + c] - Gr);
        const float dk_ = rowA + colA + colP + rK[m] * E + rB[m] * eL;
        const float dq_ = rowP + rQ[m] * E;
        const float Kb = kr * eL;  // K^ and K~ as the prep kernel forms them
        dGat(r, c) = kr * rowA + qr * rowP - kr * (colA + colP) + rK[m] * (kr * E) +
                     rQ[m] * blk[Y::QT + e] - rB[m] * Kb;
        if (r < L) {
            p.gq[((t0 + r) * H + h) * DK + c] = dq_;
            p.gk[((t0 + r) * H + h) * DK + c] = dk_;
        }
        csum += rB[m] * Kb;
    }
    atomicAdd(&sCS[ec], csum);
    __syncthreads();
    // G_{C-1} (= G of the chunk's last token) also takes sum_r dK^ K^ and
    // dgamma gamma; dg = reverse cumsum of dG over the chunk
    for (int c = tid; c < DK; c += NT) {
        float run = sCS[c] + aG[c] * blk[Y::GAM + c];
        for (int r = C - 1; r >= 0; --r) {
            run += dGat(r, c);
            if (r < L) p.gg[((t0 + r) * H + h) * DK + c] = run;
        }
    }
}

namespace {
template <int DK, typename TI>
hipError_t run_cb(const CbParams &p, int n_items, hipStream_t s) {
    hipLaunchKernelGGL((cb_prep_kernel<DK, TI>), dim3(n_items), dim3(256), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    {
        const size_t lds = CbScanLds<DK>::FLOATS * sizeof(float);
        auto kern = cb_scan_kernel<DK>;
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                static_cast<int>(lds));
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(p.N) * p.H * (p.dv / CB_SCAN_BV)), dim3(256), lds, s, p);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const size_t lds = CbGradLds<DK>::FLOATS * sizeof(float);
    auto kern = cb_grad_kernel<DK, TI>;
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(lds));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(n_items), dim3(CB_GRAD_NT), lds, s, p);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_backward_chunked(const CbParams &p, int n_items, hipStream_t s) {
    switch (p.dk) {
        case 16: return run_cb<16, bf16_t>(p, n_items, s);
        case 32: return run_cb<32, bf16_t>(p, n_items, s);
        case 64: return run_cb<64, bf16_t>(p, n_items, s);
        default: return run_cb<128, bf16_t>(p, n_items, s);
    }
}

}  // namespace kda
