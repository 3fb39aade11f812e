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
// Three kernels, all in fp32 (prep on the vector ALUs, scan and grad on the
// fp32 matrix cores):
//   prep  (chunk, head):  G, K~, Q~, K^, g, Gh = k k^T e^{..}, P, M, W -> a block
//   scan  (sequence, head, 16-column tile): dS' of every chunk, last first
//   grad  (chunk, head):  every gradient of the chunk's tokens from its
//         entering state (the forward checkpoint), dS', dO and the block.
// No atomics: each chunk-head writes its own tokens' gradients.
#include <type_traits>

#include "kda_chunk_block.hpp"
#include "kda_chunk_prep.hpp"
#include "kda_launch.hpp"

namespace kda {

size_t cb_block_bytes(int dk) {
    switch (dk) {
        case 16: return CbLay<16>::FLOATS * 4;
        case 32: return CbLay<32>::FLOATS * 4;
        case 64: return CbLay<64>::FLOATS * 4;
        default: return CbLay<128>::FLOATS * 4;
    }
}

// ------------------------------------------------------------------ prep --
template <int DK, typename TI, bool FWD>
__global__ void __launch_bounds__(256) cb_prep_kernel(CbParams p) {
    if (*p.status != 0) return;
    const int x = blockIdx.x / p.H, h = blockIdx.x % p.H;
    if (x >= p.chunk_off[p.N]) return;  // the grid covers a bound on the chunk count
    cb_prep_run<DK, TI, FWD>(p, x, h);
}

// ------------------------------------------------------------------ scan --
// dS entering chunk c from the right (dS'), for every chunk, last first:
//     dS = Diag(g) dS' + Q~^T dO - W^T (P^T dO + K^ dS')
// One workgroup per (sequence, head, 16-column tile), 4 waves, on the fp32
// matrix cores (v_mfma_f32_16x16x4f32).  A 16 x 16 block product over 16
// contraction indices is four steps; in step s lane l (g = l / 16,
// n = l % 16) supplies A[n][4g + s] and B[4g + s][n] and holds
// D[4g + u][n], u = 0..3.  Wave w computes token block w of
// Y = P^T dO + K^ dS' and owns key blocks w, w + 4 of dS, which stay in
// accumulators for the whole walk.  dO, dS' and -Y pass between the waves
// through LDS, stored with the contraction index contiguous (one float4
// per lane and step group).  The chunk's operands from the prep block are
// loaded into registers one chunk ahead: P^T and K^ right after the Y
// products use them, Q~, W and the decay right after the dS products.
constexpr int CB_SCAN_BV = 16;

template <int DK>
struct CbScanOps {
    static constexpr int NKB = DK / 16;           // key blocks
    static constexpr int KPW = (NKB + 3) / 4;     // key blocks per wave
    f32x4 pt[4];          // P^T[16w + n][16ib + 4g ..] = P[16ib + 4g ..][16w + n], token blocks ib >= w
    f32x4 kb[NKB];        // K^[16w + n][16cb + 4g ..]
    f32x4 qt[KPW][4];     // Q~[16rb + 4g + s][16kb + n], s = 0..3
    f32x4 wt[KPW][4];     // W [16rb + 4g + s][16kb + n]
    f32x4 gm[KPW];        // e^{G_L}[16kb + 4g ..]
    float dov[4];         // dO of this thread's four (token, column) pairs

    __device__ __forceinline__ void load_y(const float *blk, int w, int g, int n) {
        using Y = CbLay<DK>;
#pragma unroll
        for (int ib = 0; ib < 4; ++ib)
            if (ib >= w)
#pragma unroll
                for (int s = 0; s < 4; ++s) pt[ib][s] = blk[Y::P + (16 * ib + 4 * g + s) * CB_C + 16 * w + n];
#pragma unroll
        for (int cb = 0; cb < NKB; ++cb)
            kb[cb] = *reinterpret_cast<const f32x4 *>(blk + Y::KB + (16 * w + n) * DK + 16 * cb + 4 * g);
    }
    __device__ __forceinline__ void load_s(const float *blk, int w, int g, int n) {
        using Y = CbLay<DK>;
#pragma unroll
        for (int i = 0; i < KPW; ++i) {
            const int kbk = w + 4 * i;
            if (kbk >= NKB) continue;
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int off = (16 * rb + 4 * g + s) * DK + 16 * kbk + n;
                    qt[i][rb][s] = blk[Y::QT + off];
                    wt[i][rb][s] = blk[Y::W + off];
                }
            gm[i] = *reinterpret_cast<const f32x4 *>(blk + Y::GAM + 16 * kbk + 4 * g);
        }
    }
    __device__ __forceinline__ void load_do(const float *d_o, int64_t t0, int L, int H, int h, int dv, int j0,
                                            int tid) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int e = tid + 256 * m, r = e / 16, j = e % 16;
            dov[m] = r < L ? d_o[((t0 + r) * H + h) * dv + j0 + j] : 0.f;
        }
    }
};

// 16 x 16 x 16 block product: a = A[n][4g .. 4g + 3], b = B[4g .. 4g + 3][n]
__device__ __forceinline__ f32x4 mm16x16(const f32x4 &a, const f32x4 &b, f32x4 acc) {
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], acc, 0, 0, 0);
    return acc;
}

template <int DK>
__global__ void __launch_bounds__(256) cb_scan_kernel(CbParams p) {
    if (*p.status != 0) return;
    using Y = CbLay<DK>;
    using Ops = CbScanOps<DK>;
    constexpr int BV = CB_SCAN_BV, C = CB_C, NKB = Ops::NKB, KPW = Ops::KPW;
    constexpr int LC = C + 4, LK = DK + 4;   // padded strides of the [column][row] tiles
    const int H = p.H, dv = p.dv;
    const int nvt = dv / BV;
    // XCD-aware order: the nvt column tiles of one (sequence, head) share
    // blockIdx % 8, hence one XCD and its L2, where the chunk blocks they all
    // read are shared
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int vt = slot % nvt, pair = xcd + 8 * (slot / nvt);
    if (pair >= p.N * H) return;
    const int h = pair % H, n_seq = pair / H;
    const int j0 = vt * BV;
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, n = lane & 15;
    const int64_t cbase = p.chunk_off[n_seq];
    const int nch = p.chunk_off[n_seq + 1] - p.chunk_off[n_seq];

    __shared__ __attribute__((aligned(16))) float doT[BV][LC];    // dO^T
    __shared__ __attribute__((aligned(16))) float dsT[BV][LK];    // dS'^T
    __shared__ __attribute__((aligned(16))) float ynT[BV][LC];    // -Y^T

    // the wave's key blocks of dS (accumulator layout)
    const int64_t sbase = (static_cast<int64_t>(n_seq) * H + h) * DK * dv;
    f32x4 ds[KPW];
#pragma unroll
    for (int i = 0; i < KPW; ++i) {
        const int kbk = w + 4 * i;
#pragma unroll
        for (int u = 0; u < 4; ++u)
            ds[i][u] = (kbk < NKB && p.d_final) ? p.d_final[sbase + static_cast<int64_t>(16 * kbk + 4 * g + u) * dv + j0 + n]
                                                : 0.f;
    }
    if (nch <= 0) {
        if (p.d_initial)
#pragma unroll
            for (int i = 0; i < KPW; ++i) {
                const int kbk = w + 4 * i;
                if (kbk >= NKB) continue;
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    p.d_initial[sbase + static_cast<int64_t>(16 * kbk + 4 * g + u) * dv + j0 + n] = ds[i][u];
            }
        return;
    }
    auto blk_of = [&](int ch) { return p.blocks + (static_cast<size_t>(cbase + ch) * H + h) * Y::FLOATS; };
    auto coords = [&](int ch, int64_t &t0, int &L) {
        const int4 ci = p.chunk_info[cbase + ch];
        t0 = static_cast<int64_t>(static_cast<uint32_t>(ci.x)) | (static_cast<int64_t>(ci.y) << 32);
        L = ci.z;
    };
    // L2 warm-up (as in the forward scan): while chunk ch is computed, the
    // column tiles of the head together touch every 128-byte line of the
    // block regions this scan reads (Q~, K^ and W, which are contiguous, P
    // and e^{G_L}) of chunk ch - kWarmAhead, one line per thread, so the
    // next chunk's operand loads find them in L2; the loaded word is only
    // consumed (without instructions) a chunk later.  Threads without a
    // line repeat the first one, so the load needs no branch.
    constexpr int kWarmAhead = 2;
    constexpr int kLinesA = 3 * C * DK * 4 / 128, kLinesB = C * C * 4 / 128, kLinesC = (DK * 4 + 127) / 128;
    static_assert(Y::KB == Y::QT + C * DK && Y::W == Y::KB + C * DK, "Q~, K^, W contiguous");
    const int wl = vt + nvt * tid;
    const int woff = wl < kLinesA ? static_cast<int>(Y::QT) + 32 * wl
                   : wl < kLinesA + kLinesB ? static_cast<int>(Y::P) + 32 * (wl - kLinesA)
                   : wl < kLinesA + kLinesB + kLinesC ? static_cast<int>(Y::GAM) + 32 * (wl - kLinesA - kLinesB)
                   : static_cast<int>(Y::QT);
    uint32_t warm = 0;
    auto warm_up = [&](int ch) {
        asm volatile("" ::"v"(warm));
        warm = *reinterpret_cast<const uint32_t *>(blk_of(ch > kWarmAhead ? ch - kWarmAhead : 0) + woff);
    };
    Ops op;
    {
        int64_t t0; int L;
        coords(nch - 1, t0, L);
        op.load_y(blk_of(nch - 1), w, g, n);
        op.load_s(blk_of(nch - 1), w, g, n);
        op.load_do(p.d_o, t0, L, H, h, dv, j0, tid);
    }
    for (int ch = nch - 1; ch >= 0; --ch) {
        const int64_t x = cbase + ch;
        const int nx = ch > 0 ? ch - 1 : 0;   // the chunk whose operands are loaded next
        warm_up(ch);
        lds_barrier();  // the previous chunk's readers of doT, dsT are done
        // dO and dS' -> LDS; dS' is also recorded for the gradient kernel
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int e = tid + 256 * m;
            doT[e % 16][e / 16] = op.dov[m];
        }
        float *rec = p.dS_right + (x * H + h) * static_cast<int64_t>(DK) * dv;
#pragma unroll
        for (int i = 0; i < KPW; ++i) {
            const int kbk = w + 4 * i;
            if (kbk >= NKB) continue;
            *reinterpret_cast<f32x4 *>(&dsT[n][16 * kbk + 4 * g]) = ds[i];
#pragma unroll
            for (int u = 0; u < 4; ++u) rec[static_cast<int64_t>(16 * kbk + 4 * g + u) * dv + j0 + n] = ds[i][u];
        }
        {
            int64_t t0; int L;
            coords(nx, t0, L);
            op.load_do(p.d_o, t0, L, H, h, dv, j0, tid);
        }
        lds_barrier();
        // Y block w = P^T dO + K^ dS'  (token rows 16w ..)
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ib = 0; ib < 4; ++ib)
            if (ib >= w) y = mm16x16(op.pt[ib], *reinterpret_cast<const f32x4 *>(&doT[n][16 * ib + 4 * g]), y);
#pragma unroll
        for (int cb = 0; cb < NKB; ++cb)
            y = mm16x16(op.kb[cb], *reinterpret_cast<const f32x4 *>(&dsT[n][16 * cb + 4 * g]), y);
        *reinterpret_cast<f32x4 *>(&ynT[n][16 * w + 4 * g]) = -y;
        op.load_y(blk_of(nx), w, g, n);
        lds_barrier();
        // dS = Diag(g) dS' + Q~^T dO + W^T (-Y)  (the wave's key blocks)
#pragma unroll
        for (int i = 0; i < KPW; ++i) {
            const int kbk = w + 4 * i;
            if (kbk >= NKB) continue;
            f32x4 acc = op.gm[i] * ds[i];
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                acc = mm16x16(op.qt[i][rb], *reinterpret_cast<const f32x4 *>(&doT[n][16 * rb + 4 * g]), acc);
                acc = mm16x16(op.wt[i][rb], *reinterpret_cast<const f32x4 *>(&ynT[n][16 * rb + 4 * g]), acc);
            }
            ds[i] = acc;
        }
        op.load_s(blk_of(nx), w, g, n);
    }
    asm volatile("" ::"v"(warm));
    if (p.d_initial)
#pragma unroll
        for (int i = 0; i < KPW; ++i) {
            const int kbk = w + 4 * i;
            if (kbk >= NKB) continue;
#pragma unroll
            for (int u = 0; u < 4; ++u)
                p.d_initial[sbase + static_cast<int64_t>(16 * kbk + 4 * g + u) * dv + j0 + n] = ds[i][u];
        }
}

// ------------------------------------------------------------------ grad --
// All gradients of one (chunk, head): 512 threads (8 waves) on the fp32
// matrix cores (v_mfma_f32_16x16x4f32: fp32 products, fp32 sums).  A 16 x 16
// block product over 16 contraction indices is four such steps; in step s
// lane l (g = l / 16, n = l % 16) supplies A[n][4g + s] and B[4g + s][n],
// and D[4g + u][n] (u = 0..3) is the lane's u-th accumulator.  Operands are
// stored with the contraction index contiguous, so a lane reads the values
// of its four steps as one float4.
//
// The value dimension is walked in 16-column tiles.  Per tile, with R the
// wave's 16-row block (wave mod 4):
//   waves 0-3:  X = V - K~ S,            then Delta = M Diag(beta) X
//   waves 4-7:  dDelta = P^T dO + K^ dS', then dX = Diag(beta) M^T dDelta  (= dv)
//   all waves:  dQ~ += dO S^T, dK~ -= dX S^T, dK^ += Delta dS'^T  (C x DK, half
//               the key blocks each), dP += dO Delta^T, dT += dDelta X^T
//               (C x C, blocks on or below the diagonal)
// The left operands of the first two steps (K~, K^, M Diag(beta), P^T,
// Diag(beta) M^T) are fixed for the chunk and stay in registers for the
// whole walk; the triangular ones skip their zero blocks.  After the walk
// the LDS holds dT -> dA, Z, dP, M, M^T, the staged decays and inputs, and
// dG.  No atomics reach global memory: each chunk-head writes its own
// tokens' gradients.
constexpr int CB_GRAD_NT = 512;
template <int DK>
struct CbGradLds {
    static constexpr int C = CB_C, BV = 16;
    static constexpr int LB = BV + 4;  // row stride of the [row][j] tiles
    static constexpr int LC = C + 4;   // column stride of the [j][row] tiles of C rows
    static constexpr int LK = DK + 4;  // column stride of the [j][row] tiles of DK rows
    static constexpr int LA = C + 1;   // row stride of dT / dA and dP
    // the walk: S, dS' as [DK][LB] and [BV][LK]; dO, X, Delta, dDelta, dX as
    // [C][LB]; dO, X, dDelta also as [BV][LC]
    static constexpr int SR = 0, RR = SR + DK * LB, SC = RR + DK * LB, RC = SC + BV * LK;
    static constexpr int OR = RC + BV * LK, XR = OR + C * LB, DR = XR + C * LB, ER = DR + C * LB;
    static constexpr int FR = ER + C * LB, OC = FR + C * LB, XC = OC + BV * LC, EC = XC + BV * LC;
    static constexpr int WALK = EC + BV * LC;
    // after the walk
    static constexpr int LM = C + 4;            // row stride of M, M^T and Z
    static constexpr int GC = 0;                // G [C][DK], then k and q (bf16) [C][DK] each
    static constexpr int TA = GC + 2 * C * DK;  // dT -> dGh [C][LA]
    static constexpr int ZZ = TA + C * LA;      // Z [C][LM]  -> dG rows [C/2, C)
    static constexpr int DB = ZZ + C * LM;      // dbeta [C]
    static constexpr int MM = DB + C;           // M [C][LM]  -> dG rows [0, C/2)
    static constexpr int MTT = MM + C * LM;     // M^T [C][LM]
    static constexpr int DP = MTT + C * LM;     // dP [C][LA]
    static_assert(C / 2 * DK <= C * LM, "dG halves fit the M and Z slots");
    static constexpr int POST = DP + C * LA;
    static constexpr int BASE = WALK > POST ? WALK : POST;
    static constexpr int AG = BASE;             // dgamma [DK]
    static constexpr int SB = AG + DK;          // beta [C]
    static constexpr int PD = SB + C;           // diagonal of dP [C]
    static constexpr int DBP = PD + C;          // dbeta partial sums [C][4 key blocks]
    static constexpr int FLOATS = DBP + 4 * C;
};

__device__ __forceinline__ f32x4 mfma4(float a0, float a1, float a2, float a3, const float4 &b, f32x4 acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, b.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, b.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a2, b.z, acc, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a3, b.w, acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma4(const float4 &a, const float4 &b, f32x4 acc) {
    return mfma4(a.x, a.y, a.z, a.w, b, acc);
}
__device__ __forceinline__ float4 ld4(const float *p) { return *reinterpret_cast<const float4 *>(p); }
__device__ __forceinline__ float wave_max_f(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
    return x;
}
// Diagonal blocks of the pair sums are split around the midpoint of their
// own decay while the largest decay over the block (in nats, over the
// wave's 16 channels) stays below this; beyond it they are summed pair by
// pair.  e^32 keeps the split factors far from fp32 overflow.
constexpr float kCbSpanMax = 64.f;

template <int DK, typename TI>
__global__ void __launch_bounds__(CB_GRAD_NT) cb_grad_kernel(CbParams p) {
    if (*p.status != 0) return;
    using Y = CbLay<DK>;
    using Q = CbGradLds<DK>;
    constexpr int NT = CB_GRAD_NT, BV = Q::BV, C = CB_C, LB = Q::LB, LC = Q::LC, LK = Q::LK, LA = Q::LA, LM = Q::LM;
    constexpr int NKB = DK / 16;        // 16-wide blocks of the key dimension
    constexpr int NCW = (NKB + 1) / 2;  // key blocks per wave in the C x DK products
    static_assert(NT == 512 && C == 64 && BV == 16, "wave roles: 8 waves, 4 row blocks of 16, 16 columns");
    const int H = p.H, dv = p.dv;
    const int x = blockIdx.x / H, h = blockIdx.x % H;
    if (x >= p.chunk_off[p.N]) return;  // the grid covers a bound on the chunk count
    const int4 ci = p.chunk_info[x];
    const int64_t t0 = static_cast<int64_t>(static_cast<uint32_t>(ci.x)) | (static_cast<int64_t>(ci.y) << 32);
    const int L = ci.z;
    const int tid = threadIdx.x, lane = tid % 64, wv = tid / 64;
    const int g = lane / 16, n = lane % 16;
    const int R = wv % 4, half = wv / 4;
    const float *blk = p.blocks + (static_cast<size_t>(x) * H + h) * Y::FLOATS;
    const float *S = p.checkpoints + (static_cast<int64_t>(x) * H + h) * DK * dv;
    const float *dSr = p.dS_right + (static_cast<int64_t>(x) * H + h) * DK * dv;
    const TI *v = static_cast<const TI *>(p.v);

    extern __shared__ float lds[];
    float *tSr = lds + Q::SR, *tRr = lds + Q::RR, *tSc = lds + Q::SC, *tRc = lds + Q::RC;
    float *tOr = lds + Q::OR, *tXr = lds + Q::XR, *tDr = lds + Q::DR, *tEr = lds + Q::ER, *tFr = lds + Q::FR;
    float *tOc = lds + Q::OC, *tXc = lds + Q::XC, *tEc = lds + Q::EC;
    float *aG = lds + Q::AG, *sB = lds + Q::SB, *sPD = lds + Q::PD;

    // A tile's S, dS' and dO vectors (thread e: row e / (BV/4), columns
    // 4 (e % (BV/4)) ..) and the V values of waves 0-3 are loaded into
    // registers one tile ahead, unconditionally (rows clamped, surplus values
    // unused); the walk's barriers are LDS-only, so these loads and the dv
    // stores stay in flight across them.
    static_assert(DK * BV / 4 <= NT && C * BV / 4 <= NT, "one vector per thread and tile");
    const int er = tid / (BV / 4), ejq = 4 * (tid % (BV / 4));
    const bool has_s = tid < DK * BV / 4, has_o = tid < C * BV / 4;
    float4 nsv, nrv, nov;
    float nvv[4];
    auto load_tile = [&](int j0) {
        const int c = has_s ? er : 0;
        nsv = ld4(S + static_cast<int64_t>(c) * dv + j0 + ejq);
        nrv = ld4(dSr + static_cast<int64_t>(c) * dv + j0 + ejq);
        nov = ld4(p.d_o + ((t0 + min(er, L - 1)) * H + h) * dv + j0 + ejq);
#pragma unroll
        for (int u = 0; u < 4; ++u)
            nvv[u] = io<TI>::ld(v, ((t0 + min(R * 16 + 4 * g + u, L - 1)) * H + h) * dv + j0 + n);
    };
    load_tile(0);   // in flight with the fixed operands' loads below

    // the fixed left operands, row R*16 + n, contraction indices 16 kb + 4g + s:
    //   waves 0-3: fa = -K~, fb = M Diag(beta);  waves 4-7: fa = K^, fb = P^T, fc = Diag(beta) M^T
    float fa[4 * NKB], fb[16], fc[16];
    {
        const int row = R * 16 + n;
        const float *ka = blk + (half ? Y::KB : Y::KT) + row * DK;
        const float sg = half ? 1.f : -1.f;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            const float4 t = ld4(ka + kb * 16 + 4 * g);
            fa[4 * kb] = sg * t.x; fa[4 * kb + 1] = sg * t.y; fa[4 * kb + 2] = sg * t.z; fa[4 * kb + 3] = sg * t.w;
        }
        // P^T and M^T rows are P and M columns
        const float *mc = blk + Y::M + row;
        const float br = blk[Y::BETA + row];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            if (half) {
#pragma unroll
                for (int s = 0; s < 4; ++s) fb[4 * kb + s] = blk[Y::P + (kb * 16 + 4 * g + s) * C + row];
            } else {
                const float4 t = ld4(blk + Y::M + row * C + kb * 16 + 4 * g);
                const float4 bc = ld4(blk + Y::BETA + kb * 16 + 4 * g);
                fb[4 * kb] = t.x * bc.x; fb[4 * kb + 1] = t.y * bc.y; fb[4 * kb + 2] = t.z * bc.z; fb[4 * kb + 3] = t.w * bc.w;
            }
#pragma unroll
            for (int s = 0; s < 4; ++s) fc[4 * kb + s] = br * mc[(kb * 16 + 4 * g + s) * C];
        }
    }
    for (int e = tid; e < DK; e += NT) aG[e] = 0.f;

    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    f32x4 aQ[NCW], aK[NCW], aB[NCW], aP[2], aT[2];
#pragma unroll
    for (int t = 0; t < NCW; ++t) aQ[t] = aK[t] = aB[t] = z4;
    aP[0] = aP[1] = aT[0] = aT[1] = z4;

    for (int j0 = 0; j0 < dv; j0 += BV) {
        lds_barrier();  // the previous tile's readers are done
        if (has_s) {
            const int c = er, jq = ejq;
            const float4 sv = nsv, rv = nrv;
            *reinterpret_cast<float4 *>(tSr + c * LB + jq) = sv;
            *reinterpret_cast<float4 *>(tRr + c * LB + jq) = rv;
            tSc[jq * LK + c] = sv.x; tSc[(jq + 1) * LK + c] = sv.y; tSc[(jq + 2) * LK + c] = sv.z; tSc[(jq + 3) * LK + c] = sv.w;
            tRc[jq * LK + c] = rv.x; tRc[(jq + 1) * LK + c] = rv.y; tRc[(jq + 2) * LK + c] = rv.z; tRc[(jq + 3) * LK + c] = rv.w;
        }
        if (has_o) {
            const int r = er, jq = ejq;
            const float4 ov = r < L ? nov : make_float4(0.f, 0.f, 0.f, 0.f);
            *reinterpret_cast<float4 *>(tOr + r * LB + jq) = ov;
            tOc[jq * LC + r] = ov.x; tOc[(jq + 1) * LC + r] = ov.y; tOc[(jq + 2) * LC + r] = ov.z; tOc[(jq + 3) * LC + r] = ov.w;
        }
        float vv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) vv[u] = R * 16 + 4 * g + u < L ? nvv[u] : 0.f;
        load_tile(j0 + BV < dv ? j0 + BV : j0);
        lds_barrier();
        if (half == 0) {  // X = V - K~ S
            f32x4 acc;
#pragma unroll
            for (int u = 0; u < 4; ++u) acc[u] = vv[u];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
                acc = mfma4(fa[4 * kb], fa[4 * kb + 1], fa[4 * kb + 2], fa[4 * kb + 3], ld4(tSc + n * LK + kb * 16 + 4 * g), acc);
            *reinterpret_cast<float4 *>(tXc + n * LC + R * 16 + 4 * g) = make_float4(acc[0], acc[1], acc[2], acc[3]);
#pragma unroll
            for (int u = 0; u < 4; ++u) tXr[(R * 16 + 4 * g + u) * LB + n] = acc[u];
        } else {  // dDelta = P^T dO + K^ dS'
            f32x4 acc = z4;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
                if (kb >= R)
                    acc = mfma4(fb[4 * kb], fb[4 * kb + 1], fb[4 * kb + 2], fb[4 * kb + 3], ld4(tOc + n * LC + kb * 16 + 4 * g), acc);
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
                acc = mfma4(fa[4 * kb], fa[4 * kb + 1], fa[4 * kb + 2], fa[4 * kb + 3], ld4(tRc + n * LK + kb * 16 + 4 * g), acc);
            *reinterpret_cast<float4 *>(tEc + n * LC + R * 16 + 4 * g) = make_float4(acc[0], acc[1], acc[2], acc[3]);
#pragma unroll
            for (int u = 0; u < 4; ++u) tEr[(R * 16 + 4 * g + u) * LB + n] = acc[u];
        }
        lds_barrier();
        if (half == 0) {  // Delta = M Diag(beta) X
            f32x4 acc = z4;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
                if (kb <= R)
                    acc = mfma4(fb[4 * kb], fb[4 * kb + 1], fb[4 * kb + 2], fb[4 * kb + 3], ld4(tXc + n * LC + kb * 16 + 4 * g), acc);
#pragma unroll
            for (int u = 0; u < 4; ++u) tDr[(R * 16 + 4 * g + u) * LB + n] = acc[u];
        } else {  // dX = Diag(beta) M^T dDelta
            f32x4 acc = z4;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
                if (kb >= R)
                    acc = mfma4(fc[4 * kb], fc[4 * kb + 1], fc[4 * kb + 2], fc[4 * kb + 3], ld4(tEc + n * LC + kb * 16 + 4 * g), acc);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int r = R * 16 + 4 * g + u;
                tFr[r * LB + n] = acc[u];
                if (r < L) p.gv[((t0 + r) * H + h) * dv + j0 + n] = acc[u];
            }
        }
        lds_barrier();
        {   // the products over this tile's 16 columns
            const float4 aO = ld4(tOr + (R * 16 + n) * LB + 4 * g);
            const float4 aF = ld4(tFr + (R * 16 + n) * LB + 4 * g);
            const float4 aD = ld4(tDr + (R * 16 + n) * LB + 4 * g);
            const float4 aE = ld4(tEr + (R * 16 + n) * LB + 4 * g);
#pragma unroll
            for (int t = 0; t < NCW; ++t) {
                const int cb = half + 2 * t;
                if (cb < NKB) {
                    const float4 bS = ld4(tSr + (cb * 16 + n) * LB + 4 * g);
                    const float4 bR = ld4(tRr + (cb * 16 + n) * LB + 4 * g);
                    aQ[t] = mfma4(aO, bS, aQ[t]);
                    aK[t] = mfma4(aF, bS, aK[t]);
                    aB[t] = mfma4(aD, bR, aB[t]);
                }
            }
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int ib = half + 2 * t;
                if (ib <= R) {
                    aP[t] = mfma4(aO, ld4(tDr + (ib * 16 + n) * LB + 4 * g), aP[t]);
                    aT[t] = mfma4(aE, ld4(tXr + (ib * 16 + n) * LB + 4 * g), aT[t]);
                }
            }
        }
        for (int c = tid; c < DK; c += NT) {
            float g_ = 0.f;
#pragma unroll
            for (int j = 0; j < BV; ++j) g_ += tRr[c * LB + j] * tSr[c * LB + j];
            aG[c] += g_;
        }
    }
    // G, k and q of the chunk for the pair sums, requested now (the walk's
    // fixed operands are dead) as 16-byte vectors, staged in LDS once Z is
    // formed, so the transfers overlap the dT / M staging and the Z products
    constexpr int NG4 = (C * DK / 4 + NT - 1) / NT, NQ8 = (C * DK / 8 + NT - 1) / NT;
    typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
    const bool kq_vec = ((reinterpret_cast<uintptr_t>(p.k) | reinterpret_cast<uintptr_t>(p.q)) & 15) == 0;
    float4 gpre[NG4];
    u32x4 kpre[NQ8], qpre[NQ8];
#pragma unroll
    for (int i = 0; i < NG4; ++i) gpre[i] = ld4(blk + Y::G + 4 * min(tid + NT * i, C * DK / 4 - 1));
    if (kq_vec) {
#pragma unroll
        for (int i = 0; i < NQ8; ++i) {
            const int e = 8 * min(tid + NT * i, C * DK / 8 - 1), r = e / DK, c0 = e % DK;
            const int64_t off = ((t0 + min(r, L - 1)) * H + h) * DK + c0;
            kpre[i] = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(p.k) + off);
            qpre[i] = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(p.q) + off);
        }
    }
    lds_barrier();  // the tiles are dead
    float *sGc = lds + Q::GC;
    uint16_t *sk16 = reinterpret_cast<uint16_t *>(sGc + C * DK), *sq16 = sk16 + C * DK;
    float *sT = lds + Q::TA, *Z = lds + Q::ZZ, *sDB = lds + Q::DB, *sM = lds + Q::MM, *sMT = lds + Q::MTT;
    float *sdP = lds + Q::DP, *sDBP = lds + Q::DBP;
    // dT on and below the diagonal, dP strictly below it with its diagonal
    // apart; the rest is zero
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int ib = half + 2 * t;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int o = (R * 16 + 4 * g + u) * LA + ib * 16 + n;
            const bool low = ib < R || (ib == R && n <= 4 * g + u), diag = ib == R && n == 4 * g + u;
            sdP[o] = low && !diag ? aP[t][u] : 0.f;
            sT[o] = low ? aT[t][u] : 0.f;
            if (diag) sPD[R * 16 + n] = aP[t][u];
        }
    }
    for (int e = tid; e < C * C / 4; e += NT) {
        const int r = e / (C / 4), a4 = 4 * (e % (C / 4));
        const float4 t = ld4(blk + Y::M + r * C + a4);
        *reinterpret_cast<float4 *>(sM + r * LM + a4) = t;
        sMT[a4 * LM + r] = t.x;
        sMT[(a4 + 1) * LM + r] = t.y;
        sMT[(a4 + 2) * LM + r] = t.z;
        sMT[(a4 + 3) * LM + r] = t.w;
    }
    for (int e = tid; e < C; e += NT) sB[e] = blk[Y::BETA + e];
    lds_barrier();
    // T = M Diag(beta): dM = dT Diag(beta), dbeta_i = (M^T dT)_ii;
    // M = (I + A)^-1: dA = -(M^T dM M^T) on the strict lower triangle;
    // A = Diag(beta) Gh: dbeta_r += sum_i dA_ri Gh_ri, dGh = Diag(beta) dA.
    // Z = M^T dT Diag(beta): blocks (R, ib <= R), M^T upper: a from block R on
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int ib = half + 2 * t;
        if (ib > R) break;
        f32x4 acc = z4;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            if (kb < R) continue;
            const float *bt = sT + (kb * 16 + 4 * g) * LA + ib * 16 + n;
            acc = mfma4(ld4(sMT + (R * 16 + n) * LM + kb * 16 + 4 * g),
                        make_float4(bt[0], bt[LA], bt[2 * LA], bt[3 * LA]), acc);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int r = R * 16 + 4 * g + u, i = ib * 16 + n;
            Z[r * LM + i] = acc[u] * sB[i];
            if (i == r) sDB[r] = acc[u];
        }
    }
    // stage the decays and the raw q, k (bf16) for the pair sums
#pragma unroll
    for (int i = 0; i < NG4; ++i)
        if (tid + NT * i < C * DK / 4) *reinterpret_cast<float4 *>(sGc + 4 * (tid + NT * i)) = gpre[i];
    if (kq_vec) {
        const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < NQ8; ++i) {
            if (tid + NT * i >= C * DK / 8) continue;
            const int e = 8 * (tid + NT * i), r = e / DK;
            *reinterpret_cast<u32x4 *>(sk16 + e) = r < L ? kpre[i] : zero;
            *reinterpret_cast<u32x4 *>(sq16 + e) = r < L ? qpre[i] : zero;
        }
    } else {
        for (int e = tid; e < C * DK; e += NT) {
            const int r = e / DK, c = e % DK;
            const int64_t off = ((t0 + r) * H + h) * DK + c;
            sk16[e] = r < L ? static_cast<const uint16_t *>(p.k)[off] : 0;
            sq16[e] = r < L ? static_cast<const uint16_t *>(p.q)[off] : 0;
        }
    }
    lds_barrier();
    // dA = -Z M^T, blocks (R, ib <= R), M lower: a up to block ib; strict
    // lower triangle only.  dGh = Diag(beta) dA replaces dT.
    float *sDA = sT;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int ib = half + 2 * t;
        if (ib > R) break;
        f32x4 acc = z4;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            if (kb > ib) break;
            acc = mfma4(ld4(Z + (R * 16 + n) * LM + kb * 16 + 4 * g), ld4(sM + (ib * 16 + n) * LM + kb * 16 + 4 * g), acc);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int r = R * 16 + 4 * g + u, i = ib * 16 + n;
            const float dA = i < r ? -acc[u] : 0.f;
            float gs = dA * blk[Y::GH + r * C + i];
#pragma unroll
            for (int o = 8; o > 0; o >>= 1) gs += __shfl_xor(gs, o);  // over the 16 columns
            if (n == 0) sDBP[r * 4 + ib] = gs;  // summed below in a fixed order
            sDA[r * LA + i] = dA * sB[r];
        }
    }
    lds_barrier();
    if (tid < L) {  // blocks ib <= the row's own block, in order
        float db = sDB[tid];
        for (int ib = 0; ib <= tid / 16; ++ib) db += sDBP[tid * 4 + ib];
        p.gbeta[(t0 + tid) * H + h] = db;
    }
    // pair sums over the decay factors, per (row r, channel c):
    //   rowA = sum_{i<r} dGh_ri k_i e^{G_r-G_i}    rowP = sum_{i<r} dP_ri k_i e^{G_r-G_i}
    //   colA = sum_{i>r} dGh_ir k_i e^{G_i-G_r}    colP = sum_{i>r} dP_ir q_i e^{G_i-G_r}
    //   dk = rowA + colA + colP + dP_rr q + dK~ e^G + dK^ e^{G_L-G},
    //   dq = rowP + dP_rr k + dQ~ e^G,
    //   dg_t = sum_{r>=t} dG_r + sum_{r<t} dK^_r K^_r + dgamma gamma,
    //   dG = k rowA + q rowP - k (colA + colP) + dK~ K~ + dQ~ Q~.
    // (G_L - G_r depends on g_t for r < t <= L: summing dK^ K^ forwards
    // avoids adding it at the chunk's end and taking it back row by row,
    // which cancels to fp32 noise when the chunk decays strongly; the
    // diagonal pairs of P leave dG for the same reason.)
    // For the lane's accumulator elements (R*16 + 4g + u, cb*16 + n), on the
    // matrix cores.  The decay factor of a pair is split around a reference
    // row: for rows against earlier blocks the row before block R,
    // e^{G_r-G_i} = e^{G_r-G_m} e^{G_m-G_i}; for columns against later blocks
    // the last row of block R, e^{G_i-G_r} = e^{G_i-G_e} e^{G_e-G_r}; all four
    // factors are <= 1.  Within block R the split is around the midpoint of
    // the block's decay (factors within e^(+-span/2)), or, where some channel
    // of the wave decays by more than kCbSpanMax over the block, pair by pair.
    // dG rows [0, C/2) go to M's slot, rows [C/2, C) to Z's slot (both dead);
    // dK^ K^ stays in registers until the staged inputs are dead.
    auto dGat = [&](int r, int c) -> float & {
        return r < C / 2 ? sM[r * DK + c] : Z[(r - C / 2) * DK + c];
    };
    float vKK[NCW][4];
#pragma unroll
    for (int t = 0; t < NCW; ++t) {
        const int cb = half + 2 * t;
        if (cb >= NKB) break;
        const int c = cb * 16 + n;
        const float Gm = R > 0 ? sGc[(R * 16 - 1) * DK + c] : 0.f;
        const float Ge = sGc[(R * 16 + 15) * DK + c];
        const float Gmid = 0.5f * (Gm + Ge);
        const bool exact = wave_max_f(Gm - Ge) > kCbSpanMax;
        f32x4 rA = z4, rP = z4, cA = z4, cP = z4, dRA = z4, dRP = z4, dCA = z4, dCP = z4;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            if (b == R && exact) continue;
            const float ref = b < R ? Gm : b > R ? Ge : Gmid;
            float bk[4], bq[4], brow[4], a0[4], a1[4], a2[4], a3[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int i = b * 16 + 4 * g + s;
                const float Gi = sGc[i * DK + c];
                const float ki = bf16_to_f32(sk16[i * DK + c]);
                const float ec = __expf(Gi - ref);            // columns: e^{G_i - ref}
                brow[s] = b <= R ? ki * __expf(ref - Gi) : 0.f;  // rows: e^{ref - G_i}
                bk[s] = ki * ec;
                bq[s] = bf16_to_f32(sq16[i * DK + c]) * ec;
                a0[s] = sDA[(R * 16 + n) * LA + i];   // dGh[r][i]
                a1[s] = sdP[(R * 16 + n) * LA + i];   // dP[r][i]
                a2[s] = sDA[i * LA + R * 16 + n];     // dGh[i][r]
                a3[s] = sdP[i * LA + R * 16 + n];     // dP[i][r]
            }
            const float4 Br = make_float4(brow[0], brow[1], brow[2], brow[3]);
            const float4 Bk = make_float4(bk[0], bk[1], bk[2], bk[3]);
            const float4 Bq = make_float4(bq[0], bq[1], bq[2], bq[3]);
            if (b < R) {
                rA = mfma4(a0[0], a0[1], a0[2], a0[3], Br, rA);
                rP = mfma4(a1[0], a1[1], a1[2], a1[3], Br, rP);
            } else if (b > R) {
                cA = mfma4(a2[0], a2[1], a2[2], a2[3], Bk, cA);
                cP = mfma4(a3[0], a3[1], a3[2], a3[3], Bq, cP);
            } else {
                dRA = mfma4(a0[0], a0[1], a0[2], a0[3], Br, dRA);
                dRP = mfma4(a1[0], a1[1], a1[2], a1[3], Br, dRP);
                dCA = mfma4(a2[0], a2[1], a2[2], a2[3], Bk, dCA);
                dCP = mfma4(a3[0], a3[1], a3[2], a3[3], Bq, dCP);
            }
        }
        const float GL = sGc[(C - 1) * DK + c];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int r = R * 16 + 4 * g + u;
            const float Gr = sGc[r * DK + c];
            float rowA = rA[u] * __expf(Gr - Gm), rowP = rP[u] * __expf(Gr - Gm);
            float colA = cA[u] * __expf(Ge - Gr), colP = cP[u] * __expf(Ge - Gr);
            if (!exact) {
                const float fr = __expf(Gr - Gmid), fc = __expf(Gmid - Gr);
                rowA += dRA[u] * fr;
                rowP += dRP[u] * fr;
                colA += dCA[u] * fc;
                colP += dCP[u] * fc;
            } else {
                for (int i = R * 16; i < R * 16 + 16; ++i) {
                    const float ki = bf16_to_f32(sk16[i * DK + c]);
                    const float Gi = sGc[i * DK + c];
                    if (i <= r) {
                        const float f = __expf(Gr - Gi) * ki;
                        rowA += sDA[r * LA + i] * f;
                        rowP += sdP[r * LA + i] * f;
                    }
                    if (i >= r) {
                        const float f = __expf(Gi - Gr);
                        colA += sDA[i * LA + r] * ki * f;
                        colP += sdP[i * LA + r] * bf16_to_f32(sq16[i * DK + c]) * f;
                    }
                }
            }
            const float kr = bf16_to_f32(sk16[r * DK + c]), qr = bf16_to_f32(sq16[r * DK + c]);
            const float E = __expf(Gr), eL = __expf(GL - Gr), pd = sPD[r];
            const float rq = aQ[t][u], rk = -aK[t][u], rb = aB[t][u];
            dGat(r, c) = kr * rowA + qr * rowP - kr * (colA + colP) + rk * (kr * E) + rq * blk[Y::QT + r * DK + c];
            vKK[t][u] = rb * (kr * eL);  // K^ and K~ as the prep kernel forms them
            if (r < L) {
                p.gq[((t0 + r) * H + h) * DK + c] = rowP + pd * kr + rq * E;
                p.gk[((t0 + r) * H + h) * DK + c] = rowA + colA + colP + pd * qr + rk * E + rb * eL;
            }
        }
    }
    lds_barrier();  // the staged decays and inputs are dead
    float *sKK = lds + Q::GC;
#pragma unroll
    for (int t = 0; t < NCW; ++t) {
        const int cb = half + 2 * t;
        if (cb >= NKB) break;
#pragma unroll
        for (int u = 0; u < 4; ++u) sKK[(R * 16 + 4 * g + u) * DK + cb * 16 + n] = vKK[t][u];
    }
    lds_barrier();
    // dg: per channel the reverse cumulative sum of dG plus the forward
    // exclusive sum of dK^ K^ and dgamma gamma, on every token.  A channel's
    // rows are split into NSEG segments over all the threads: the segment
    // sums meet in LDS (the dead k, q staging), then each thread runs its
    // own rows.  (Rows >= L contribute zeros to both sums.)
    {
        constexpr int NSEG = NT / DK, RPS = C / NSEG;   // segments per channel, rows per segment
        static_assert(NSEG * DK == NT && RPS * NSEG == C && 2 * NT <= C * DK, "segments tile the chunk");
        float *segG = lds + Q::GC + C * DK, *segK = segG + NT;
        const int c = tid % DK, sgi = tid / DK, r0 = sgi * RPS;
        float sgs = 0.f, sks = 0.f;
#pragma unroll
        for (int i = 0; i < RPS; ++i) {
            sgs += dGat(r0 + i, c);
            sks += sKK[(r0 + i) * DK + c];
        }
        segG[sgi * DK + c] = sgs;
        segK[sgi * DK + c] = sks;
        lds_barrier();
        float run = 0.f, pre = aG[c] * blk[Y::GAM + c];
        for (int u = 0; u < NSEG; ++u) {
            if (u > sgi) run += segG[u * DK + c];
            if (u < sgi) pre += segK[u * DK + c];
        }
        float val[RPS];
#pragma unroll
        for (int i = RPS - 1; i >= 0; --i) {
            run += dGat(r0 + i, c);
            val[i] = run;
        }
#pragma unroll
        for (int i = 0; i < RPS; ++i) {
            const int r = r0 + i;
            if (r < L) p.gg[((t0 + r) * H + h) * DK + c] = val[i] + pre;
            pre += sKK[r * DK + c];
        }
    }
}

namespace {
template <int DK, typename TI>
hipError_t run_cb(const CbParams &p, int n_items, hipStream_t s) {
    hipLaunchKernelGGL((cb_prep_kernel<DK, TI, false>), dim3(n_items), dim3(256), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned pairs8 = static_cast<unsigned>((p.N * p.H + 7) / 8);
    hipLaunchKernelGGL((cb_scan_kernel<DK>), dim3(pairs8 * 8 * (p.dv / CB_SCAN_BV)), dim3(256), 0, s, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t lds = CbGradLds<DK>::FLOATS * sizeof(float);
    auto kern = cb_grad_kernel<DK, TI>;
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(lds));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(n_items), dim3(CB_GRAD_NT), lds, s, p);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_chunk_prep_fwd(const CbParams &p, int n_items, int in_dtype, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(n_items)), block(256);
    if (in_dtype == 0) {
        switch (p.dk) {
            case 16: hipLaunchKernelGGL((cb_prep_kernel<16, float, true>), grid, block, 0, s, p); break;
            case 32: hipLaunchKernelGGL((cb_prep_kernel<32, float, true>), grid, block, 0, s, p); break;
            case 64: hipLaunchKernelGGL((cb_prep_kernel<64, float, true>), grid, block, 0, s, p); break;
            default: hipLaunchKernelGGL((cb_prep_kernel<128, float, true>), grid, block, 0, s, p); break;
        }
    } else {
        switch (p.dk) {
            case 16: hipLaunchKernelGGL((cb_prep_kernel<16, bf16_t, true>), grid, block, 0, s, p); break;
            case 32: hipLaunchKernelGGL((cb_prep_kernel<32, bf16_t, true>), grid, block, 0, s, p); break;
            case 64: hipLaunchKernelGGL((cb_prep_kernel<64, bf16_t, true>), grid, block, 0, s, p); break;
            default: hipLaunchKernelGGL((cb_prep_kernel<128, bf16_t, true>), grid, block, 0, s, p); break;
        }
    }
    return hipGetLastError();
}

hipError_t launch_backward_chunked(const CbParams &p, int n_items, hipStream_t s) {
    switch (p.dk) {
        case 16: return run_cb<16, bf16_t>(p, n_items, s);
        case 32: return run_cb<32, bf16_t>(p, n_items, s);
        case 64: return run_cb<64, bf16_t>(p, n_items, s);
        default: return run_cb<128, bf16_t>(p, n_items, s);
    }
}

}  // namespace kda
