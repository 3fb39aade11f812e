// Matrix-core chunked KDA prefill for bf16 inputs, d_k = d_v = D in {64, 128},
// chunk C in {16, 32, 64}; fp32 state and accumulation.
//
// The chunk decomposition follows Module 04 — KDA II: Chunked Parallelism &
// the Full Sublayer, §1 "The recurrence has affine form": each chunk's
// composed transition is built independently of the incoming state, in
// structured form (per-channel decay plus a rank-L correction, never a dense
// d_k x d_k matrix), and the chunks are then applied in order (§2: prefill
// uses a chunked kernel).  For a chunk of L tokens with incoming state S and
// cumulative log-decay G_r = sum_{i<=r} log_alpha_i (per channel):
//   A_ri = beta_r sum_c k_r[c] k_i[c] e^{G_r[c]-G_i[c]}   (i < r)
//   P_ri =        sum_c q_r[c] k_i[c] e^{G_r[c]-G_i[c]}   (i <= r)
//   T = (I + A)^-1 Diag(beta),  W = T (k * e^G),  U = T V
//   Delta = U - W S                      (row r = beta_r (v_r - S_{r-1}^T ... ))
//   O     = (q * e^G) S + P Delta
//   S'    = Diag(e^{G_L}) S + (k * e^{G_L - G})^T Delta
//
// Two kernels:
//   intra (K1): one workgroup per (chunk, head), fully parallel.  Gate
//     cumsum, Gram matrices A and P on MFMA, the UT solve for T on the
//     vector ALUs in fp32, then W and U on MFMA.  Its results are written to
//     the workspace already in the register order the scan's MFMA operands
//     use, so the scan streams them with 16-byte coalesced loads.
//   scan (K2): one workgroup per (sequence, head, 16-column tile of the
//     state), walking the sequence's chunks in order.  The fp32 state tile
//     stays in MFMA accumulators for the whole sequence; wave w owns state
//     rows [32w, 32w + 32).
//
// Precision (fixed by a rounding study against the fp64 oracle, worst case
// ~3e-3 of RMS against a 2e-2 contract): operands that carry the state or
// the outputs are split into bf16 hi + lo parts (three MFMA passes:
// hi*hi + hi*lo + lo*hi, ~16 significant bits); W and T-inside-W are plain
// bf16 (their error only reaches the outputs through the first tokens of a
// chunk).  Split: the Gram factors, T in U, q*e^G, k*e^{G_L-G}, P, Delta and
// S inside (q*e^G) S.
//
// Overflow: Gram blocks are factorised around a reference row m (the row
// before the 16-row block): e^{G_r-G_i} = e^{G_r-G_m} e^{G_m-G_i}.  Off the
// diagonal both factors are <= 1.  On a diagonal block the column factor is
// >= 1 and bounded by the block's own decay; when that exceeds 2^100 in some
// channel the block is computed exactly, pair by pair, on the vector ALUs.
#include "kda_launch.hpp"

namespace kda {

template <int C, int D>
struct Lay {
    static constexpr int CP = C < 32 ? 32 : C;    // token rows padded to a 32-wide k step
    static constexpr int NMT = C / 16;            // token tiles
    static constexpr int KSD = D / 32;            // channel k-steps
    static constexpr int KSC = CP / 32;           // token k-steps
    static constexpr int NDT = D / 16;            // channel tiles
    static constexpr size_t FRAG = 1024;          // 64 lanes x 16 bytes
    static constexpr size_t W = 0;
    static constexpr size_t QH = W + NMT * KSD * FRAG;
    static constexpr size_t QL = QH + NMT * KSD * FRAG;
    static constexpr size_t KBH = QL + NMT * KSD * FRAG;
    static constexpr size_t KBL = KBH + NDT * KSC * FRAG;
    static constexpr size_t PH = KBL + NDT * KSC * FRAG;
    static constexpr size_t PL = PH + NMT * KSC * FRAG;
    static constexpr size_t U = PL + NMT * KSC * FRAG;
    static constexpr size_t GAM = U + NMT * NDT * FRAG;
    static constexpr size_t BYTES = (GAM + D * sizeof(float) + 255) / 256 * 256;
};

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
    return x;
}

__device__ __forceinline__ uint4 ld16(const char *p) { return *reinterpret_cast<const uint4 *>(p); }
__device__ __forceinline__ void st16(char *p, uint4 v) { *reinterpret_cast<uint4 *>(p) = v; }
__device__ __forceinline__ f32x4 ldf4(const char *p) { return *reinterpret_cast<const f32x4 *>(p); }

// 4 bf16 packed in 8 bytes
__device__ __forceinline__ uint2 pack4(const bf16_t *s) {
    uint2 r;
    r.x = static_cast<uint32_t>(s[0]) | (static_cast<uint32_t>(s[1]) << 16);
    r.y = static_cast<uint32_t>(s[2]) | (static_cast<uint32_t>(s[3]) << 16);
    return r;
}

// log2-domain threshold for factorising a diagonal Gram block
constexpr float kDiagSpanMax = 100.f;

// ------------------------------------------------------------------ K1 --
template <int C, int D>
__global__ void __launch_bounds__(256) intra_kernel(PrefillParams p, char *__restrict__ blocks) {
    using Y = Lay<C, D>;
    constexpr int CP = Y::CP;
    if (*p.status != 0) return;
    const int x = blockIdx.x;
    const int h = blockIdx.y;
    const int H = p.H;
    if (x >= p.chunk_off[p.N]) return;
    const int n = chunk_to_seq(p.chunk_off, p.N, x);
    const SeqRange sr = seq_range(p, n);
    const int cidx = x - p.chunk_off[n];
    const int64_t t0 = sr.start + static_cast<int64_t>(cidx) * C;
    const int L = min(C, sr.len - cidx * C);
    char *blk = blocks + (static_cast<size_t>(x) * H + h) * Y::BYTES;

    __shared__ __attribute__((aligned(16))) bf16_t sk[CP][D];
    __shared__ __attribute__((aligned(16))) bf16_t sv[CP][D];
    __shared__ __attribute__((aligned(16))) float sG[CP][D];   // base-2 cumulative log-decay
    __shared__ __attribute__((aligned(16))) float sA[CP][CP];
    __shared__ __attribute__((aligned(16))) float sT[CP][CP];  // (I + A)^-1 (beta applied on use)
    __shared__ float sbeta[CP];

    const bf16_t *Kg = static_cast<const bf16_t *>(p.k);
    const bf16_t *Vg = static_cast<const bf16_t *>(p.v);
    const bf16_t *Qg = static_cast<const bf16_t *>(p.q);
    const bf16_t *Ag = static_cast<const bf16_t *>(p.log_alpha);
    const bf16_t *Bg = static_cast<const bf16_t *>(p.beta);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, li = lane & 15;

    // ---- 1. stage k, v (zero beyond L), gate cumsum, beta; clear A, T
    for (int e = tid; e < CP * D / 8; e += 256) {
        const int r = e / (D / 8), c8 = (e % (D / 8)) * 8;
        uint4 kk = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
        if (r < L) {
            const int64_t off = ((t0 + r) * H + h) * D + c8;
            kk = *reinterpret_cast<const uint4 *>(Kg + off);
            vv = *reinterpret_cast<const uint4 *>(Vg + off);
        }
        *reinterpret_cast<uint4 *>(&sk[r][c8]) = kk;
        *reinterpret_cast<uint4 *>(&sv[r][c8]) = vv;
    }
    for (int e = tid; e < CP * CP; e += 256) {
        (&sA[0][0])[e] = 0.f;
        (&sT[0][0])[e] = 0.f;
    }
    for (int ch = tid; ch < D; ch += 256) {
        float acc = 0.f;
        for (int r = 0; r < CP; ++r) {
            if (r < L) acc += bf16_to_f32(Ag[((t0 + r) * H + h) * D + ch]) * kLog2e;
            sG[r][ch] = acc;
        }
    }
    for (int r = tid; r < CP; r += 256) sbeta[r] = r < L ? bf16_to_f32(Bg[(t0 + r) * H + h]) : 0.f;
    __syncthreads();

    // ---- 2. Gram blocks: wave a computes row block a (rows 16a..16a+15)
    //      as transposed tiles A^T(b,a), P^T(b,a) for column blocks b <= a.
    if (wave < Y::NMT) {
        const int a = wave;
        const int r = 16 * a + li;  // row (token) this lane feeds as B operand
        float span = 0.f;
        for (int ch = lane; ch < D; ch += 64) {
            const float gm = a > 0 ? sG[16 * a - 1][ch] : 0.f;
            span = fmaxf(span, gm - sG[16 * a + 15][ch]);
        }
        const bool diag_mfma = wave_max(span) <= kDiagSpanMax;

        f32x4 accA[Y::NMT], accP[Y::NMT];
#pragma unroll
        for (int b = 0; b < Y::NMT; ++b) {
            accA[b] = f32x4{0.f, 0.f, 0.f, 0.f};
            accP[b] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int ks = 0; ks < Y::KSD; ++ks) {
            const int c0 = 32 * ks + 8 * g;
            float gm[8];
            frag8 krh, krl, qrh, qrl;
            const uint4 kraw = *reinterpret_cast<const uint4 *>(&sk[r][c0]);
            uint4 qraw = make_uint4(0, 0, 0, 0);
            if (r < L) qraw = *reinterpret_cast<const uint4 *>(Qg + ((t0 + r) * H + h) * D + c0);
            const bf16_t *kr = reinterpret_cast<const bf16_t *>(&kraw);
            const bf16_t *qr = reinterpret_cast<const bf16_t *>(&qraw);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                gm[j] = a > 0 ? sG[16 * a - 1][c0 + j] : 0.f;
                const float rf = fast_exp2(sG[r][c0 + j] - gm[j]);
                split_bf16(bf16_to_f32(kr[j]) * rf, krh.s[j], krl.s[j]);
                split_bf16(bf16_to_f32(qr[j]) * rf, qrh.s[j], qrl.s[j]);
            }
#pragma unroll
            for (int b = 0; b < Y::NMT; ++b) {
                if (b > a || (b == a && !diag_mfma)) continue;
                const int i = 16 * b + li;
                frag8 kih, kil;
                const uint4 kiraw = *reinterpret_cast<const uint4 *>(&sk[i][c0]);
                const bf16_t *ki = reinterpret_cast<const bf16_t *>(&kiraw);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float cf = fast_exp2(gm[j] - sG[i][c0 + j]);
                    split_bf16(bf16_to_f32(ki[j]) * cf, kih.s[j], kil.s[j]);
                }
                accA[b] = mfma16(kih.v, krh.v, accA[b]);
                accA[b] = mfma16(kih.v, krl.v, accA[b]);
                accA[b] = mfma16(kil.v, krh.v, accA[b]);
                accP[b] = mfma16(kih.v, qrh.v, accP[b]);
                accP[b] = mfma16(kih.v, qrl.v, accP[b]);
                accP[b] = mfma16(kil.v, qrh.v, accP[b]);
            }
        }
        if (!diag_mfma) {
            // exact pairwise diagonal block: lane holds (i = 16a + 4g + j, r)
            float ea[4] = {0.f, 0.f, 0.f, 0.f}, ep[4] = {0.f, 0.f, 0.f, 0.f};
            const bool rvalid = r < L;
            for (int ch = 0; ch < D; ++ch) {
                const float gr = sG[r][ch];
                const float kr_ = bf16_to_f32(sk[r][ch]);
                const float qr_ = rvalid ? bf16_to_f32(Qg[((t0 + r) * H + h) * D + ch]) : 0.f;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int i = 16 * a + 4 * g + j;
                    if (i <= r) {
                        const float f = bf16_to_f32(sk[i][ch]) * fast_exp2(gr - sG[i][ch]);
                        ea[j] += kr_ * f;
                        ep[j] += qr_ * f;
                    }
                }
            }
#pragma unroll
            for (int b = 0; b < Y::NMT; ++b)
                if (b == a) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        accA[b][j] = ea[j];
                        accP[b][j] = ep[j];
                    }
                }
        }
        // A (rows scaled by beta_r, strictly lower) -> LDS; P -> workspace
        const float br = sbeta[r];
#pragma unroll
        for (int b = 0; b < Y::NMT; ++b) {
            if (b > a) continue;
            bf16_t ph[4], pl[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int i = 16 * b + 4 * g + j;
                sA[r][i] = (i < r) ? accA[b][j] * br : 0.f;
                split_bf16((i <= r) ? accP[b][j] : 0.f, ph[j], pl[j]);
            }
            const size_t fo = ((static_cast<size_t>(a) * Y::KSC + b / 2) * 64 + lane) * 16 + (b & 1) * 8;
            *reinterpret_cast<uint2 *>(blk + Y::PH + fo) = pack4(ph);
            *reinterpret_cast<uint2 *>(blk + Y::PL + fo) = pack4(pl);
            if (b == a && (b & 1) == 0) {  // upper half of the same k step is zero
                *reinterpret_cast<uint2 *>(blk + Y::PH + fo + 8) = make_uint2(0, 0);
                *reinterpret_cast<uint2 *>(blk + Y::PL + fo + 8) = make_uint2(0, 0);
            }
        }
    }
    __syncthreads();

    // ---- 3. X = (I + A)^-1 by blocked forward substitution (fp32 VALU)
    if (wave < Y::NMT && li == lane) {  // lanes 0..15: column jj of diagonal block a
        const int a = wave, jj = li, base = 16 * a;
        float xc[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            float s = (rr == jj) ? 1.f : 0.f;
#pragma unroll
            for (int i = 0; i < rr; ++i)
                if (i >= jj) s -= sA[base + rr][base + i] * xc[i];
            xc[rr] = (rr >= jj) ? s : 0.f;
        }
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) sT[base + rr][base + jj] = xc[rr];
    }
    __syncthreads();
#pragma unroll
    for (int lev = 1; lev < Y::NMT; ++lev) {
        // block (a, b) with a - b = lev handled by wave b
        const bool act = wave < Y::NMT - lev;
        const int b = wave, a = wave + lev;
        const int rr = lane >> 2, cc0 = (lane & 3) * 4;
        float y[4] = {0.f, 0.f, 0.f, 0.f};
        if (act) {
            for (int c = b; c < a; ++c)
#pragma unroll
                for (int kk = 0; kk < 16; ++kk) {
                    const float av = sA[16 * a + rr][16 * c + kk];
#pragma unroll
                    for (int q = 0; q < 4; ++q) y[q] += av * sT[16 * c + kk][16 * b + cc0 + q];
                }
#pragma unroll
            for (int q = 0; q < 4; ++q) sT[16 * a + rr][16 * b + cc0 + q] = y[q];
        }
        __syncthreads();
        float xo[4] = {0.f, 0.f, 0.f, 0.f};
        if (act) {
#pragma unroll
            for (int kk = 0; kk < 16; ++kk) {
                const float xa = sT[16 * a + rr][16 * a + kk];
#pragma unroll
                for (int q = 0; q < 4; ++q) xo[q] -= xa * sT[16 * a + kk][16 * b + cc0 + q];
            }
        }
        __syncthreads();
        if (act) {
#pragma unroll
            for (int q = 0; q < 4; ++q) sT[16 * a + rr][16 * b + cc0 + q] = xo[q];
        }
        __syncthreads();
    }

    // ---- 4. W^T = (k e^G)^T T^T  (bf16)  and  U = T V  (T split)
    //      T[r][i] = X[r][i] * beta_i.  Wave w: channel tiles ct = w, w+4, ...
    for (int ct = wave; ct < Y::NDT; ct += 4) {
        const int ch = 16 * ct + li;
        f32x4 accW[Y::NMT], accU[Y::NMT];
#pragma unroll
        for (int tt = 0; tt < Y::NMT; ++tt) {
            accW[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
            accU[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int s = 0; s < Y::KSC; ++s) {
            frag8 kt, vb;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int i = 32 * s + 8 * g + j;
                kt.s[j] = f32_to_bf16(bf16_to_f32(sk[i][ch]) * fast_exp2(sG[i][ch]));
                vb.s[j] = sv[i][ch];
            }
#pragma unroll
            for (int tt = 0; tt < Y::NMT; ++tt) {
                if (32 * s > 16 * tt + 15) continue;
                const int r = 16 * tt + li;
                frag8 tb, th, tl;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int i = 32 * s + 8 * g + j;
                    const float tv = sT[r][i] * sbeta[i];
                    tb.s[j] = f32_to_bf16(tv);
                    split_bf16(tv, th.s[j], tl.s[j]);
                }
                accW[tt] = mfma16(kt.v, tb.v, accW[tt]);  // rows: channels, cols: tokens
                accU[tt] = mfma16(th.v, vb.v, accU[tt]);  // rows: tokens, cols: channels
                accU[tt] = mfma16(tl.v, vb.v, accU[tt]);
            }
        }
#pragma unroll
        for (int tt = 0; tt < Y::NMT; ++tt) {
            bf16_t wb[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) wb[j] = f32_to_bf16(accW[tt][j]);
            const size_t fo = ((static_cast<size_t>(tt) * Y::KSD + ct / 2) * 64 + lane) * 16 + (ct & 1) * 8;
            *reinterpret_cast<uint2 *>(blk + Y::W + fo) = pack4(wb);
            *reinterpret_cast<f32x4 *>(blk + Y::U + ((static_cast<size_t>(tt) * Y::NDT + ct) * 64 + lane) * 16) =
                accU[tt];
        }
    }

    // ---- 5. q e^G (split, scan A-operand order), (k e^{G_L - G})^T (split), e^{G_L}
    for (int f = wave; f < Y::NMT * Y::KSD; f += 4) {
        const int mt = f / Y::KSD, ks = f % Y::KSD;
        const int r = 16 * mt + li;
        frag8 hi, lo;
        uint2 q0 = make_uint2(0, 0), q1 = make_uint2(0, 0);
        if (r < L) {
            const bf16_t *qp = Qg + ((t0 + r) * H + h) * D + 32 * ks + 4 * g;
            q0 = *reinterpret_cast<const uint2 *>(qp);
            q1 = *reinterpret_cast<const uint2 *>(qp + 16);
        }
        const bf16_t *qa = reinterpret_cast<const bf16_t *>(&q0);
        const bf16_t *qb = reinterpret_cast<const bf16_t *>(&q1);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int ch = 32 * ks + kperm(g, j);
            const float qv = bf16_to_f32(j < 4 ? qa[j] : qb[j - 4]);
            split_bf16(qv * fast_exp2(sG[r][ch]), hi.s[j], lo.s[j]);
        }
        const size_t fo = (static_cast<size_t>(f) * 64 + lane) * 16;
        st16(blk + Y::QH + fo, hi.u);
        st16(blk + Y::QL + fo, lo.u);
    }
    for (int f = wave; f < Y::NDT * Y::KSC; f += 4) {
        const int mt = f / Y::KSC, ks = f % Y::KSC;
        const int ch = 16 * mt + li;
        const float gl = sG[C - 1][ch];
        frag8 hi, lo;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int i = 32 * ks + kperm(g, j);
            split_bf16(bf16_to_f32(sk[i][ch]) * fast_exp2(gl - sG[i][ch]), hi.s[j], lo.s[j]);
        }
        const size_t fo = (static_cast<size_t>(f) * 64 + lane) * 16;
        st16(blk + Y::KBH + fo, hi.u);
        st16(blk + Y::KBL + fo, lo.u);
    }
    for (int ch = tid; ch < D; ch += 256)
        reinterpret_cast<float *>(blk + Y::GAM)[ch] = fast_exp2(sG[C - 1][ch]);
}

// ------------------------------------------------------------------ K2 --
template <int C, int D, typename TO>
__global__ void __launch_bounds__(64 * (D / 32)) scan_kernel(PrefillParams p, const char *__restrict__ blocks) {
    using Y = Lay<C, D>;
    constexpr int NW = D / 32;    // waves; wave w owns state rows [32w, 32w + 32)
    constexpr int NVT = D / 16;   // 16-column state tiles per head
    constexpr int OWN = (Y::NMT + NW - 1) / NW;  // token tiles reduced per wave
    if (*p.status != 0) return;
    // XCD-aware order: the NVT column tiles of one (sequence, head) share
    // blockIdx % 8, hence one XCD and its L2.
    const int bid = blockIdx.x;
    const int xcd = bid & 7, slot = bid >> 3;
    const int nt = slot % NVT;
    const int pair = xcd + 8 * (slot / NVT);
    if (pair >= p.N * p.H) return;
    const int H = p.H;
    const int n = pair / H, h = pair % H;
    const SeqRange sr = seq_range(p, n);
    const int nch = (sr.len + C - 1) / C;
    const int64_t cbase = p.chunk_off[n];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int g = lane >> 4, li = lane & 15;
    const int col = 16 * nt + li;
    TO *o = static_cast<TO *>(p.o);

    __shared__ f32x4 red[2][NW][Y::NMT][64];
    __shared__ uint4 dls[Y::NMT][64];

    const int64_t soff = (static_cast<int64_t>(n) * H + h) * D * D;
    f32x4 S[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = 32 * w + 16 * i + 4 * g + j;
            S[i][j] = p.initial_state ? p.initial_state[soff + static_cast<int64_t>(row) * D + col] : 0.f;
        }

    for (int c = 0; c < nch; ++c) {
        const int64_t x = cbase + c;
        const char *blk = blocks + (static_cast<size_t>(x) * H + h) * Y::BYTES;
        const int64_t t0 = sr.start + static_cast<int64_t>(c) * C;
        const int L = min(C, sr.len - c * C);
        if (p.chunk_states) {
            float *cs = p.chunk_states + (x * H + h) * static_cast<int64_t>(D) * D;
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    cs[static_cast<int64_t>(32 * w + 16 * i + 4 * g + j) * D + col] = S[i][j];
        }
        // (a) state rows of this wave as a B operand, hi/lo
        frag8 sh, sl;
        acc2_to_split(S[0], S[1], sh, sl);
        // (b) partial W S and (q e^G) S over this wave's 32 channels
#pragma unroll
        for (int mt = 0; mt < Y::NMT; ++mt) {
            const size_t fo = ((static_cast<size_t>(mt) * Y::KSD + w) * 64 + lane) * 16;
            frag8 wf, qh, ql;
            wf.u = ld16(blk + Y::W + fo);
            qh.u = ld16(blk + Y::QH + fo);
            ql.u = ld16(blk + Y::QL + fo);
            f32x4 z = {0.f, 0.f, 0.f, 0.f};
            red[0][w][mt][lane] = mfma16(wf.v, sh.v, z);
            f32x4 pq = mfma16(qh.v, sh.v, z);
            pq = mfma16(qh.v, sl.v, pq);
            pq = mfma16(ql.v, sh.v, pq);
            red[1][w][mt][lane] = pq;
        }
        __syncthreads();
        // (c) reduce the token tiles this wave owns: Delta = U - sum W S
        f32x4 oq[OWN];
#pragma unroll
        for (int u = 0; u < OWN; ++u) {
            const int mt = w + u * NW;
            if (mt >= Y::NMT) continue;
            f32x4 d = ldf4(blk + Y::U + ((static_cast<size_t>(mt) * Y::NDT + nt) * 64 + lane) * 16);
            f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) {
                d -= red[0][ww][mt][lane];
                s += red[1][ww][mt][lane];
            }
            oq[u] = s;
            frag8 dd;
            bf16_t hi[4], lo[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) split_bf16(d[j], hi[j], lo[j]);
            const uint2 ph = pack4(hi), pl = pack4(lo);
            dls[mt][lane] = make_uint4(ph.x, ph.y, pl.x, pl.y);
        }
        __syncthreads();
        // (d) Delta as B operands, one per 32-token k step
        frag8 dh[Y::KSC], dl[Y::KSC];
#pragma unroll
        for (int s = 0; s < Y::KSC; ++s) {
            const uint4 t0v = dls[2 * s][lane];
            const uint4 t1v = (2 * s + 1 < Y::NMT) ? dls[2 * s + 1][lane] : make_uint4(0, 0, 0, 0);
            dh[s].u = make_uint4(t0v.x, t0v.y, t1v.x, t1v.y);
            dl[s].u = make_uint4(t0v.z, t0v.w, t1v.z, t1v.w);
        }
        // (e) outputs of the owned token tiles: O = (q e^G) S + P Delta
#pragma unroll
        for (int u = 0; u < OWN; ++u) {
            const int mt = w + u * NW;
            if (mt >= Y::NMT) continue;
            f32x4 acc = oq[u];
#pragma unroll
            for (int s = 0; s < Y::KSC; ++s) {
                if (32 * s > 16 * mt + 15) continue;
                const size_t fo = ((static_cast<size_t>(mt) * Y::KSC + s) * 64 + lane) * 16;
                frag8 ph, pl;
                ph.u = ld16(blk + Y::PH + fo);
                pl.u = ld16(blk + Y::PL + fo);
                acc = mfma16(ph.v, dh[s].v, acc);
                acc = mfma16(ph.v, dl[s].v, acc);
                acc = mfma16(pl.v, dh[s].v, acc);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int tok = 16 * mt + 4 * g + j;
                if (tok < L) io<TO>::st(o, ((t0 + tok) * H + h) * D + col, acc[j]);
            }
        }
        // (f) state: S = e^{G_L} S + (k e^{G_L - G})^T Delta
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int mtc = 2 * w + i;
            const f32x4 gam = ldf4(blk + Y::GAM + (32 * w + 16 * i + 4 * g) * sizeof(float));
            S[i] *= gam;
#pragma unroll
            for (int s = 0; s < Y::KSC; ++s) {
                const size_t fo = ((static_cast<size_t>(mtc) * Y::KSC + s) * 64 + lane) * 16;
                frag8 kh, kl;
                kh.u = ld16(blk + Y::KBH + fo);
                kl.u = ld16(blk + Y::KBL + fo);
                S[i] = mfma16(kh.v, dh[s].v, S[i]);
                S[i] = mfma16(kh.v, dl[s].v, S[i]);
                S[i] = mfma16(kl.v, dh[s].v, S[i]);
            }
        }
    }
    if (p.final_state) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                p.final_state[soff + static_cast<int64_t>(32 * w + 16 * i + 4 * g + j) * D + col] = S[i][j];
    }
}

// ---------------------------------------------------------------- host --
size_t mfma_block_bytes(int C, int D) {
    if (D == 128) {
        if (C == 64) return Lay<64, 128>::BYTES;
        if (C == 32) return Lay<32, 128>::BYTES;
        return Lay<16, 128>::BYTES;
    }
    if (C == 64) return Lay<64, 64>::BYTES;
    if (C == 32) return Lay<32, 64>::BYTES;
    return Lay<16, 64>::BYTES;
}

bool mfma_supported(int dk, int dv, int C) {
    return dk == dv && (dk == 64 || dk == 128) && (C == 16 || C == 32 || C == 64);
}

namespace {
template <int C, int D, typename TO>
hipError_t run_mfma(const PrefillParams &p, char *blocks, hipStream_t s, hipEvent_t mid) {
    hipLaunchKernelGGL((intra_kernel<C, D>), dim3(p.n_chunks_bound, p.H), dim3(256), 0, s, p, blocks);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && mid) e = hipEventRecord(mid, s);
    if (e != hipSuccess) return e;
    constexpr int NVT = D / 16;
    const int pairs = p.N * p.H;
    const unsigned grid = static_cast<unsigned>((pairs + 7) / 8) * NVT * 8;
    hipLaunchKernelGGL((scan_kernel<C, D, TO>), dim3(grid), dim3(64 * (D / 32)), 0, s, p,
                       static_cast<const char *>(blocks));
    return hipGetLastError();
}

template <int D, typename TO>
hipError_t run_mfma_c(const PrefillParams &p, char *blocks, hipStream_t s, hipEvent_t mid) {
    if (p.C == 64) return run_mfma<64, D, TO>(p, blocks, s, mid);
    if (p.C == 32) return run_mfma<32, D, TO>(p, blocks, s, mid);
    return run_mfma<16, D, TO>(p, blocks, s, mid);
}
}  // namespace

hipError_t launch_prefill_mfma(const PrefillParams &p, void *blocks, int out_dtype, hipStream_t s,
                               hipEvent_t mid) {
    char *b = static_cast<char *>(blocks);
    if (p.dk == 128)
        return out_dtype == 0 ? run_mfma_c<128, float>(p, b, s, mid) : run_mfma_c<128, bf16_t>(p, b, s, mid);
    return out_dtype == 0 ? run_mfma_c<64, float>(p, b, s, mid) : run_mfma_c<64, bf16_t>(p, b, s, mid);
}

}  // namespace kda
