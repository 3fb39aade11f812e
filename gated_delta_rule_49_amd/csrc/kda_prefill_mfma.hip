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
// Overflow: off-diagonal Gram blocks are factorised around a reference row m
// (the row before the 16-row block): e^{G_r-G_i} = e^{G_r-G_m} e^{G_m-G_i},
// both factors <= 1.  A diagonal block is factorised per channel around the
// midpoint c of its own decay (c halfway between G at the row before the
// block and G at its last row): e^{G_r-c} e^{c-G_i}, both within
// 2^(+-span/2), span = that decay in powers of two.  When the span exceeds
// 200 in some channel of a wave's channel half, that half of the block is
// computed exactly, pair by pair, on the vector ALUs.
#include <type_traits>

#include "kda_handoff.hpp"
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

// Four 16-bit values of a row-major [row][col] LDS tile, transposed across the
// 16 lanes of each lane group (ds_read_b64_tr_b16): lane i of group g
// receives X[r0 + 4g + j][c0 + i], j = 0..3, when every lane of the group
// addresses X[r0 + 4g + i / 4][c0 + 4 (i % 4)] (its 8-byte piece of the four
// rows).  Two such reads (r0 and r0 + 16) give an MFMA operand with K along
// the rows in the kperm order.
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
__device__ __forceinline__ uint2 lds_read_tr16(const bf16_t *piece) {
    // piece points into LDS (a __shared__ array): the C-style cast is the
    // generic-to-local address-space conversion
    const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(piece));
    return __builtin_bit_cast(uint2, r);
}

// persistent intra-chunk grid: one workgroup per CU of an MI355X (256 CUs)
constexpr int kIntraGrid = 256;

// Diagonal Gram blocks are factorised around the midpoint of their own decay
// (both factors within 2^(+-span/2)); beyond this span (log2 units) they are
// computed pair by pair instead.
constexpr float kDiagSpanMax = 200.f;

// ------------------------------------------------------------------ K1 --
// LDS plan of the intra-chunk kernel (bytes).  Rows are padded so that the
// 16 lanes of a fragment that read 16 consecutive rows hit distinct banks.
template <int C, int D>
struct IntraLds {
    static constexpr int CP = Lay<C, D>::CP;
    static constexpr int RK = D + 8;       // bf16 row stride of [token][channel]
    static constexpr int RTF = CP + 8;     // bf16 row stride of the T fragments
    static constexpr int RG = D + 4;       // fp32 row stride of G
    static constexpr int RA = CP + 4;      // fp32 row stride of A and X
    static constexpr int CPW = D / 8;      // cumsum: channels per wave
    static constexpr int NSEG = 64 / CPW;  // cumsum: token segments per channel
    static constexpr size_t SK = 0;                                   // k   [CP][RK] bf16
    static constexpr size_t SQ = SK + CP * RK * 2;                    // q   [CP][RK] bf16
    static constexpr size_t SA = SQ + CP * RK * 2;                    // A   [CP][RA] f32
    static constexpr size_t SV = SA + CP * RA * 4;                    // v   [CP][RK] bf16
    static constexpr size_t SG = SV + CP * RK * 2;                    // G   [CP][RG] f32 (log2 units)
    static constexpr size_t ST = SG + CP * RG * 4;                    // X = (I+A)^-1 [CP][RA] f32
    static constexpr size_t SB = ST + CP * RA * 4;                    // beta [CP]
    static constexpr size_t SNK = SB + CP * 4;                        // 1/|k_r| [CP] (1 without the norm)
    static constexpr size_t SNQ = SNK + CP * 4;                       // 1/|q_r| [CP]
    static constexpr size_t SCNT = SNQ + CP * 4;                      // work counter (int)
    static constexpr size_t SKG = SCNT + 16;                          // k e^G [CP][RK] bf16 (for W)
    static constexpr size_t END = SKG + CP * RK * 2;
    // after the Gram phase q and A are dead: the T fragments reuse [SQ, SV)
    // when they fit there, else they get their own region
    static constexpr bool REUSE = 3 * CP * RTF * 2 <= SV - SQ;
    static constexpr size_t TB = REUSE ? SQ : END;                    // T   bf16 [CP][RTF]
    static constexpr size_t TH = TB + CP * RTF * 2;                   // hi
    static constexpr size_t TL = TH + CP * RTF * 2;                   // lo
    static constexpr size_t BYTES = REUSE ? END : TL + CP * RTF * 2;
    // raw inputs prefetched per thread
    static constexpr int NVEC = CP * D / 8;                           // 16-byte vectors per array
    static constexpr int NV = (NVEC + 511) / 512;
    static constexpr int RS = CP / NSEG;                              // rows per cumsum segment
};

// One thread's share of a (chunk, head)'s raw inputs, held in registers so
// the next item's loads are in flight while the current one is computed.
template <int C, int D>
struct IntraRaw {
    using M = IntraLds<C, D>;
    // Raw bits only, loaded from rows clamped into [0, L): nothing here
    // depends on the loaded values, so the loads stay in flight until the
    // next item stages them (rows >= L are zeroed there).
    typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;  // one 128-bit register tuple
    u32x4 k[M::NV], v[M::NV], q[M::NV], a[M::NV];
    uint32_t beta;

    // Marks the loaded registers as redefined here, so that nothing derived
    // from them is scheduled before this point (which would wait for the
    // loads right after they are issued).
    __device__ __forceinline__ void settle() {
#pragma unroll
        for (int u = 0; u < M::NV; ++u) asm volatile("" : "+v"(k[u]), "+v"(v[u]), "+v"(q[u]), "+v"(a[u]));
        asm volatile("" : "+v"(beta));
    }

    // element offset of this thread's vector u of the (chunk, head) tile
    __device__ __forceinline__ static int64_t offset(int64_t t0, int L, int h, int H, int tid, int u) {
        const int e = min(tid + 512 * u, M::NVEC - 1);
        const int r = min(e / (D / 8), L - 1), c8 = (e % (D / 8)) * 8;
        return ((t0 + r) * H + h) * D + c8;
    }
    // Two load sites, each reached once per item: k and q (issued after the
    // Gram phase), then v, the gate and beta (issued after the UT solve), so
    // that no phase stalls on issuing all 64 KB of the next item's inputs.
    __device__ __forceinline__ void load_kq(const PrefillParams &p, int64_t t0, int L, int h, int tid) {
        const bf16_t *Kg = static_cast<const bf16_t *>(p.k);
        const bf16_t *Qg = static_cast<const bf16_t *>(p.q);
#pragma unroll
        for (int u = 0; u < M::NV; ++u) {
            const int64_t off = offset(t0, L, h, p.H, tid, u);
            k[u] = *reinterpret_cast<const u32x4 *>(Kg + off);
            q[u] = *reinterpret_cast<const u32x4 *>(Qg + off);
        }
    }
    __device__ __forceinline__ void load_va(const PrefillParams &p, int64_t t0, int L, int h, int tid) {
        const bf16_t *Vg = static_cast<const bf16_t *>(p.v);
        const bf16_t *Ag = static_cast<const bf16_t *>(p.log_alpha);
        const bf16_t *Bg = static_cast<const bf16_t *>(p.beta);
#pragma unroll
        for (int u = 0; u < M::NV; ++u) {
            const int64_t off = offset(t0, L, h, p.H, tid, u);
            v[u] = *reinterpret_cast<const u32x4 *>(Vg + off);
            a[u] = *reinterpret_cast<const u32x4 *>(Ag + off);
        }
        beta = Bg[(t0 + min(tid, L - 1)) * p.H + h];
    }
};

// A wave's W and U tiles of the previous item, held until they are stored.
// Wave w computes W channel tile w (if w < D/16) and U value tile
// (w >= D/16 ? w : w + 8) - D/16 (if that is < D/16).
template <int C, int D>
struct IntraPend {
    using Y = Lay<C, D>;
    uint2 w[Y::NMT];
    f32x4 u[Y::NMT];
    char *blk;

    __device__ __forceinline__ void flush(int wave, int lane) {
        if (blk == nullptr) return;
        if (wave < Y::NDT) {
            const int ct = wave;
#pragma unroll
            for (int tt = 0; tt < Y::NMT; ++tt) {
                const size_t fo = ((static_cast<size_t>(tt) * Y::KSD + ct / 2) * 64 + lane) * 16 + (ct & 1) * 8;
                *reinterpret_cast<uint2 *>(blk + Y::W + fo) = w[tt];
            }
        }
        const int wi = wave >= Y::NDT ? wave : wave + 8;
        if (wi < 2 * Y::NDT) {
            const int ct = wi - Y::NDT;
#pragma unroll
            for (int tt = 0; tt < Y::NMT; ++tt)
                *reinterpret_cast<f32x4 *>(blk + Y::U + ((static_cast<size_t>(tt) * Y::NDT + ct) * 64 + lane) * 16) = u[tt];
        }
        blk = nullptr;
    }
};

// (chunk, head) work item -> chunk-local coordinates
struct IntraItem {
    int x, h, L;
    int64_t t0;
};

__device__ __forceinline__ IntraItem intra_item(int item, int H, const int4 &ci) {
    IntraItem it;
    it.x = item / H;
    it.h = item % H;
    it.t0 = static_cast<int64_t>(static_cast<uint32_t>(ci.x)) | (static_cast<int64_t>(ci.y) << 32);
    it.L = ci.z;
    return it;
}

// P Q for 16 x 16 fp32 matrices held in accumulator layout (lane l: rows
// 4(l/16) + j, column l % 16), with P given transposed: four
// v_mfma_f32_16x16x4_f32 steps, step s taking k = 4(l/16) + s, so the A value
// of lane l is P[l%16][4(l/16)+s] = pt[s] and the B value is q[s].
__device__ __forceinline__ f32x4 mm16(const f32x4 &pt, const f32x4 &q) {
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(pt[s], q[s], c, 0, 0, 0);
    return c;
}

// (I + N)^-1 for a strictly lower 16 x 16 N (nilpotent): with M = -N,
// (I + M)(I + M^2)(I + M^4)(I + M^8), four levels of 16 x 16 products on
// fp32 matrix cores.  n and nt are N and N^T in accumulator layout; returns
// the inverse in accumulator layout (exactly zero above the diagonal).
__device__ __forceinline__ f32x4 unit_lower_inverse16(const f32x4 &n, const f32x4 &nt, int lane) {
    const int g = lane >> 4, li = lane & 15;
    const f32x4 m = -n, mt = -nt;
    const f32x4 m2 = mm16(mt, m), m2t = mm16(m, mt);
    const f32x4 m3 = mm16(mt, m2), m3t = mm16(m2, mt);
    const f32x4 m4 = mm16(m2t, m2), m4t = mm16(m2, m2t);
    const f32x4 m8 = mm16(m4t, m4);
    f32x4 id;
#pragma unroll
    for (int j = 0; j < 4; ++j) id[j] = (4 * g + j == li) ? 1.f : 0.f;
    const f32x4 r1 = id + m + m2 + m3, r1t = id + mt + m2t + m3t;  // (I + M)(I + M^2)
    const f32x4 r2 = r1 + mm16(r1t, m4), r2t = r1t + mm16(m4, r1t);  // ... (I + M^4)
    return r2 + mm16(r2t, m8);                                          // ... (I + M^8)
}

// Gram work plan: the block pair (a, b <= a) that wave group grp (0..3)
// handles in its u-th slot, as a * 8 + b, or -1.  With four row blocks the ten
// pairs are dealt 3, 3, 2, 2 so that each SIMD (waves w and w + 4) carries five
// half-pairs:  g0 (3,3) (3,2) (3,1) | g1 (3,0) (2,2) (2,1) | g2 (2,0) (1,1) |
// g3 (1,0) (0,0).  One byte per group, 0xff = none.
template <int NB>
__device__ __forceinline__ int gram_pair(int grp, int u) {
    uint32_t w;
    if (NB == 4)
        w = u == 0 ? 0x0810181bu : u == 1 ? 0x0009121au : 0xffff1119u;
    else if (NB == 2)
        w = u == 0 ? 0xff000809u : 0xffffffffu;  // g0 (1,1) | g1 (1,0) | g2 (0,0)
    else
        w = u == 0 ? 0xffffff00u : 0xffffffffu;  // g0 (0,0)
    const int code = static_cast<int>((w >> (8 * grp)) & 0xffu);
    return code == 0xff ? -1 : code;
}

// The (chunk, head) items one workgroup of the per-chunk stage computes, in
// order: schedule positions first, first + stride, ... below total.  In the
// plain order (npx == 0) position k is item k = chunk * H + head; in the
// XCD-local order of a single sequence (npx > 0) it is chunk k / npx of head
// x + 8 (k % npx), one of the npx heads whose scan runs on XCD x.
struct IntraSched {
    int first, stride, total;
    int npx, x, H;
    __device__ __forceinline__ int item(int k) const { return npx == 0 ? k : (k / npx) * H + x + 8 * (k % npx); }
};

// The per-chunk stage over the items of schedule sc, with its LDS at smem
// (IntraLds<C, D>::BYTES bytes).  Persistent: pass i computes one item and
// loads the inputs of the next.  PUB (the overlapped launch): once every
// store of an item's block has completed, its flag is set to 1 + the XCD
// the workgroup runs on (xcc).
template <int C, int D, bool PUB>
__device__ __forceinline__ void intra_run(const PrefillParams &p, char *__restrict__ blocks, char *smem,
                                          const IntraSched &sc, int32_t *ready, int xcc) {
    using Y = Lay<C, D>;
    using M = IntraLds<C, D>;
    constexpr int CP = Y::CP;
    constexpr int KH = Y::KSD / 2;  // channel k-steps per Gram half
    const int H = p.H;
    auto SK = reinterpret_cast<bf16_t(*)[M::RK]>(smem + M::SK);
    auto SQ = reinterpret_cast<bf16_t(*)[M::RK]>(smem + M::SQ);
    auto SA = reinterpret_cast<float(*)[M::RA]>(smem + M::SA);
    auto SV = reinterpret_cast<bf16_t(*)[M::RK]>(smem + M::SV);
    auto SKG = reinterpret_cast<bf16_t(*)[M::RK]>(smem + M::SKG);
    auto SG = reinterpret_cast<float(*)[M::RG]>(smem + M::SG);
    auto SX = reinterpret_cast<float(*)[M::RA]>(smem + M::ST);
    auto SBETA = reinterpret_cast<float *>(smem + M::SB);
    auto SNK = reinterpret_cast<float *>(smem + M::SNK);
    auto SNQ = reinterpret_cast<float *>(smem + M::SNQ);
    auto TB = reinterpret_cast<bf16_t(*)[M::RTF]>(smem + M::TB);
    auto TH = reinterpret_cast<bf16_t(*)[M::RTF]>(smem + M::TH);
    auto TL = reinterpret_cast<bf16_t(*)[M::RTF]>(smem + M::TL);

    if (sc.first >= sc.total) return;
    IntraRaw<C, D> raw;
    IntraItem it{};
    int4 nci = p.chunk_info[sc.item(sc.first) / H];  // coordinates of the next item
    IntraPend<C, D> pend;
    pend.blk = nullptr;
    int pub = -1;  // PUB: the item whose block is stored last, published after its W and U tiles

    // Pass i computes item_i and loads the raw inputs of item_{i+1}; the first
    // pass (item < 0) only loads.  A single load site keeps the prefetched
    // registers in place across the loop instead of being copied (a copy
    // would wait for the loads).
    for (int item = sc.first - sc.stride;; item += sc.stride) {  // schedule positions
        // The thread index is made opaque for each item so that the compiler
        // recomputes per-thread addresses inside the loop instead of keeping
        // dozens of them live (and spilled) across the whole kernel.
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int g = lane >> 4, li = lane & 15;
        const int L = it.L;
        const int next = item + sc.stride;
        const bool live = item >= 0;
        char *blk = blocks + (static_cast<size_t>(it.x) * H + it.h) * Y::BYTES;
        // (the wait for this load coincides with the staging's wait for the
        // prefetched inputs, which were issued before it)
        const IntraItem itn = intra_item(sc.item(next), H, make_int4(__builtin_amdgcn_readfirstlane(nci.x),
                                                            __builtin_amdgcn_readfirstlane(nci.y),
                                                            __builtin_amdgcn_readfirstlane(nci.z), 0));
        const int kh = wave & 1, grp = wave >> 1;
        f32x4 accA[3], accP[3];
        int pab[3];

        if (live) {
            raw.settle();
            // ---- 1. stage k, q, v (bf16) and log alpha (fp32; becomes G in
            //         place), all in natural [token][channel] layout, zero beyond L;
            //         then the gate cumsum, one wave per D/8 channels: lane
            //         (channel, token segment) sums its segment and the segment
            //         offsets come from a scan across lanes.
#pragma unroll
            for (int u = 0; u < M::NV; ++u) {
                const int e = tid + 512 * u;
                if (e >= M::NVEC) continue;
                const int r = e / (D / 8), c8 = (e % (D / 8)) * 8;
                const bool live = r < L;
                using u32x4 = typename IntraRaw<C, D>::u32x4;
                const u32x4 z = {0u, 0u, 0u, 0u};
                const u32x4 kv = live ? raw.k[u] : z, vv = live ? raw.v[u] : z, qv = live ? raw.q[u] : z;
                const u32x4 av = live ? raw.a[u] : z;
                *reinterpret_cast<u32x4 *>(&SK[r][c8]) = kv;
                *reinterpret_cast<u32x4 *>(&SQ[r][c8]) = qv;
                *reinterpret_cast<u32x4 *>(&SV[r][c8]) = vv;
                if (C < CP && r >= C) *reinterpret_cast<u32x4 *>(&SKG[r][c8]) = z;
                // 32-bit word operations on the raw registers (element j of a
                // vector is the low (j even) or high (j odd) half of word j / 2)
                const uint32_t kw[4] = {kv.x, kv.y, kv.z, kv.w};
                const uint32_t aw[4] = {av.x, av.y, av.z, av.w};
                f32x4 g0 = {__uint_as_float(aw[0] << 16), __uint_as_float(aw[0] & 0xffff0000u),
                            __uint_as_float(aw[1] << 16), __uint_as_float(aw[1] & 0xffff0000u)};
                f32x4 g1 = {__uint_as_float(aw[2] << 16), __uint_as_float(aw[2] & 0xffff0000u),
                            __uint_as_float(aw[3] << 16), __uint_as_float(aw[3] & 0xffff0000u)};
                if (p.prologue & kProGate) {  // rows beyond L hold x = 0: zeroed below by live
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        g0[j] = live ? -softplus_f32(g0[j]) : 0.f;
                        g1[j] = live ? -softplus_f32(g1[j]) : 0.f;
                    }
                }
                *reinterpret_cast<f32x4 *>(&SG[r][c8]) = g0;
                *reinterpret_cast<f32x4 *>(&SG[r][c8 + 4]) = g1;
                // 1 / |k_r|, 1 / |q_r| (1 without the norm): the D/8 lanes of
                // row r are consecutive, so the sum of squares is a butterfly
                // over them
                float nk = 1.f, nq = 1.f;
                if (p.prologue & kProQKNorm) {
                    const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
                    float sk = 0.f, sq = 0.f;
#pragma unroll
                    for (int j2 = 0; j2 < 4; ++j2) {
                        const float k0 = __uint_as_float(kw[j2] << 16), k1 = __uint_as_float(kw[j2] & 0xffff0000u);
                        const float q0 = __uint_as_float(qw[j2] << 16), q1 = __uint_as_float(qw[j2] & 0xffff0000u);
                        sk += k0 * k0 + k1 * k1;
                        sq += q0 * q0 + q1 * q1;
                    }
#pragma unroll
                    for (int o = 1; o < D / 8; o <<= 1) {
                        sk += __shfl_xor(sk, o);
                        sq += __shfl_xor(sq, o);
                    }
                    nk = 1.f / __builtin_sqrtf(sk + kQKNormEps);
                    nq = 1.f / __builtin_sqrtf(sq + kQKNormEps);
                }
                if (c8 == 0) {
                    SNK[r] = nk;
                    SNQ[r] = nq;
                }
            }
            if (tid < CP) {
                float b = bf16_to_f32(static_cast<bf16_t>(raw.beta));
                if (p.prologue & kProBeta) b = sigmoid_f32(b);
                SBETA[tid] = tid < L ? b : 0.f;
            }
            // fragments 0 .. 7 - C/16 go to the waves that do not invert a diagonal block
            if (tid == 0) *reinterpret_cast<int *>(smem + M::SCNT) = 8 - Y::NMT;
            lds_barrier();
            pend.flush(wave, lane);  // the previous item's W and U tiles
            {
                const int chl = lane % M::CPW, seg = lane / M::CPW;
                const int ch = wave * M::CPW + chl;
                float gv[M::RS];
#pragma unroll
                for (int j = 0; j < M::RS; ++j) gv[j] = SG[seg * M::RS + j][ch];
#pragma unroll
                for (int j = 1; j < M::RS; ++j) gv[j] += gv[j - 1];
                float t = gv[M::RS - 1];
#pragma unroll
                for (int o = M::CPW; o < 64; o <<= 1) {
                    const float n = __shfl_up(t, o);
                    if (lane >= o) t += n;
                }
                const float off = t - gv[M::RS - 1];
#pragma unroll
                for (int j = 0; j < M::RS; ++j) SG[seg * M::RS + j][ch] = (off + gv[j]) * kLog2e;
            }
            // PUB: the previous item's W and U tiles were stored at the
            // staging barrier, its other parts during that item
            if (PUB && pub >= 0) wait_memory();
            lds_barrier();
            if (PUB && pub >= 0) {
                if (tid == 0) publish_ready(ready + pub, xcc);
                pub = -1;
            }

            // ---- 2. Gram blocks A^T(b,a), P^T(b,a) for b <= a.  Work unit =
            //         (block pair, half of the channels): wave w = kh + 2 grp takes
            //         channel half kh of the pairs in group grp (gram_pair), so every
            //         SIMD gets the same number of units and a wave reuses its row
            //         operands across the pairs of one row block.  Operands are
            //         split into bf16 hi + lo (three MFMA passes, ~16 bits; fp32
            //         matrix cores cost ~5x the matrix time and measured slower).
            //         Factors around
            //         reference row m = 16a - 1: rows (<= 1) e^{G_r - G_m}, columns
            //         e^{G_m - G_i}.  Half 1 leaves its partial sums in LDS (A in SA,
            //         P in SX) and half 0 adds them and finalises.
            bool exact[3];
            {
                frag8 krh[KH], krl[KH], qrh[KH], qrl[KH];
                int cur_a = -1;
#pragma unroll
                for (int u = 0; u < 3; ++u) {
                    const int code = gram_pair<Y::NMT>(grp, u);
                    pab[u] = code;
                    exact[u] = false;
                    accA[u] = f32x4{0.f, 0.f, 0.f, 0.f};
                    accP[u] = accA[u];
                    if (code < 0) continue;
                    const int a = code >> 3, b = code & 7;
                    const int r = 16 * a + li;
                    if (a == b) {
                        float span = 0.f;
                        if (lane < 32 * KH) {
                            const int ch = 32 * KH * kh + lane;
                            const float gm = a > 0 ? SG[16 * a - 1][ch] : 0.f;
                            span = gm - SG[16 * a + 15][ch];
                        }
                        exact[u] = wave_max(span) > kDiagSpanMax;
                        if (exact[u]) continue;  // done pair by pair below
                        // Factorise around c = (G_m + G_{16a+15}) / 2 per channel:
                        // rows e^{G_r - c}, columns e^{c - G_i}, both within
                        // 2^(+-span/2) and kept in fp32 (fp32 matrix cores: no
                        // hi/lo split).  Rows and columns are the same 16 tokens,
                        // so a lane builds both operands of its own token.
#pragma unroll
                        for (int s2 = 0; s2 < KH; ++s2) {
                            const int c0 = 32 * (KH * kh + s2) + 8 * g;
                            const uint4 kraw = *reinterpret_cast<const uint4 *>(&SK[r][c0]);
                            const uint4 qraw = *reinterpret_cast<const uint4 *>(&SQ[r][c0]);
                            const bf16_t *kr = reinterpret_cast<const bf16_t *>(&kraw);
                            const bf16_t *qr = reinterpret_cast<const bf16_t *>(&qraw);
                            const f32x4 gr0 = *reinterpret_cast<const f32x4 *>(&SG[r][c0]);
                            const f32x4 gr1 = *reinterpret_cast<const f32x4 *>(&SG[r][c0 + 4]);
                            const f32x4 ge0 = *reinterpret_cast<const f32x4 *>(&SG[16 * a + 15][c0]);
                            const f32x4 ge1 = *reinterpret_cast<const f32x4 *>(&SG[16 * a + 15][c0 + 4]);
                            f32x4 gm0 = {0.f, 0.f, 0.f, 0.f}, gm1 = gm0;
                            if (a > 0) {
                                gm0 = *reinterpret_cast<const f32x4 *>(&SG[16 * a - 1][c0]);
                                gm1 = *reinterpret_cast<const f32x4 *>(&SG[16 * a - 1][c0 + 4]);
                            }
#pragma unroll
                            for (int j = 0; j < 8; ++j) {
                                const float gr = j < 4 ? gr0[j] : gr1[j - 4];
                                const float cmid = 0.5f * ((j < 4 ? gm0[j] : gm1[j - 4]) + (j < 4 ? ge0[j] : ge1[j - 4]));
                                const float kv = bf16_to_f32(kr[j]);
                                const float rf = fast_exp2(gr - cmid), cf = fast_exp2(cmid - gr);
                                // step j: lane group g contributes channel c0 + j
                                accA[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(kv * cf, kv * rf, accA[u], 0, 0, 0);
                                accP[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(kv * cf, bf16_to_f32(qr[j]) * rf, accP[u],
                                                                               0, 0, 0);
                            }
                        }
                        continue;
                    }
                    if (a != cur_a) {  // row operands of block a, this channel half
#pragma unroll
                        for (int s2 = 0; s2 < KH; ++s2) {
                            const int c0 = 32 * (KH * kh + s2) + 8 * g;
                            const uint4 kraw = *reinterpret_cast<const uint4 *>(&SK[r][c0]);
                            const uint4 qraw = *reinterpret_cast<const uint4 *>(&SQ[r][c0]);
                            const bf16_t *kr = reinterpret_cast<const bf16_t *>(&kraw);
                            const bf16_t *qr = reinterpret_cast<const bf16_t *>(&qraw);
                            const f32x4 gr0 = *reinterpret_cast<const f32x4 *>(&SG[r][c0]);
                            const f32x4 gr1 = *reinterpret_cast<const f32x4 *>(&SG[r][c0 + 4]);
                            f32x4 gm0 = {0.f, 0.f, 0.f, 0.f}, gm1 = gm0;
                            if (a > 0) {
                                gm0 = *reinterpret_cast<const f32x4 *>(&SG[16 * a - 1][c0]);
                                gm1 = *reinterpret_cast<const f32x4 *>(&SG[16 * a - 1][c0 + 4]);
                            }
#pragma unroll
                            for (int j = 0; j < 8; ++j) {
                                const float rf = fast_exp2(j < 4 ? gr0[j] - gm0[j] : gr1[j - 4] - gm1[j - 4]);
                                split_bf16(bf16_to_f32(kr[j]) * rf, krh[s2].s[j], krl[s2].s[j]);
                                split_bf16(bf16_to_f32(qr[j]) * rf, qrh[s2].s[j], qrl[s2].s[j]);
                            }
                        }
                        cur_a = a;
                    }
                    const int i = 16 * b + li;
#pragma unroll
                    for (int s2 = 0; s2 < KH; ++s2) {
                        const int c0 = 32 * (KH * kh + s2) + 8 * g;
                        const uint4 kiraw = *reinterpret_cast<const uint4 *>(&SK[i][c0]);
                        const bf16_t *ki = reinterpret_cast<const bf16_t *>(&kiraw);
                        const f32x4 gi0 = *reinterpret_cast<const f32x4 *>(&SG[i][c0]);
                        const f32x4 gi1 = *reinterpret_cast<const f32x4 *>(&SG[i][c0 + 4]);
                        f32x4 gm0 = {0.f, 0.f, 0.f, 0.f}, gm1 = gm0;
                        if (a > 0) {
                            gm0 = *reinterpret_cast<const f32x4 *>(&SG[16 * a - 1][c0]);
                            gm1 = *reinterpret_cast<const f32x4 *>(&SG[16 * a - 1][c0 + 4]);
                        }
                        frag8 kih, kil;
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            const float cf = fast_exp2(j < 4 ? gm0[j] - gi0[j] : gm1[j - 4] - gi1[j - 4]);
                            split_bf16(bf16_to_f32(ki[j]) * cf, kih.s[j], kil.s[j]);
                        }
                        accA[u] = mfma16(kih.v, krh[s2].v, accA[u]);
                        accA[u] = mfma16(kih.v, krl[s2].v, accA[u]);
                        accA[u] = mfma16(kil.v, krh[s2].v, accA[u]);
                        accP[u] = mfma16(kih.v, qrh[s2].v, accP[u]);
                        accP[u] = mfma16(kih.v, qrl[s2].v, accP[u]);
                        accP[u] = mfma16(kil.v, qrh[s2].v, accP[u]);
                    }
                }
            }
            // Diagonal blocks whose decay is too steep to factorise in this
            // channel half, exactly, pair by pair: lane holds (i = 16a + 4g + j, r).
#pragma unroll
            for (int u = 0; u < 3; ++u) {
                if (!exact[u]) continue;
                const int a = pab[u] >> 3;
                const int r = 16 * a + li;
#pragma unroll 1
                for (int c8 = 32 * KH * kh; c8 < 32 * KH * (kh + 1); c8 += 8) {
                    const uint4 kr8 = *reinterpret_cast<const uint4 *>(&SK[r][c8]);
                    const uint4 qr8 = *reinterpret_cast<const uint4 *>(&SQ[r][c8]);
                    const f32x4 gr0 = *reinterpret_cast<const f32x4 *>(&SG[r][c8]);
                    const f32x4 gr1 = *reinterpret_cast<const f32x4 *>(&SG[r][c8 + 4]);
                    const bf16_t *krb = reinterpret_cast<const bf16_t *>(&kr8);
                    const bf16_t *qrb = reinterpret_cast<const bf16_t *>(&qr8);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int i = 16 * a + 4 * g + j;
                        const uint4 ki8 = *reinterpret_cast<const uint4 *>(&SK[i][c8]);
                        const f32x4 gi0 = *reinterpret_cast<const f32x4 *>(&SG[i][c8]);
                        const f32x4 gi1 = *reinterpret_cast<const f32x4 *>(&SG[i][c8 + 4]);
                        const bf16_t *kib = reinterpret_cast<const bf16_t *>(&ki8);
                        float sa = 0.f, sp = 0.f;
#pragma unroll
                        for (int c = 0; c < 8; ++c) {
                            const float gd = (c < 4 ? gr0[c] : gr1[c - 4]) - (c < 4 ? gi0[c] : gi1[c - 4]);
                            const float f = bf16_to_f32(kib[c]) * fast_exp2(fminf(gd, 0.f));
                            sa += bf16_to_f32(krb[c]) * f;
                            sp += bf16_to_f32(qrb[c]) * f;
                        }
                        if (i <= r) {
                            accA[u][j] += sa;
                            accP[u][j] += sp;
                        }
                    }
                }
            }
            if (kh == 1) {  // partial sums -> LDS; the same lanes of half 0 read them
#pragma unroll
                for (int u = 0; u < 3; ++u) {
                    if (pab[u] < 0) continue;
                    const int a = pab[u] >> 3, b = pab[u] & 7;
                    const int r = 16 * a + li;
                    *reinterpret_cast<f32x4 *>(&SA[r][16 * b + 4 * g]) = accA[u];
                    *reinterpret_cast<f32x4 *>(&SX[r][16 * b + 4 * g]) = accP[u];
                }
            }
            lds_barrier();
            if (kh == 0) {
#pragma unroll
                for (int u = 0; u < 3; ++u) {
                    const int code = pab[u];
                    if (code < 0) continue;
                    const int a = code >> 3, b = code & 7;
                    const int r = 16 * a + li;
                    const f32x4 pa = *reinterpret_cast<const f32x4 *>(&SA[r][16 * b + 4 * g]);
                    const f32x4 pp = *reinterpret_cast<const f32x4 *>(&SX[r][16 * b + 4 * g]);
                    // A (rows scaled by beta_r, strictly lower) -> LDS; P -> workspace
                    // rows scaled by beta_r; the q/k norms enter as 1/|k_r| 1/|k_i|
                    // (A) and 1/|q_r| 1/|k_i| (P)
                    const float ar = SBETA[r] * SNK[r], pr = SNQ[r];
                    const f32x4 nki = *reinterpret_cast<const f32x4 *>(&SNK[16 * b + 4 * g]);
                    f32x4 av;
                    bf16_t ph[4], pl[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int i = 16 * b + 4 * g + j;
                        av[j] = (i < r) ? (accA[u][j] + pa[j]) * ar * nki[j] : 0.f;
                        split_bf16((i <= r) ? (accP[u][j] + pp[j]) * pr * nki[j] : 0.f, ph[j], pl[j]);
                    }
                    *reinterpret_cast<f32x4 *>(&SA[r][16 * b + 4 * g]) = av;
                    const size_t fo = ((static_cast<size_t>(a) * Y::KSC + b / 2) * 64 + lane) * 16 + (b & 1) * 8;
                    *reinterpret_cast<uint2 *>(blk + Y::PH + fo) = pack4(ph);
                    *reinterpret_cast<uint2 *>(blk + Y::PL + fo) = pack4(pl);
                    if (b == a && (b & 1) == 0) {  // the upper half of this k step is zero
                        *reinterpret_cast<uint2 *>(blk + Y::PH + fo + 8) = make_uint2(0, 0);
                        *reinterpret_cast<uint2 *>(blk + Y::PL + fo + 8) = make_uint2(0, 0);
                    }
                }
            }
        }  // live
        // the next item's k and q: loads in flight during the rest of this
        // item (issued after the Gram phase, whose registers they would crowd)
        if (next < sc.total) raw.load_kq(p, itn.t0, itn.L, itn.h, tid);
        if (live) {
            lds_barrier();

            // ---- 2b (any idle wave). One scan-operand fragment: q e^G in the
            //      scan's A-operand order, or (k e^{G_L - G})^T, as bf16 hi/lo.
            constexpr int NF = Y::NMT * Y::KSD + Y::NDT * Y::KSC;
            auto operand_fragment = [&](int f) {
                frag8 hi, lo;
                size_t dst_h, dst_l;
                if (f < Y::NMT * Y::KSD) {
                    const int mt = f / Y::KSD, ks = f % Y::KSD;
                    const int r = 16 * mt + li;
                    const int cA = 32 * ks + 4 * g, cB = cA + 16;
                    const uint2 q0 = *reinterpret_cast<const uint2 *>(&SQ[r][cA]);
                    const uint2 q1 = *reinterpret_cast<const uint2 *>(&SQ[r][cB]);
                    const f32x4 g0 = *reinterpret_cast<const f32x4 *>(&SG[r][cA]);
                    const f32x4 g1 = *reinterpret_cast<const f32x4 *>(&SG[r][cB]);
                    const bf16_t *qa = reinterpret_cast<const bf16_t *>(&q0);
                    const bf16_t *qb = reinterpret_cast<const bf16_t *>(&q1);
                    const float nq = SNQ[r];
                    // the same elements of k e^G (bf16, natural layout) for W
                    const uint2 k0 = *reinterpret_cast<const uint2 *>(&SK[r][cA]);
                    const uint2 k1 = *reinterpret_cast<const uint2 *>(&SK[r][cB]);
                    const bf16_t *ka = reinterpret_cast<const bf16_t *>(&k0);
                    const bf16_t *kb = reinterpret_cast<const bf16_t *>(&k1);
                    bf16_t kga[4], kgb[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float ea = fast_exp2(g0[j]), eb = fast_exp2(g1[j]);
                        split_bf16(bf16_to_f32(qa[j]) * nq * ea, hi.s[j], lo.s[j]);
                        split_bf16(bf16_to_f32(qb[j]) * nq * eb, hi.s[4 + j], lo.s[4 + j]);
                        kga[j] = f32_to_bf16(bf16_to_f32(ka[j]) * ea);
                        kgb[j] = f32_to_bf16(bf16_to_f32(kb[j]) * eb);
                    }
                    *reinterpret_cast<uint2 *>(&SKG[r][cA]) = pack4(kga);
                    *reinterpret_cast<uint2 *>(&SKG[r][cB]) = pack4(kgb);
                    const size_t fo = (static_cast<size_t>(f) * 64 + lane) * 16;
                    dst_h = Y::QH + fo;
                    dst_l = Y::QL + fo;
                } else {
                    const int f2 = f - Y::NMT * Y::KSD;
                    const int mt = f2 / Y::KSC, ks = f2 % Y::KSC;
                    const int ch = 16 * mt + li;
                    const float gl = SG[C - 1][ch];
                    const int iA = 32 * ks + 4 * g, iB = iA + 16;
                    // k at tokens iA..iA+3 and iB..iB+3 of channel ch
                    const bf16_t *kp = &SK[32 * ks + 4 * g + li / 4][16 * mt + 4 * (li % 4)];
                    const uint2 k0 = lds_read_tr16(kp);
                    const uint2 k1 = lds_read_tr16(kp + 16 * M::RK);
                    const bf16_t *ka = reinterpret_cast<const bf16_t *>(&k0);
                    const bf16_t *kb = reinterpret_cast<const bf16_t *>(&k1);
                    const f32x4 nka = *reinterpret_cast<const f32x4 *>(&SNK[iA]);
                    const f32x4 nkb = *reinterpret_cast<const f32x4 *>(&SNK[iB]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        split_bf16(bf16_to_f32(ka[j]) * nka[j] * fast_exp2(gl - SG[iA + j][ch]), hi.s[j], lo.s[j]);
                        split_bf16(bf16_to_f32(kb[j]) * nkb[j] * fast_exp2(gl - SG[iB + j][ch]), hi.s[4 + j],
                                   lo.s[4 + j]);
                    }
                    const size_t fo = (static_cast<size_t>(f2) * 64 + lane) * 16;
                    dst_h = Y::KBH + fo;
                    dst_l = Y::KBL + fo;
                }
                st16(blk + dst_h, hi.u);
                st16(blk + dst_l, lo.u);
            };

            // ---- 3. X = (I + A)^-1 in fp32 on matrix cores.  (a) wave a < C/16
            //         inverts diagonal block a while the other waves take one
            //         operand fragment each; (b) wave b < C/16 - 1 walks block
            //         column b down, X_ab = -X_aa sum_{c=b}^{a-1} A_ac X_cb, one
            //         product chain per term; every wave then takes the remaining
            //         fragments from a counter in LDS.
            f32x4 xdiag = {0.f, 0.f, 0.f, 0.f};
            if (wave < Y::NMT) {
                const int base = 16 * wave;
                f32x4 n, nt;
                nt = *reinterpret_cast<const f32x4 *>(&SA[base + li][base + 4 * g]);
#pragma unroll
                for (int j = 0; j < 4; ++j) n[j] = SA[base + 4 * g + j][base + li];
                xdiag = unit_lower_inverse16(n, nt, lane);
#pragma unroll
                for (int j = 0; j < 4; ++j) SX[base + 4 * g + j][base + li] = xdiag[j];
            } else if (wave - Y::NMT < NF) {
                operand_fragment(wave - Y::NMT);
            }
            lds_barrier();
            if (wave < Y::NMT - 1) {
                const int b = wave;
                f32x4 xcol[Y::NMT];  // X_cb, c >= b, accumulator layout
#pragma unroll
                for (int c = 0; c < Y::NMT; ++c) xcol[c] = xdiag;
#pragma unroll
                for (int a = 1; a < Y::NMT; ++a) {
                    if (a <= b) continue;
                    f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int c = 0; c < Y::NMT - 1; ++c) {
                        if (c < b || c >= a) continue;
                        y += mm16(*reinterpret_cast<const f32x4 *>(&SA[16 * a + li][16 * c + 4 * g]), xcol[c]);
                    }
                    const f32x4 z = mm16(*reinterpret_cast<const f32x4 *>(&SX[16 * a + li][16 * a + 4 * g]), y);
                    xcol[a] = -z;
#pragma unroll
                    for (int j = 0; j < 4; ++j) SX[16 * a + 4 * g + j][16 * b + li] = -z[j];
                }
            }
            if (tid >= 512 - D) reinterpret_cast<float *>(blk + Y::GAM)[tid - (512 - D)] = fast_exp2(SG[C - 1][tid - (512 - D)]);
            int *cnt = reinterpret_cast<int *>(smem + M::SCNT);
            for (;;) {
                int f = 0;
                if (lane == 0) f = atomicAdd(cnt, 1);
                f = __shfl(f, 0);
                if (f >= NF) break;
                operand_fragment(f);
            }
        }  // live
        // the next item's v, gate and beta
        if (next < sc.total) raw.load_va(p, itn.t0, itn.L, itn.h, tid);
        if (live) {
            lds_barrier();

            // ---- 3b. T = X Diag(beta) as MFMA operands: bf16, and hi/lo (q, A
            //          dead).  Columns (tokens) are stored in the kperm order of
            //          their 32-token step, so that the 8 values an MFMA lane
            //          takes are one 16-byte row piece: tokens 4g..4g+3 and
            //          16+4g..16+4g+3 of the step at positions 8g..8g+7.
            for (int e = tid; e < CP * CP / 4; e += 512) {
                const int r = e / (CP / 4), i4 = (e % (CP / 4)) * 4;
                // X is only defined on the lower block triangle of the C x C part
                const bool live = r < C && (i4 >> 4) <= (r >> 4);
                const f32x4 xv = live ? *reinterpret_cast<const f32x4 *>(&SX[r][i4]) : f32x4{0.f, 0.f, 0.f, 0.f};
                bf16_t tb[4], th[4], tl[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float t = xv[j] * SBETA[i4 + j];
                    tb[j] = f32_to_bf16(t * SNK[i4 + j]);  // W = T Diag(1/|k|) (k e^G)
                    split_bf16(t, th[j], tl[j]);
                }
                const int pos = (i4 & ~31) + 8 * ((i4 >> 2) & 3) + 4 * ((i4 >> 4) & 1);
                *reinterpret_cast<uint2 *>(&TB[r][pos]) = pack4(tb);
                *reinterpret_cast<uint2 *>(&TH[r][pos]) = pack4(th);
                *reinterpret_cast<uint2 *>(&TL[r][pos]) = pack4(tl);
            }
            lds_barrier();

            // ---- 4. W^T = (k e^G)^T T^T (bf16) per channel tile; U = T V (T split)
            //         per value tile.  Items: NDT W tiles then NDT U tiles.
            pend.blk = blk;
            pub = ready_index(p, it.x, it.h);
            for (int wi = wave; wi < 2 * Y::NDT; wi += 8) {
                const bool isW = wi < Y::NDT;
                const int ct = isW ? wi : wi - Y::NDT;
                f32x4 acc[Y::NMT];
#pragma unroll
                for (int tt = 0; tt < Y::NMT; ++tt) acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s2 = 0; s2 < Y::KSC; ++s2) {
                    // token k-step s2 in the kperm order: tokens iA..iA+3 and
                    // iA+16..iA+19 of the step for lane group g
                    const int iA = 32 * s2 + 4 * g;
                    frag8 opk;  // W: (k e^G)^T, channel row ch; U: V^T, value column ch
                    {
                        const bf16_t *src = isW ? &SKG[iA + li / 4][16 * ct + 4 * (li % 4)]
                                                : &SV[iA + li / 4][16 * ct + 4 * (li % 4)];
                        const uint2 lo4 = lds_read_tr16(src), hi4 = lds_read_tr16(src + 16 * M::RK);
                        opk.u = make_uint4(lo4.x, lo4.y, hi4.x, hi4.y);
                    }
#pragma unroll
                    for (int tt = 0; tt < Y::NMT; ++tt) {
                        if (32 * s2 > 16 * tt + 15) continue;
                        const int r = 16 * tt + li;
                        const int tp = 32 * s2 + 8 * g;   // this lane group's kperm piece
                        if (isW) {
                            frag8 tb;
                            tb.u = *reinterpret_cast<const uint4 *>(&TB[r][tp]);
                            acc[tt] = mfma16(opk.v, tb.v, acc[tt]);   // rows: channels, cols: tokens
                        } else {
                            frag8 th, tl;
                            th.u = *reinterpret_cast<const uint4 *>(&TH[r][tp]);
                            tl.u = *reinterpret_cast<const uint4 *>(&TL[r][tp]);
                            acc[tt] = mfma16(th.v, opk.v, acc[tt]);   // rows: tokens, cols: channels
                            acc[tt] = mfma16(tl.v, opk.v, acc[tt]);
                        }
                    }
                }
                // stored after the next item's staging (or at exit), so that the
                // staging's wait for its prefetched inputs does not also wait for
                // these stores to complete
#pragma unroll
                for (int tt = 0; tt < Y::NMT; ++tt) {
                    if (isW) {
                        bf16_t wb[4];
#pragma unroll
                        for (int j = 0; j < 4; ++j) wb[j] = f32_to_bf16(acc[tt][j]);
                        pend.w[tt] = pack4(wb);
                    } else {
                        pend.u[tt] = acc[tt];
                    }
                }
            }
            lds_barrier();  // LDS is restaged by the next item
        }  // live
        if (next >= sc.total) break;
        it = itn;
        const int after = next + sc.stride;
        nci = after < sc.total ? p.chunk_info[sc.item(after) / H] : make_int4(0, 0, 1, 0);
    }
    pend.flush(__builtin_amdgcn_readfirstlane(threadIdx.x >> 6), threadIdx.x & 63);
    if (PUB && pub >= 0) {
        wait_memory();
        lds_barrier();
        if (threadIdx.x == 0) publish_ready(ready + pub, xcc);
    }
}

// The per-chunk stage on its own: workgroup b computes items b, b + G, ...
// (G = gridDim.x) of the chunk-major order.
template <int C, int D>
__global__ void __launch_bounds__(512) intra_kernel(PrefillParams p, char *__restrict__ blocks) {
    __shared__ __attribute__((aligned(16))) char smem[IntraLds<C, D>::BYTES];
    if (*p.status != 0) return;
    const IntraSched sc{static_cast<int>(blockIdx.x), static_cast<int>(gridDim.x), p.chunk_off[p.N] * p.H, 0, 0,
                        p.H};
    intra_run<C, D, false>(p, blocks, smem, sc, nullptr, 0);
}

// ------------------------------------------------------------------ K2 --
// One wave's operands for one chunk, read from the chunk's workspace block in
// MFMA register order as 128-bit register tuples.  Wave w owns state rows
// [32w, 32w + 32): channel k-step w of the W S and (q e^G) S products and
// channel tiles 2w, 2w + 1 of the state update; it also finishes the output
// token tiles w, w + D/32, ...
template <int C, int D>
struct ScanOps {
    using Y = Lay<C, D>;
    static constexpr int NW = D / 32;
    static constexpr int OWN = (Y::NMT + NW - 1) / NW;
    typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
    u32x4 w[Y::NMT], qh[Y::NMT], ql[Y::NMT];   // token tile mt, channel step = wave
    u32x4 kh[2][Y::KSC], kl[2][Y::KSC];       // the wave's two channel tiles x token steps
    u32x4 ph[OWN][Y::KSC], pl[OWN][Y::KSC];   // owned token tiles x token steps
    f32x4 u[OWN];                             // owned token tiles, this column tile
    f32x4 gam[2];

    // blk: the chunk's block (uniform); lane16 = 16 * lane.  Four parts, so
    // that the requests can be spread over the previous chunk's computation.
    __device__ __forceinline__ void load(int part, const char *blk, uint32_t lane16, int wv, int nt, int g) {
        auto at = [&](size_t off) { return reinterpret_cast<const u32x4 *>(blk + off + lane16); };
        if (part == 0) {
#pragma unroll
            for (int mt = 0; mt < Y::NMT; ++mt) {
                const size_t fo = (static_cast<size_t>(mt) * Y::KSD + wv) * Y::FRAG;
                w[mt] = *at(Y::W + fo);
                qh[mt] = *at(Y::QH + fo);
                ql[mt] = *at(Y::QL + fo);
            }
        } else if (part == 1) {
#pragma unroll
            for (int uu = 0; uu < OWN; ++uu) {
                const int mt = wv + uu * NW;
                if (mt >= Y::NMT) continue;
                u[uu] = __builtin_bit_cast(f32x4, *at(Y::U + (static_cast<size_t>(mt) * Y::NDT + nt) * Y::FRAG));
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
                gam[i] = *reinterpret_cast<const f32x4 *>(blk + Y::GAM + (32 * wv + 16 * i + 4 * g) * sizeof(float));
        } else if (part == 2) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int st = 0; st < Y::KSC; ++st) {
                    const size_t fo = (static_cast<size_t>(2 * wv + i) * Y::KSC + st) * Y::FRAG;
                    kh[i][st] = *at(Y::KBH + fo);
                    kl[i][st] = *at(Y::KBL + fo);
                }
        } else {
#pragma unroll
            for (int uu = 0; uu < OWN; ++uu) {
                const int mt = wv + uu * NW;
                if (mt >= Y::NMT) continue;
#pragma unroll
                for (int st = 0; st < Y::KSC; ++st) {
                    if (32 * st > 16 * mt + 15) continue;  // zero above the diagonal
                    const size_t fo = (static_cast<size_t>(mt) * Y::KSC + st) * Y::FRAG;
                    ph[uu][st] = *at(Y::PH + fo);
                    pl[uu][st] = *at(Y::PL + fo);
                }
            }
        }
    }
    __device__ __forceinline__ void load(const char *blk, uint32_t lane16, int wv, int nt, int g) {
#pragma unroll
        for (int part = 0; part < 4; ++part) load(part, blk, lane16, wv, nt, g);
    }
};

template <int C, int D>
struct ScanShared {
    using Y = Lay<C, D>;
    f32x4 red[2][D / 32][Y::NMT][64];
    uint4 dls[Y::NMT][64];
};

__device__ __forceinline__ bf16x8 as_bf16x8(const ScanOps<64, 128>::u32x4 &u) { return __builtin_bit_cast(bf16x8, u); }

// One chunk of the scan for one wave: consumes the operands in `op` and
// updates the state tiles S in place.
// The next chunk's operands are requested into `nx` in four parts between
// the phases, so that the transfers overlap this chunk's computation.
// gate() runs before the first load of the next block (the overlapped
// launch waits there until that block is published).
template <int C, int D, typename TO, typename Gate>
__device__ __forceinline__ void scan_chunk(const ScanOps<C, D> &op, ScanOps<C, D> &nx, const char *nblk,
                                           uint32_t lane16, f32x4 (&S)[2], ScanShared<C, D> &sh,
                                           const PrefillParams &p, int64_t x, int64_t t0, int L, int h, int w,
                                           int nt, int lane, Gate &&gate) {
    using Y = Lay<C, D>;
    constexpr int NW = D / 32;
    constexpr int OWN = ScanOps<C, D>::OWN;
    const int g = lane >> 4, li = lane & 15;
    const int col = 16 * nt + li;
    const int H = p.H;
    if (p.chunk_states) {
        float *cs = p.chunk_states + (x * H + h) * static_cast<int64_t>(D) * D;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) cs[static_cast<int64_t>(32 * w + 16 * i + 4 * g + j) * D + col] = S[i][j];
    }
    // (a) this wave's state rows as a B operand, hi/lo
    frag8 sh_, sl_;
    acc2_to_split(S[0], S[1], sh_, sl_);
    // (b) partial W S (W and S both rounded to bf16: the product only reaches
    //     the outputs through Delta's first-order term) and (q e^G) S over this
    //     wave's 32 channels
#pragma unroll
    for (int mt = 0; mt < Y::NMT; ++mt) {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        sh.red[0][w][mt][lane] = mfma16(as_bf16x8(op.w[mt]), sh_.v, z);
        f32x4 pq = mfma16(as_bf16x8(op.qh[mt]), sh_.v, z);
        pq = mfma16(as_bf16x8(op.qh[mt]), sl_.v, pq);
        pq = mfma16(as_bf16x8(op.ql[mt]), sh_.v, pq);
        sh.red[1][w][mt][lane] = pq;
    }
    gate();
    nx.load(0, nblk, lane16, w, nt, g);
    lds_barrier();
    // (c) reduce the owned token tiles: Delta = U - sum_w W S
    f32x4 oq[OWN];
#pragma unroll
    for (int uu = 0; uu < OWN; ++uu) {
        const int mt = w + uu * NW;
        if (mt >= Y::NMT) continue;
        f32x4 d = op.u[uu];
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
            d -= sh.red[0][ww][mt][lane];
            acc += sh.red[1][ww][mt][lane];
        }
        oq[uu] = acc;
        bf16_t hi[4], lo[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) split_bf16(d[j], hi[j], lo[j]);
        const uint2 ph = pack4(hi), pl = pack4(lo);
        sh.dls[mt][lane] = make_uint4(ph.x, ph.y, pl.x, pl.y);
    }
    nx.load(1, nblk, lane16, w, nt, g);
    lds_barrier();
    // (d) Delta as B operands, one per 32-token step
    frag8 dh[Y::KSC], dl[Y::KSC];
#pragma unroll
    for (int st = 0; st < Y::KSC; ++st) {
        const uint4 a0 = sh.dls[2 * st][lane];
        const uint4 a1 = (2 * st + 1 < Y::NMT) ? sh.dls[2 * st + 1][lane] : make_uint4(0, 0, 0, 0);
        dh[st].u = make_uint4(a0.x, a0.y, a1.x, a1.y);
        dl[st].u = make_uint4(a0.z, a0.w, a1.z, a1.w);
    }
    // (e) state: S = e^{G_L} S + (k e^{G_L - G})^T Delta  (first: it carries
    //     the dependency into the next chunk)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        S[i] *= op.gam[i];
#pragma unroll
        for (int st = 0; st < Y::KSC; ++st) {
            S[i] = mfma16(as_bf16x8(op.kh[i][st]), dh[st].v, S[i]);
            S[i] = mfma16(as_bf16x8(op.kh[i][st]), dl[st].v, S[i]);
            S[i] = mfma16(as_bf16x8(op.kl[i][st]), dh[st].v, S[i]);
        }
    }
    nx.load(2, nblk, lane16, w, nt, g);
    // (f) outputs of the owned token tiles: O = (q e^G) S + P Delta
    TO *o = static_cast<TO *>(p.o);
#pragma unroll
    for (int uu = 0; uu < OWN; ++uu) {
        const int mt = w + uu * NW;
        if (mt >= Y::NMT) continue;
        f32x4 acc = oq[uu];
#pragma unroll
        for (int st = 0; st < Y::KSC; ++st) {
            if (32 * st > 16 * mt + 15) continue;
            acc = mfma16(as_bf16x8(op.ph[uu][st]), dh[st].v, acc);
            acc = mfma16(as_bf16x8(op.ph[uu][st]), dl[st].v, acc);
            acc = mfma16(as_bf16x8(op.pl[uu][st]), dh[st].v, acc);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int tok = 16 * mt + 4 * g + j;
            if (tok < L) io<TO>::st(o, ((t0 + tok) * H + h) * D + col, acc[j]);
        }
    }
    nx.load(3, nblk, lane16, w, nt, g);
}

// The scan of one (sequence, head) pair's 16-column state tile nt, with its
// LDS at sh; wave w = threadIdx.x / 64 < D / 32.  WAIT (the overlapped
// launch, one sequence): every block is read only after its flag is set,
// the L2 warm-up included (a line read before it is written could stay in
// this CU's L1).
template <int C, int D, typename TO, bool WAIT>
__device__ __forceinline__ void scan_run(const PrefillParams &p, const char *__restrict__ blocks,
                                         ScanShared<C, D> &sh, int pair, int nt, const int32_t *ready, int xcc) {
    using Y = Lay<C, D>;
    constexpr int NVT = D / 16;   // 16-column state tiles per head
    const int H = p.H;
    const int n = pair / H, h = pair % H;
    const SeqRange sr = seq_range(p, n);
    const int nch = (sr.len + C - 1) / C;
    const int64_t cbase = p.chunk_off[n];
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, li = lane & 15;
    const int col = 16 * nt + li;

    const int64_t soff = (static_cast<int64_t>(n) * H + h) * D * D;
    f32x4 S[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = 32 * w + 16 * i + 4 * g + j;
            S[i][j] = p.initial_state ? p.initial_state[soff + static_cast<int64_t>(row) * D + col] : 0.f;
        }

    auto blk_of = [&](int c) {
        return blocks + (static_cast<size_t>(cbase + c) * H + h) * Y::BYTES;
    };
    // Every operand of chunk c + 1 is requested while chunk c is computed
    // (two buffers, alternating); chunk indices are clamped, so every load is
    // inside the sequence's blocks.  Waves exchange data through LDS only.
    // L2 warm-up: while chunk c is computed, the column tiles of the head
    // together touch every 128-byte line of chunk c + kWarmAhead's block (one
    // dword per line, this workgroup's eighth), so that block is in L2 before
    // its operands are requested; the loaded word is only consumed (without
    // instructions) two chunks later (two registers, by chunk parity), so the
    // wait for it is free.
    constexpr int kWarmAhead = 2;
    constexpr int kLines = static_cast<int>(Y::BYTES / 128);
    constexpr int kSlots = NVT * (D / 32) * 64;  // lanes of all the head's workgroups
    const uint32_t warm_off = static_cast<uint32_t>(((nt * (D / 32) + w) * 64 + lane) * kLines / kSlots) * 128u;
    uint32_t warmA = 0, warmB = 0;
    auto warm_up = [&](uint32_t &warm, int c) {
        asm volatile("" ::"v"(warm));
        warm = *reinterpret_cast<const uint32_t *>(blk_of(min(c + kWarmAhead, nch - 1)) + warm_off);
    };
    // WAIT: a block is warmed only when its writers are at least
    // kWarmPublished chunks further on (it may have left the L2 since it was
    // written); closer behind them the warm-up measured slower than none.
    constexpr int kWarmPublished = 16;
    ScanOps<C, D> A, B;
    if (nch > 0) {
        const uint32_t lane16 = 16u * lane;
        ReadyView rv{WAIT ? ready + ready_index(p, 0, h) : nullptr, nch, WAIT ? 0 : nch, xcc};
        if (WAIT) rv.ensure(0, p);
        A.load(blk_of(0), lane16, w, nt, g);
        for (int c = 0; c < nch; c += 2) {
            if (!WAIT || min(c + kWarmAhead, nch - 1) + kWarmPublished < rv.known) warm_up(warmA, c);
            scan_chunk<C, D, TO>(A, B, blk_of(min(c + 1, nch - 1)), lane16, S, sh, p, cbase + c,
                                 sr.start + static_cast<int64_t>(c) * C, min(C, sr.len - c * C), h, w, nt, lane,
                                 [&] { if (WAIT) rv.ensure(min(c + 1, nch - 1), p); });
            if (c + 1 >= nch) break;
            if (!WAIT || min(c + 1 + kWarmAhead, nch - 1) + kWarmPublished < rv.known) warm_up(warmB, c + 1);
            scan_chunk<C, D, TO>(B, A, blk_of(min(c + 2, nch - 1)), lane16, S, sh, p, cbase + c + 1,
                                 sr.start + static_cast<int64_t>(c + 1) * C, min(C, sr.len - (c + 1) * C), h, w, nt,
                                 lane, [&] { if (WAIT) rv.ensure(min(c + 2, nch - 1), p); });
        }
        asm volatile("" ::"v"(warmA), "v"(warmB));
    }
    if (p.final_state) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                p.final_state[soff + static_cast<int64_t>(32 * w + 16 * i + 4 * g + j) * D + col] = S[i][j];
    }
}

// -------------------------------------------------- K2, NT tiles per WG --
// The same scan for a workgroup that owns NT > 1 adjacent column tiles of a
// head (the launch picks NT; see scan_tiles_per_workgroup).  Each tile's
// arithmetic is the one-tile code's, so the results are bitwise equal.  The
// one-tile functions above are kept as they are: written in this generic
// form, their one-tile instance was scheduled differently by the compiler
// and ran 4 % slower (3.64 against 3.50 ms on the T=131072, H=32 workload).
// One wave's operands for one chunk, read from the chunk's workspace block in
// MFMA register order as 128-bit register tuples.  A workgroup owns NT
// adjacent 16-column state tiles of one head (columns [16 NT g, 16 NT g +
// 16 NT) for tile group g); wave w owns state rows [32w, 32w + 32) of each:
// channel k-step w of the W S and (q e^G) S products and channel tiles 2w,
// 2w + 1 of the state update; it also finishes the output token tiles w,
// w + D/32, ...  The W, q e^G, k e^{G_L-G} and P operands are shared by the
// NT tiles (loaded once); U is per tile.
template <int C, int D, int NT>
struct WideScanOps {
    using Y = Lay<C, D>;
    static constexpr int NW = D / 32;
    static constexpr int OWN = (Y::NMT + NW - 1) / NW;
    typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
    u32x4 w[Y::NMT], qh[Y::NMT], ql[Y::NMT];   // token tile mt, channel step = wave
    u32x4 kh[2][Y::KSC], kl[2][Y::KSC];       // the wave's two channel tiles x token steps
    u32x4 ph[OWN][Y::KSC], pl[OWN][Y::KSC];   // owned token tiles x token steps
    f32x4 u[NT][OWN];                         // the group's column tiles x owned token tiles
    f32x4 gam[2];

    // blk: the chunk's block (uniform); lane16 = 16 * lane; ng: tile group.
    // Four parts, so that the requests can be spread over the previous
    // chunk's computation.
    __device__ __forceinline__ void load(int part, const char *blk, uint32_t lane16, int wv, int ng, int g) {
        auto at = [&](size_t off) { return reinterpret_cast<const u32x4 *>(blk + off + lane16); };
        if (part == 0) {
#pragma unroll
            for (int mt = 0; mt < Y::NMT; ++mt) {
                const size_t fo = (static_cast<size_t>(mt) * Y::KSD + wv) * Y::FRAG;
                w[mt] = *at(Y::W + fo);
                qh[mt] = *at(Y::QH + fo);
                ql[mt] = *at(Y::QL + fo);
            }
        } else if (part == 1) {
#pragma unroll
            for (int j = 0; j < NT; ++j)
#pragma unroll
                for (int uu = 0; uu < OWN; ++uu) {
                    const int mt = wv + uu * NW;
                    if (mt >= Y::NMT) continue;
                    u[j][uu] = __builtin_bit_cast(
                        f32x4, *at(Y::U + (static_cast<size_t>(mt) * Y::NDT + NT * ng + j) * Y::FRAG));
                }
#pragma unroll
            for (int i = 0; i < 2; ++i)
                gam[i] = *reinterpret_cast<const f32x4 *>(blk + Y::GAM + (32 * wv + 16 * i + 4 * g) * sizeof(float));
        } else if (part == 2) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int st = 0; st < Y::KSC; ++st) {
                    const size_t fo = (static_cast<size_t>(2 * wv + i) * Y::KSC + st) * Y::FRAG;
                    kh[i][st] = *at(Y::KBH + fo);
                    kl[i][st] = *at(Y::KBL + fo);
                }
        } else {
#pragma unroll
            for (int uu = 0; uu < OWN; ++uu) {
                const int mt = wv + uu * NW;
                if (mt >= Y::NMT) continue;
#pragma unroll
                for (int st = 0; st < Y::KSC; ++st) {
                    if (32 * st > 16 * mt + 15) continue;  // zero above the diagonal
                    const size_t fo = (static_cast<size_t>(mt) * Y::KSC + st) * Y::FRAG;
                    ph[uu][st] = *at(Y::PH + fo);
                    pl[uu][st] = *at(Y::PL + fo);
                }
            }
        }
    }
    __device__ __forceinline__ void load(const char *blk, uint32_t lane16, int wv, int ng, int g) {
#pragma unroll
        for (int part = 0; part < 4; ++part) load(part, blk, lane16, wv, ng, g);
    }
};

template <int C, int D, int NT>
struct WideScanShared {
    using Y = Lay<C, D>;
    f32x4 red[NT][2][D / 32][Y::NMT][64];
    uint4 dls[NT][Y::NMT][64];
};

// One chunk of the scan for one wave: consumes the operands in `op` and
// updates the state tiles S (one pair per column tile of the group) in place.
// The next chunk's operands are requested into `nx` in four parts between
// the phases, so that the transfers overlap this chunk's computation.
// gate() runs before the first load of the next block (the overlapped
// launch waits there until that block is published).
template <int C, int D, typename TO, int NT, typename Gate>
__device__ __forceinline__ void wide_scan_chunk(const WideScanOps<C, D, NT> &op, WideScanOps<C, D, NT> &nx, const char *nblk,
                                           uint32_t lane16, f32x4 (&S)[NT][2], WideScanShared<C, D, NT> &sh,
                                           const PrefillParams &p, int64_t x, int64_t t0, int L, int h, int w,
                                           int ng, int lane, Gate &&gate) {
    using Y = Lay<C, D>;
    constexpr int NW = D / 32;
    constexpr int OWN = WideScanOps<C, D, NT>::OWN;
    const int g = lane >> 4, li = lane & 15;
    const int col0 = 16 * NT * ng + li;   // column of tile j: col0 + 16 j
    const int H = p.H;
    if (p.chunk_states) {
        float *cs = p.chunk_states + (x * H + h) * static_cast<int64_t>(D) * D;
#pragma unroll
        for (int jt = 0; jt < NT; ++jt)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    cs[static_cast<int64_t>(32 * w + 16 * i + 4 * g + j) * D + col0 + 16 * jt] = S[jt][i][j];
    }
#pragma unroll
    for (int jt = 0; jt < NT; ++jt) {
        // (a) this wave's state rows as a B operand, hi/lo
        frag8 sh_, sl_;
        acc2_to_split(S[jt][0], S[jt][1], sh_, sl_);
        // (b) partial W S (W and S both rounded to bf16: the product only
        //     reaches the outputs through Delta's first-order term) and
        //     (q e^G) S over this wave's 32 channels
#pragma unroll
        for (int mt = 0; mt < Y::NMT; ++mt) {
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            sh.red[jt][0][w][mt][lane] = mfma16(as_bf16x8(op.w[mt]), sh_.v, z);
            f32x4 pq = mfma16(as_bf16x8(op.qh[mt]), sh_.v, z);
            pq = mfma16(as_bf16x8(op.qh[mt]), sl_.v, pq);
            pq = mfma16(as_bf16x8(op.ql[mt]), sh_.v, pq);
            sh.red[jt][1][w][mt][lane] = pq;
        }
    }
    gate();
    nx.load(0, nblk, lane16, w, ng, g);
    lds_barrier();
    // (c) reduce the owned token tiles: Delta = U - sum_w W S
    f32x4 oq[NT][OWN];
#pragma unroll
    for (int jt = 0; jt < NT; ++jt)
#pragma unroll
        for (int uu = 0; uu < OWN; ++uu) {
            const int mt = w + uu * NW;
            if (mt >= Y::NMT) continue;
            f32x4 d = op.u[jt][uu];
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) {
                d -= sh.red[jt][0][ww][mt][lane];
                acc += sh.red[jt][1][ww][mt][lane];
            }
            oq[jt][uu] = acc;
            bf16_t hi[4], lo[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) split_bf16(d[j], hi[j], lo[j]);
            const uint2 ph = pack4(hi), pl = pack4(lo);
            sh.dls[jt][mt][lane] = make_uint4(ph.x, ph.y, pl.x, pl.y);
        }
    nx.load(1, nblk, lane16, w, ng, g);
    lds_barrier();
    TO *o = static_cast<TO *>(p.o);
#pragma unroll
    for (int jt = 0; jt < NT; ++jt) {
        // (d) Delta as B operands, one per 32-token step
        frag8 dh[Y::KSC], dl[Y::KSC];
#pragma unroll
        for (int st = 0; st < Y::KSC; ++st) {
            const uint4 a0 = sh.dls[jt][2 * st][lane];
            const uint4 a1 = (2 * st + 1 < Y::NMT) ? sh.dls[jt][2 * st + 1][lane] : make_uint4(0, 0, 0, 0);
            dh[st].u = make_uint4(a0.x, a0.y, a1.x, a1.y);
            dl[st].u = make_uint4(a0.z, a0.w, a1.z, a1.w);
        }
        // (e) state: S = e^{G_L} S + (k e^{G_L - G})^T Delta  (first: it
        //     carries the dependency into the next chunk)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            S[jt][i] *= op.gam[i];
#pragma unroll
            for (int st = 0; st < Y::KSC; ++st) {
                S[jt][i] = mfma16(as_bf16x8(op.kh[i][st]), dh[st].v, S[jt][i]);
                S[jt][i] = mfma16(as_bf16x8(op.kh[i][st]), dl[st].v, S[jt][i]);
                S[jt][i] = mfma16(as_bf16x8(op.kl[i][st]), dh[st].v, S[jt][i]);
            }
        }
        if (jt == 0) nx.load(2, nblk, lane16, w, ng, g);
        // (f) outputs of the owned token tiles: O = (q e^G) S + P Delta
#pragma unroll
        for (int uu = 0; uu < OWN; ++uu) {
            const int mt = w + uu * NW;
            if (mt >= Y::NMT) continue;
            f32x4 acc = oq[jt][uu];
#pragma unroll
            for (int st = 0; st < Y::KSC; ++st) {
                if (32 * st > 16 * mt + 15) continue;
                acc = mfma16(as_bf16x8(op.ph[uu][st]), dh[st].v, acc);
                acc = mfma16(as_bf16x8(op.ph[uu][st]), dl[st].v, acc);
                acc = mfma16(as_bf16x8(op.pl[uu][st]), dh[st].v, acc);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int tok = 16 * mt + 4 * g + j;
                if (tok < L) io<TO>::st(o, ((t0 + tok) * H + h) * D + col0 + 16 * jt, acc[j]);
            }
        }
    }
    nx.load(3, nblk, lane16, w, ng, g);
}

// The scan of one (sequence, head) pair's tile group ng (NT 16-column state
// tiles), with its LDS at sh; wave w = threadIdx.x / 64 < D / 32.  WAIT (the
// overlapped launch, one sequence): every block is read only after its flag
// is set, the L2 warm-up included (a line read before it is written could
// stay in this CU's L1).
template <int C, int D, typename TO, bool WAIT, int NT>
__device__ __forceinline__ void wide_scan_run(const PrefillParams &p, const char *__restrict__ blocks,
                                         WideScanShared<C, D, NT> &sh, int pair, int ng, const int32_t *ready,
                                         int xcc) {
    using Y = Lay<C, D>;
    constexpr int NG = D / 16 / NT;   // tile groups per head
    const int H = p.H;
    const int n = pair / H, h = pair % H;
    const SeqRange sr = seq_range(p, n);
    const int nch = (sr.len + C - 1) / C;
    const int64_t cbase = p.chunk_off[n];
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, li = lane & 15;
    const int col0 = 16 * NT * ng + li;

    const int64_t soff = (static_cast<int64_t>(n) * H + h) * D * D;
    f32x4 S[NT][2];
#pragma unroll
    for (int jt = 0; jt < NT; ++jt)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 32 * w + 16 * i + 4 * g + j;
                S[jt][i][j] =
                    p.initial_state ? p.initial_state[soff + static_cast<int64_t>(row) * D + col0 + 16 * jt] : 0.f;
            }

    auto blk_of = [&](int c) {
        return blocks + (static_cast<size_t>(cbase + c) * H + h) * Y::BYTES;
    };
    // Every operand of chunk c + 1 is requested while chunk c is computed
    // (two buffers, alternating); chunk indices are clamped, so every load is
    // inside the sequence's blocks.  Waves exchange data through LDS only.
    // L2 warm-up: while chunk c is computed, the tile groups of the head
    // together touch every 128-byte line of chunk c + kWarmAhead's block
    // (one dword per line; KW lines per lane when the head's lanes are fewer
    // than its lines), so that block is in L2 before its operands are
    // requested; the loaded words are only consumed (without instructions)
    // two chunks later (two register sets, by chunk parity), so the wait for
    // them is free.
    constexpr int kWarmAhead = 2;
    constexpr int kLines = static_cast<int>(Y::BYTES / 128);
    constexpr int kLanes = NG * (D / 32) * 64;  // lanes of all the head's workgroups
    constexpr int KW = (kLines + kLanes - 1) / kLanes;
    constexpr int kSlots = kLanes * KW;
    const int slot0 = ((ng * (D / 32) + w) * 64 + lane) * KW;
    uint32_t warmA[KW], warmB[KW];
#pragma unroll
    for (int k = 0; k < KW; ++k) warmA[k] = warmB[k] = 0;
    auto warm_up = [&](uint32_t (&warm)[KW], int c) {
        const char *wb = blk_of(min(c + kWarmAhead, nch - 1));
#pragma unroll
        for (int k = 0; k < KW; ++k) {
            asm volatile("" ::"v"(warm[k]));
            warm[k] = *reinterpret_cast<const uint32_t *>(
                wb + static_cast<uint32_t>((slot0 + k) * kLines / kSlots) * 128u);
        }
    };
    // WAIT: a block is warmed only when its writers are at least
    // kWarmPublished chunks further on (it may have left the L2 since it was
    // written); closer behind them the warm-up measured slower than none.
    constexpr int kWarmPublished = 16;
    WideScanOps<C, D, NT> A, B;
    if (nch > 0) {
        const uint32_t lane16 = 16u * lane;
        ReadyView rv{WAIT ? ready + ready_index(p, 0, h) : nullptr, nch, WAIT ? 0 : nch, xcc};
        if (WAIT) rv.ensure(0, p);
        A.load(blk_of(0), lane16, w, ng, g);
        for (int c = 0; c < nch; c += 2) {
            if (!WAIT || min(c + kWarmAhead, nch - 1) + kWarmPublished < rv.known) warm_up(warmA, c);
            wide_scan_chunk<C, D, TO, NT>(A, B, blk_of(min(c + 1, nch - 1)), lane16, S, sh, p, cbase + c,
                                     sr.start + static_cast<int64_t>(c) * C, min(C, sr.len - c * C), h, w, ng, lane,
                                     [&] { if (WAIT) rv.ensure(min(c + 1, nch - 1), p); });
            if (c + 1 >= nch) break;
            if (!WAIT || min(c + 1 + kWarmAhead, nch - 1) + kWarmPublished < rv.known) warm_up(warmB, c + 1);
            wide_scan_chunk<C, D, TO, NT>(B, A, blk_of(min(c + 2, nch - 1)), lane16, S, sh, p, cbase + c + 1,
                                     sr.start + static_cast<int64_t>(c + 1) * C, min(C, sr.len - (c + 1) * C), h, w,
                                     ng, lane, [&] { if (WAIT) rv.ensure(min(c + 2, nch - 1), p); });
        }
#pragma unroll
        for (int k = 0; k < KW; ++k) asm volatile("" ::"v"(warmA[k]), "v"(warmB[k]));
    }
    if (p.final_state) {
#pragma unroll
        for (int jt = 0; jt < NT; ++jt)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    p.final_state[soff + static_cast<int64_t>(32 * w + 16 * i + 4 * g + j) * D + col0 + 16 * jt] =
                        S[jt][i][j];
    }
}

template <int C, int D, typename TO, int NT>
__global__ void __launch_bounds__(64 * (D / 32)) scan_kernel(PrefillParams p, const char *__restrict__ blocks) {
    constexpr int NG = D / 16 / NT;   // tile groups per head
    using Shared = typename std::conditional<NT == 1, ScanShared<C, D>, WideScanShared<C, D, NT>>::type;
    __shared__ Shared sh;
    if (*p.status != 0) return;
    // XCD-aware order: the NG tile groups of one (sequence, head) share
    // blockIdx % 8, hence one XCD and its L2.
    const int bid = blockIdx.x;
    const int xcd = bid & 7, slot = bid >> 3;
    const int ng = slot % NG;
    const int pair = xcd + 8 * (slot / NG);
    if (pair >= p.N * p.H) return;
    if constexpr (NT == 1)
        scan_run<C, D, TO, false>(p, blocks, sh, pair, ng, nullptr, 0);
    else
        wide_scan_run<C, D, TO, false, NT>(p, blocks, sh, pair, ng, nullptr, 0);
}

// ---------------------------------------------------- overlapped launch --
// For one sequence whose scan would leave most CUs idle (at most
// kOverlapScanSlots column-tile workgroups per XCD), the two stages run in
// one launch of 8 x kOverlapSlots workgroups, one per CU.  The hardware
// deals a launch's workgroups to the 8 XCDs round-robin, but from an XCD
// that depends on earlier launches, so roles follow the XCD a workgroup
// finds itself on (xcc_id()) and its arrival there: it takes the next
// ticket of its XCD's counter.  On XCD x the first SI arrivals compute the
// per-chunk stage of the heads h = x + 8j, chunk by chunk (the order in
// which the scan consumes them), and publish each block; the next
// NVT x (number of those heads) arrivals run their scans, each reading a
// block as soon as its flag is set, so the scan no longer waits for the
// whole per-chunk stage.  Producers never wait and take the first tickets,
// so the consumers' waits end however many workgroups are resident.  Every
// role is taken once when each XCD receives kOverlapSlots workgroups (the
// round-robin deal); a workgroup that finds its XCD's roles all taken
// records kErrDeviceWait and leaves (a role of another XCD then has no
// workgroup, and the call's results are undefined).
constexpr int kOverlapSlots = 32;      // workgroups per XCD (its CUs)
constexpr int kOverlapScanSlots = 16;  // at most this many scan workgroups per XCD

template <int C, int D, typename TO>
__global__ void __launch_bounds__(512) overlap_kernel(PrefillParams p, char *__restrict__ blocks) {
    constexpr int NVT = D / 16;
    constexpr size_t LDS =
        IntraLds<C, D>::BYTES > sizeof(ScanShared<C, D>) ? IntraLds<C, D>::BYTES : sizeof(ScanShared<C, D>);
    __shared__ __attribute__((aligned(16))) char smem[LDS];
    __shared__ int s_slot;
    if (*p.status != 0) return;
    const int x = xcc_id();
    if (threadIdx.x == 0)
        s_slot = __hip_atomic_fetch_add(p.ready + x, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int slot = s_slot;
    if (slot >= kOverlapSlots) {
        if (threadIdx.x == 0) report_device_error(p, kErrDeviceWait);
        return;
    }
    const int H = p.H;  // one sequence: (sequence, head) pair = head
    const int npx = x < H ? (H - x + 7) / 8 : 0;
    const int si = kOverlapSlots - npx * NVT;
    if (slot < si) {
        const IntraSched sc{slot, si, npx * p.chunk_off[1], npx, x, H};
        intra_run<C, D, true>(p, blocks, smem, sc, p.ready, x);
    } else {
        if (threadIdx.x >= 64 * (D / 32)) return;  // the scan's D/32 waves
        const int s = slot - si;
        scan_run<C, D, TO, true>(p, blocks, *reinterpret_cast<ScanShared<C, D> *>(smem), x + 8 * (s / NVT), s % NVT,
                                 p.ready, x);
    }
}

// ---------------------------------------------------------------- host --
bool mfma_overlap_shape(int N, int H, int D, int C) {
    return N == 1 && C == 64 && (H + 7) / 8 * (D / 16) <= kOverlapScanSlots;
}

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
// Column tiles per scan workgroup.  A workgroup's time per chunk grows with
// its tile count (the tiles' products, reductions and exchanges run one
// after another in each wave: 1.77, 2.70 and 4.97 us per chunk at 1, 2, 4
// tiles on the T=131072, H=32 workload), while sharing the block's W, q e^G,
// k e^{G_L-G} and P loads saves the CUs work.  So one tile per workgroup
// while the grid does not fill the CUs, else the most tiles for which it
// still gives every CU a workgroup.
int scan_tiles_per_workgroup(int pairs, int D) {
    const long tiles = static_cast<long>(pairs) * (D / 16);
    if (tiles >= 4L * kIntraGrid) return 4;
    if (tiles >= 2L * kIntraGrid) return 2;
    return 1;
}

template <int C, int D, typename TO, int NT>
hipError_t launch_scan(const PrefillParams &p, char *blocks, hipStream_t s) {
    constexpr int NG = D / 16 / NT;   // tile groups per head
    const int pairs = p.N * p.H;
    const unsigned grid = static_cast<unsigned>((pairs + 7) / 8) * NG * 8;
    hipLaunchKernelGGL((scan_kernel<C, D, TO, NT>), dim3(grid), dim3(64 * (D / 32)), 0, s, p,
                       static_cast<const char *>(blocks));
    return hipGetLastError();
}

template <int C, int D, typename TO>
hipError_t run_mfma(const PrefillParams &p, char *blocks, hipStream_t s, hipEvent_t mid) {
    if constexpr (C == 64) {
        if (p.ready) {
            hipLaunchKernelGGL((overlap_kernel<C, D, TO>), dim3(8 * kOverlapSlots), dim3(512), 0, s, p, blocks);
            hipError_t e = hipGetLastError();
            if (e == hipSuccess && mid) e = hipEventRecord(mid, s);
            return e;
        }
    }
    const int items = p.n_chunks_bound * p.H;  // upper bound; the kernel reads the exact count
    const int igrid = items < kIntraGrid ? items : kIntraGrid;
    hipLaunchKernelGGL((intra_kernel<C, D>), dim3(igrid), dim3(512), 0, s, p, blocks);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && mid) e = hipEventRecord(mid, s);
    if (e != hipSuccess) return e;
    const int pairs = p.N * p.H;
    if constexpr (C == 64 && D == 128) {   // measured there
        const int nt = scan_tiles_per_workgroup(pairs, D);
        if (nt == 4) return launch_scan<C, D, TO, 4>(p, blocks, s);
        if (nt == 2) return launch_scan<C, D, TO, 2>(p, blocks, s);
    }
    return launch_scan<C, D, TO, 1>(p, blocks, s);
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
