// Chunked KDA prefill in fp32 on the fp32 matrix cores (v_mfma_f32_16x16x4_f32:
// fp32 products and fp32 sums), for fp32 inputs (the 1e-5 contract) and for
// head sizes the bf16 matrix-core path does not take.
//
// Module 04 — KDA II: Chunked Parallelism & the Full Sublayer, §1 "The
// recurrence has affine form": each chunk's transition is formed from the
// chunk alone, in structured form, and the chunks are then applied in order.
// For a chunk of L tokens with incoming state S (K~ = k e^G, Q~ = q e^G,
// K^ = k e^{G_L - G}, g = e^{G_L}, M = (I + Diag(beta) Gh)^-1):
//     X = V - K~ S,   Delta = M Diag(beta) X,   O = Q~ S + P Delta,
//     S' = Diag(g) S + K^^T Delta.
// Two kernels: the chunk prep kernel (forward mode; one workgroup per
// (chunk, head), shared with the chunked backward; it also applies the
// fused prologue) writes K~, Q~, K^, g, beta, P and M per (chunk, head); the scan below walks each sequence's
// chunks in order, one workgroup per (sequence, head, 16-column tile of S).
#include "kda_chunk_block.hpp"
#include "kda_chunk_prep.hpp"
#include "kda_handoff.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {

// 16 x 16 x 16 block product on fp32 matrix cores: in step s lane l
// (g = l / 16, n = l % 16) supplies A[n][4g + s] = a[s] and B[4g + s][n] = b[s];
// the lane holds D[4g + u][n] in acc[u].
__device__ __forceinline__ f32x4 mmf32(const f32x4 &a, const f32x4 &b, f32x4 acc) {
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], acc, 0, 0, 0);
    return acc;
}

}  // namespace

// One wave's operands of one chunk (token block w, key blocks w, w + 4),
// loaded into registers a chunk ahead: each part is reloaded for the next
// chunk right after the current chunk's products have used it.  The forward
// prep stores K~, Q~ and M in fragment order (frag_a), so each of those
// loads is one contiguous 1 KB per wave (row-major, a 16-byte-per-lane load
// touches 16 cache lines); P and K^ stay row-major (their fragment-order
// stores cost the prep more than they saved here).
template <int DK, typename TI>
struct F32ScanOps {
    using Y = CbLay<DK>;
    static constexpr int NKB = DK / 16, KPW = (NKB + 3) / 4;
    f32x4 kt[NKB], qt[NKB];   // K~, Q~ [16w + n][16cb + 4g ..]           (step 1)
    float vv[4];              // V [16w + 4g + u][j0 + n]                 (step 1)
    f32x4 mb[4], pb[4];       // M Diag(beta), P [16w + n][16ib + 4g ..]  (steps 2, 3)
    f32x4 ka[KPW][4];         // K^ [16rb + 4g + s][16kb + n], kb = w + 4i (step 4)
    f32x4 gm[KPW];            // e^{G_L} [16kb + 4g ..]                   (step 4)

    __device__ __forceinline__ void load1(const float *blk, const TI *v, int64_t t0, int L, int H, int h, int dv,
                                          int j0, int w, int g, int n) {
        const int lane = 16 * g + n;
#pragma unroll
        for (int cb = 0; cb < NKB; ++cb) {
            kt[cb] = *reinterpret_cast<const f32x4 *>(blk + Y::KT + ((w * NKB + cb) * 64 + lane) * 4);
            qt[cb] = *reinterpret_cast<const f32x4 *>(blk + Y::QT + ((w * NKB + cb) * 64 + lane) * 4);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int r = 16 * w + 4 * g + u;
            vv[u] = r < L ? io<TI>::ld(v, ((t0 + r) * H + h) * dv + j0 + n) : 0.f;
        }
    }
    __device__ __forceinline__ void load23(const float *blk, int w, int g, int n) {
        const int lane = 16 * g + n;
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) {
            if (ib > w) continue;
            const f32x4 m4 = *reinterpret_cast<const f32x4 *>(blk + Y::M + ((w * 4 + ib) * 64 + lane) * 4);
            mb[ib] = m4 * *reinterpret_cast<const f32x4 *>(blk + Y::BETA + 16 * ib + 4 * g);
            pb[ib] = *reinterpret_cast<const f32x4 *>(blk + Y::P + (16 * w + n) * CB_C + 16 * ib + 4 * g);
        }
    }
    __device__ __forceinline__ void load4(const float *blk, int w, int g, int n) {
#pragma unroll
        for (int i = 0; i < KPW; ++i) {
            const int kb = w + 4 * i;
            if (kb >= NKB) continue;
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2) ka[i][rb][s2] = blk[Y::KB + (16 * rb + 4 * g + s2) * DK + 16 * kb + n];
            gm[i] = *reinterpret_cast<const f32x4 *>(blk + Y::GAM + 16 * kb + 4 * g);
        }
    }
};

// The scan of one (sequence, head) pair's 16-column state tile vt; 4 waves.
// Wave w computes token block w of X, Delta and O and owns key blocks
// w, w + 4 of the state (accumulator layout, for the whole sequence).  S, X
// and Delta pass between the waves through LDS transposed ([column][row]),
// so a lane's four contraction values are one 16-byte read.  Inside the
// walk the waves meet at LDS-only barriers: __syncthreads() would also wait
// for the next chunk's operand loads and drain the prefetch.  WAIT (the
// overlapped launch, one sequence): a block's first load waits until its
// flag is set.
template <int DK, typename TI, typename TO, bool WAIT>
__device__ __forceinline__ void f32mm_scan_run(const PrefillParams &p, const float *__restrict__ blocks, int pair,
                                               int vt, const int32_t *ready, int xcc) {
    using Y = CbLay<DK>;
    using Ops = F32ScanOps<DK, TI>;
    constexpr int C = CB_C, NKB = Ops::NKB, KPW = Ops::KPW;
    constexpr int LC = C + 4, LK = DK + 4;  // padded strides of the [column][row] tiles
    const int H = p.H, dv = p.dv;
    const int h = pair % H, n_seq = pair / H;
    const int j0 = 16 * vt;
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, n = lane & 15;
    const SeqRange sr = seq_range(p, n_seq);
    const int64_t cbase = p.chunk_off[n_seq];
    const int nch = p.chunk_off[n_seq + 1] - p.chunk_off[n_seq];
    const TI *v = static_cast<const TI *>(p.v);
    TO *o = static_cast<TO *>(p.o);

    __shared__ __attribute__((aligned(16))) float sT[16][LK];   // S^T
    __shared__ __attribute__((aligned(16))) float xT[16][LC];   // X^T
    __shared__ __attribute__((aligned(16))) float dT[16][LC];   // Delta^T

    const int64_t soff = (static_cast<int64_t>(n_seq) * H + h) * DK * dv;
    f32x4 st[KPW];
#pragma unroll
    for (int i = 0; i < KPW; ++i) {
        const int kb = w + 4 * i;
#pragma unroll
        for (int u = 0; u < 4; ++u)
            st[i][u] = (kb < NKB && p.initial_state)
                           ? p.initial_state[soff + static_cast<int64_t>(16 * kb + 4 * g + u) * dv + j0 + n]
                           : 0.f;
        if (kb < NKB) *reinterpret_cast<f32x4 *>(&sT[n][16 * kb + 4 * g]) = st[i];
    }
    auto blk_of = [&](int ch) { return blocks + (static_cast<size_t>(cbase + ch) * H + h) * Y::FLOATS; };
    auto len_of = [&](int ch) { return min(p.C, sr.len - ch * p.C); };
    auto t0_of = [&](int ch) { return sr.start + static_cast<int64_t>(ch) * p.C; };
    Ops op;
    ReadyView rv{WAIT ? ready + ready_index(p, 0, h) : nullptr, nch, WAIT ? 0 : nch, xcc};
    if (nch > 0) {
        if (WAIT) rv.ensure(0, p);
        op.load1(blk_of(0), v, t0_of(0), len_of(0), H, h, dv, j0, w, g, n);
        op.load23(blk_of(0), w, g, n);
        op.load4(blk_of(0), w, g, n);
    }
    __syncthreads();

    for (int ch = 0; ch < nch; ++ch) {
        const int64_t x = cbase + ch;
        const int64_t t0 = t0_of(ch);
        const int L = len_of(ch);
        const int nx = ch + 1 < nch ? ch + 1 : ch;   // the chunk whose operands are loaded next
        if (p.chunk_states) {
            float *cs = p.chunk_states + (x * H + h) * static_cast<int64_t>(DK) * dv;
#pragma unroll
            for (int i = 0; i < KPW; ++i) {
                const int kb = w + 4 * i;
                if (kb >= NKB) continue;
#pragma unroll
                for (int u = 0; u < 4; ++u) cs[static_cast<int64_t>(16 * kb + 4 * g + u) * dv + j0 + n] = st[i][u];
            }
        }
        // Token blocks at or beyond L hold only zeros (the prep zeroes those
        // rows): their waves skip steps 1-3 and no product reads them.
        const int r0 = 16 * w;
        const bool live = r0 < L;
        const int nb = (L + 15) / 16;   // live token blocks (uniform)
        // (1) token block w: X = V - K~ S and (q e^G) S
        f32x4 xa = {0.f, 0.f, 0.f, 0.f}, oa = xa;
#pragma unroll
        for (int cb = 0; cb < NKB; ++cb) {
            if (!live) break;
            const f32x4 sb = *reinterpret_cast<const f32x4 *>(&sT[n][16 * cb + 4 * g]);
            xa = mmf32(op.kt[cb], sb, xa);
            oa = mmf32(op.qt[cb], sb, oa);
        }
        f32x4 xv;
#pragma unroll
        for (int u = 0; u < 4; ++u) xv[u] = op.vv[u] - xa[u];
        if (live) *reinterpret_cast<f32x4 *>(&xT[n][r0 + 4 * g]) = xv;
        if (WAIT) rv.ensure(nx, p);
        op.load1(blk_of(nx), v, t0_of(nx), len_of(nx), H, h, dv, j0, w, g, n);
        lds_barrier();
        // (2) token block w: Delta = M Diag(beta) X (M lower triangular)
        f32x4 da = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ib = 0; ib < C / 16; ++ib) {
            if (ib > w || !live) continue;
            da = mmf32(op.mb[ib], *reinterpret_cast<const f32x4 *>(&xT[n][16 * ib + 4 * g]), da);
        }
        if (live) *reinterpret_cast<f32x4 *>(&dT[n][r0 + 4 * g]) = da;
        lds_barrier();
        // (3) token block w: O = (q e^G) S + P Delta (P lower triangular)
#pragma unroll
        for (int ib = 0; ib < C / 16; ++ib) {
            if (ib > w || !live) continue;
            oa = mmf32(op.pb[ib], *reinterpret_cast<const f32x4 *>(&dT[n][16 * ib + 4 * g]), oa);
        }
        op.load23(blk_of(nx), w, g, n);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int r = r0 + 4 * g + u;
            if (r < L) io<TO>::st(o, ((t0 + r) * H + h) * dv + j0 + n, oa[u]);
        }
        // (4) key blocks w, w + 4: S = Diag(g) S + K^^T Delta; the new state
        //     replaces S^T in LDS (every wave's reads of it were in step 1)
#pragma unroll
        for (int i = 0; i < KPW; ++i) {
            const int kb = w + 4 * i;
            if (kb >= NKB) continue;
            f32x4 acc = op.gm[i] * st[i];
#pragma unroll
            for (int rb = 0; rb < C / 16; ++rb) {
                if (rb >= nb) break;
                acc = mmf32(op.ka[i][rb], *reinterpret_cast<const f32x4 *>(&dT[n][16 * rb + 4 * g]), acc);
            }
            st[i] = acc;
            *reinterpret_cast<f32x4 *>(&sT[n][16 * kb + 4 * g]) = acc;
        }
        op.load4(blk_of(nx), w, g, n);
        lds_barrier();
    }
    if (p.final_state)
#pragma unroll
        for (int i = 0; i < KPW; ++i) {
            const int kb = w + 4 * i;
            if (kb >= NKB) continue;
#pragma unroll
            for (int u = 0; u < 4; ++u)
                p.final_state[soff + static_cast<int64_t>(16 * kb + 4 * g + u) * dv + j0 + n] = st[i][u];
        }
}

template <int DK, typename TI, typename TO>
__global__ void __launch_bounds__(256) f32mm_scan_kernel(PrefillParams p, const float *__restrict__ blocks) {
    if (*p.status != 0) return;
    // XCD-aware order: the column tiles of one (sequence, head) share
    // blockIdx % 8, hence one XCD and its L2, where their chunk blocks are
    const int nvt = p.dv / 16;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int vt = slot % nvt, pair = xcd + 8 * (slot / nvt);
    if (pair >= p.N * p.H) return;
    f32mm_scan_run<DK, TI, TO, false>(p, blocks, pair, vt, nullptr, 0);
}

// ---------------------------------------------------- overlapped launch --
// One sequence whose scan would leave most CUs idle (at most
// kF32OverlapScanSlots column-tile workgroups per XCD; d_k = 128): the
// chunk prep and the scan run in one launch of 8 x kF32OverlapSlots
// workgroups, one per CU, with the roles of the bf16 path's overlapped
// launch (kda_prefill_mfma.hip): a workgroup takes the next ticket of the
// XCD it runs on; the first SI tickets prepare the chunks of the heads
// h = x + 8j in chunk order, flagging each block once its stores have
// completed, and the next ones run those heads' scans, each block read as
// soon as its flag is set.  Producers never wait and hold the first tickets,
// so every wait ends; a workgroup finding its XCD's roles all taken records
// KDA_ERR_DEVICE_WAIT.  The two bodies' static LDS (prep and scan) fit
// one CU together.
constexpr int kF32OverlapSlots = 32;
constexpr int kF32OverlapScanSlots = 16;

template <typename TO>
__global__ void __launch_bounds__(256) f32mm_overlap_kernel(PrefillParams p, CbParams c,
                                                            const float *__restrict__ blocks) {
    constexpr int DK = 128;
    __shared__ int s_slot;
    if (*p.status != 0) return;
    const int x = xcc_id();
    if (threadIdx.x == 0)
        s_slot = __hip_atomic_fetch_add(p.ready + x, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int slot = s_slot;
    if (slot >= kF32OverlapSlots) {
        if (threadIdx.x == 0) report_device_error(p, kErrDeviceWait);
        return;
    }
    const int H = p.H, nvt = p.dv / 16;
    const int npx = x < H ? (H - x + 7) / 8 : 0;
    const int si = kF32OverlapSlots - npx * nvt;
    if (slot < si) {
        const int total = npx * p.chunk_off[1];
        for (int k = slot; k < total; k += si) {
            const int xc = k / npx, h = x + 8 * (k % npx);
            cb_prep_run<DK, float, true>(c, xc, h);
            wait_memory();
            __syncthreads();  // every thread's stores have completed; the LDS is free
            if (threadIdx.x == 0) publish_ready(p.ready + ready_index(p, xc, h), x);
        }
    } else {
        const int s = slot - si;
        f32mm_scan_run<DK, float, TO, true>(p, blocks, x + 8 * (s / nvt), s % nvt, p.ready, x);
    }
}

namespace {

template <int DK, typename TI>
hipError_t run_scan(const PrefillParams &p, const float *blocks, int out_dtype, hipStream_t s) {
    const unsigned pairs8 = static_cast<unsigned>((p.N * p.H + 7) / 8);
    const dim3 grid(pairs8 * 8 * (p.dv / 16)), block(256);
    if (out_dtype == 0)
        hipLaunchKernelGGL((f32mm_scan_kernel<DK, TI, float>), grid, block, 0, s, p, blocks);
    else
        hipLaunchKernelGGL((f32mm_scan_kernel<DK, TI, bf16_t>), grid, block, 0, s, p, blocks);
    return hipGetLastError();
}

template <typename TI>
hipError_t run_scan_dk(const PrefillParams &p, const float *blocks, int out_dtype, hipStream_t s) {
    switch (p.dk) {
        case 16: return run_scan<16, TI>(p, blocks, out_dtype, s);
        case 32: return run_scan<32, TI>(p, blocks, out_dtype, s);
        case 64: return run_scan<64, TI>(p, blocks, out_dtype, s);
        default: return run_scan<128, TI>(p, blocks, out_dtype, s);
    }
}

}  // namespace

bool f32mm_overlap_shape(int N, int H, int dk, int dv) {
    return N == 1 && dk == 128 && (H + 7) / 8 * (dv / 16) <= kF32OverlapScanSlots;
}

bool f32mm_supported(int dk, int dv, int C, uint32_t prologue) {
    const bool dim = [](int d) { return d == 16 || d == 32 || d == 64 || d == 128; }(dk);
    return dim && dv % 16 == 0 && dv >= 16 && dv <= 128 && (C == 16 || C == 32 || C == 64);
}

hipError_t launch_prefill_f32mm(const PrefillParams &p, float *blocks, int in_dtype, int out_dtype, hipStream_t s,
                                hipEvent_t mid) {
    CbParams c{};
    c.q = p.q; c.k = p.k; c.v = p.v; c.beta = p.beta; c.log_alpha = p.log_alpha;
    c.blocks = blocks;
    c.chunk_off = p.chunk_off;
    c.chunk_info = p.chunk_info;
    c.status = p.status;
    c.N = p.N; c.H = p.H; c.dk = p.dk; c.dv = p.dv;
    c.prologue = p.prologue;
    if (p.ready && p.dk == 128 && in_dtype == 0) {  // the overlapped launch (fp32 inputs)
        if (out_dtype == 0)
            hipLaunchKernelGGL((f32mm_overlap_kernel<float>), dim3(8 * kF32OverlapSlots), dim3(256), 0, s, p, c,
                               static_cast<const float *>(blocks));
        else
            hipLaunchKernelGGL((f32mm_overlap_kernel<bf16_t>), dim3(8 * kF32OverlapSlots), dim3(256), 0, s, p, c,
                               static_cast<const float *>(blocks));
        hipError_t e = hipGetLastError();
        if (e == hipSuccess && mid) e = hipEventRecord(mid, s);
        return e;
    }
    hipError_t e = launch_chunk_prep_fwd(c, p.n_chunks_bound * p.H, in_dtype, s);
    if (e == hipSuccess && mid) e = hipEventRecord(mid, s);
    if (e != hipSuccess) return e;
    return in_dtype == 0 ? run_scan_dk<float>(p, blocks, out_dtype, s) : run_scan_dk<bf16_t>(p, blocks, out_dtype, s);
}

}  // namespace kda
