// Short causal convolution with a rolling state: the small local mixing step
// the executed sublayer applies to q, k and/or v before the recurrence
// (Module 04 — KDA II, §3 "The sublayer is bigger than the recurrence"); its
// state (the last W-1 inputs of each sequence) is serving state that a
// rollback restores (Module 11, §2, row "Serving state").
//
// Per channel c (depthwise), taps oldest input first:
//     y_t[c] = sum_{j<W} w[c][j] x_{t-W+1+j}[c] (+ bias[c]), optionally SiLU,
// where inputs before a sequence's first token come from its conv state.
//
// HBM-bound: every input is read once per tile plus W-1 halo rows (which the
// neighbouring tile also reads, mostly from L2), every output written once.
// A thread owns 8 consecutive channels (one 16-byte bf16 vector per token)
// and a tile of TT consecutive tokens; consecutive threads take consecutive
// channel groups of the same tokens, so every row of x and y is read and
// written in full 16-byte lanes.  The tile's rows are all requested before
// the filter runs.  Tiles whose window crosses a sequence start take the
// missing inputs from that sequence's conv state.  A second small kernel
// writes each sequence's final state.
#include "kda_launch.hpp"

namespace kda {

constexpr int CONV_THREADS = 256;
constexpr int CONV_CPT = 8;   // channels per thread
constexpr int CONV_TT_LONG = 16;  // tokens per thread when sequences are long

// 8 consecutive channels of one token: loaded as raw 16-byte vectors (bf16
// stays packed in registers until used), stored from fp32.  Outputs are
// stored non-temporally (this kernel does not read them again; 4 % faster
// on MI355X for a [1, 131072, 4096] bf16 input than ordinary stores).
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
template <typename T> struct vec8;
template <> struct vec8<bf16_t> {
    struct raw { uint4 u; };
    __device__ static raw ld(const bf16_t *p) { return {*reinterpret_cast<const uint4 *>(p)}; }
    __device__ static raw zero() { return {make_uint4(0, 0, 0, 0)}; }
    __device__ static float get(const raw &r, int c) {
        const uint32_t w = c < 2 ? r.u.x : c < 4 ? r.u.y : c < 6 ? r.u.z : r.u.w;
        return __uint_as_float((c & 1) ? (w & 0xffff0000u) : (w << 16));
    }
    __device__ static void st(bf16_t *p, const float (&v)[8]) {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w[i] = static_cast<uint32_t>(f32_to_bf16(v[2 * i])) | (static_cast<uint32_t>(f32_to_bf16(v[2 * i + 1])) << 16);
        __builtin_nontemporal_store(u32x4{w[0], w[1], w[2], w[3]}, reinterpret_cast<u32x4 *>(p));
    }
};
template <> struct vec8<float> {
    struct raw { float4 a, b; };
    __device__ static raw ld(const float *p) {
        return {reinterpret_cast<const float4 *>(p)[0], reinterpret_cast<const float4 *>(p)[1]};
    }
    __device__ static raw zero() { return {make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f)}; }
    __device__ static float get(const raw &r, int c) {
        const float4 &h = c < 4 ? r.a : r.b;
        const int k = c & 3;
        return k == 0 ? h.x : k == 1 ? h.y : k == 2 ? h.z : h.w;
    }
    __device__ static void st(float *p, const float (&v)[8]) {
        __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4 *>(p));
        __builtin_nontemporal_store(f32x4{v[4], v[5], v[6], v[7]}, reinterpret_cast<f32x4 *>(p) + 1);
    }
};

// Sequence bounds containing token t (flattened token axis).  Any contents
// of cu_seqlens give bounds with start <= t < end inside [0, ntok], so that a
// malformed table yields wrong values but no out-of-range address.
struct SeqPos {
    int n, start, end;
};
__device__ __forceinline__ SeqPos conv_seq(const ConvParams &p, int t) {
    SeqPos s;
    if (!p.cu_seqlens) {
        s.n = t / p.T;
        s.start = s.n * p.T;
        s.end = s.start + p.T;
        return s;
    }
    int lo = 0, hi = p.N;  // last n with cu[n] <= t
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (p.cu_seqlens[mid] <= t) lo = mid; else hi = mid;
    }
    s.n = lo;
    s.start = min(max(p.cu_seqlens[lo], 0), t);
    s.end = max(min(p.cu_seqlens[lo + 1], p.B * p.T), t + 1);
    return s;
}

// TT tokens per thread: 16 for long sequences, 1 for decode-like calls
// (one or a few tokens per sequence), where longer tiles would leave most of
// the chip idle and cross a sequence start at nearly every token.
template <typename TI, typename TO, int W, int TT>
__global__ void __launch_bounds__(CONV_THREADS) short_conv_kernel(ConvParams p) {
    constexpr int CONV_TT = TT;
    const int ngrp = p.C / CONV_CPT;
    const int ntok = p.B * p.T;
    const int64_t item = static_cast<int64_t>(blockIdx.x) * CONV_THREADS + threadIdx.x;
    const int grp = static_cast<int>(item % ngrp);
    const int64_t tile = item / ngrp;
    const int t0 = static_cast<int>(tile * CONV_TT);
    if (t0 >= ntok) return;
    const int c0 = grp * CONV_CPT;
    const TI *x = static_cast<const TI *>(p.x);
    TO *y = static_cast<TO *>(p.y);
    const int nt = min(CONV_TT, ntok - t0);
    constexpr int HW = W - 1;  // halo rows before the tile

    float w[CONV_CPT][W], bias[CONV_CPT];
#pragma unroll
    for (int c = 0; c < CONV_CPT; ++c) {
#pragma unroll
        for (int j = 0; j < W; ++j) w[c][j] = p.weight[static_cast<int64_t>(c0 + c) * W + j];
        bias[c] = p.bias ? p.bias[c0 + c] : 0.f;
    }
    // rows t0 - HW .. t0 + nt - 1 of x (rows before 0 read as 0), all
    // requested before any is used; row r of `rows` is token t0 - HW + r
    typename vec8<TI>::raw rows[HW + CONV_TT];
#pragma unroll
    for (int r = 0; r < HW + CONV_TT; ++r) {
        const int pos = t0 - HW + r;
        rows[r] = (pos >= 0 && r < HW + nt) ? vec8<TI>::ld(x + static_cast<int64_t>(pos) * p.C + c0)
                                            : vec8<TI>::zero();
    }

    SeqPos sp = conv_seq(p, t0);
    // a tile whose window stays inside one sequence needs no state
    const bool plain = t0 - HW >= sp.start && t0 + nt <= sp.end;
#pragma unroll
    for (int i = 0; i < CONV_TT; ++i) {
        if (i >= nt) continue;
        const int t = t0 + i;
        if (!plain && t >= sp.end) sp = conv_seq(p, t);  // a sequence starts inside the tile
        float out[CONV_CPT];
#pragma unroll
        for (int c = 0; c < CONV_CPT; ++c) out[c] = bias[c];
#pragma unroll
        for (int j = 0; j < W; ++j) {
            const int pos = t - HW + j;  // row i + j of `rows`
            if (plain || pos >= sp.start) {
#pragma unroll
                for (int c = 0; c < CONV_CPT; ++c) out[c] += w[c][j] * vec8<TI>::get(rows[i + j], c);
            } else if (p.initial_state) {  // before the sequence: its conv state
                const int si = HW - (sp.start - pos);  // in [0, W-2]
                const float *st = p.initial_state + (static_cast<int64_t>(sp.n) * p.C + c0) * HW + si;
#pragma unroll
                for (int c = 0; c < CONV_CPT; ++c) out[c] += w[c][j] * st[c * HW];
            }
        }
        if (p.silu)
#pragma unroll
            for (int c = 0; c < CONV_CPT; ++c) out[c] = out[c] * sigmoid_f32(out[c]);
        vec8<TO>::st(y + static_cast<int64_t>(t) * p.C + c0, out);
    }
}

// final_state[n][c][j] = input at position end_n - (W-1) + j, from the
// sequence or (when it is shorter) from its initial state.  One thread per
// (sequence, channel), j ascending: with final_state aliasing
// initial_state, entry j is written after entry j + len is read.
template <typename TI, int W>
__global__ void __launch_bounds__(CONV_THREADS) conv_state_kernel(ConvParams p) {
    const int64_t item = static_cast<int64_t>(blockIdx.x) * CONV_THREADS + threadIdx.x;
    if (item >= static_cast<int64_t>(p.N) * p.C) return;
    const int n = static_cast<int>(item / p.C), c = static_cast<int>(item % p.C);
    const int ntok = p.B * p.T;
    int start, end;
    if (p.cu_seqlens) {
        start = min(max(p.cu_seqlens[n], 0), ntok);
        end = min(max(p.cu_seqlens[n + 1], start), ntok);
    } else {
        start = n * p.T;
        end = start + p.T;
    }
    const TI *x = static_cast<const TI *>(p.x);
    const int64_t so = (static_cast<int64_t>(n) * p.C + c) * (W - 1);
    for (int j = 0; j < W - 1; ++j) {
        const int pos = end - (W - 1) + j;
        float v;
        if (pos >= start) {
            v = io<TI>::ld(x, static_cast<int64_t>(pos) * p.C + c);
        } else {
            const int si = (W - 1) - (start - pos);
            v = p.initial_state ? p.initial_state[so + si] : 0.f;
        }
        p.final_state[so + j] = v;
    }
}

// Batch rows of a few tokens each (decode): one thread per (row, 8-channel
// group) runs the row's tokens in order with the window in registers, then
// writes the rolled state.  The state of 8 consecutive channels is 8 (W-1)
// contiguous floats, read and written as float4 vectors by the thread that
// owns them, so an in-place update (final_state == initial_state) is safe.
template <typename TI, typename TO, int W>
__global__ void __launch_bounds__(CONV_THREADS) conv_rows_kernel(ConvParams p) {
    constexpr int HW = W - 1;
    constexpr int NV4 = 2 * HW;  // float4 vectors of state per thread
    const int ngrp = p.C / CONV_CPT;
    const int64_t item = static_cast<int64_t>(blockIdx.x) * CONV_THREADS + threadIdx.x;
    if (item >= static_cast<int64_t>(p.B) * ngrp) return;
    const int n = static_cast<int>(item / ngrp), c0 = static_cast<int>(item % ngrp) * CONV_CPT;
    const TI *x = static_cast<const TI *>(p.x);
    TO *y = static_cast<TO *>(p.y);

    float w[CONV_CPT][W], bias[CONV_CPT];
#pragma unroll
    for (int c = 0; c < CONV_CPT; ++c) {
#pragma unroll
        for (int j = 0; j < W; ++j) w[c][j] = p.weight[static_cast<int64_t>(c0 + c) * W + j];
        bias[c] = p.bias ? p.bias[c0 + c] : 0.f;
    }
    // window [channel][j], j = 0 oldest
    float win[CONV_CPT][HW > 0 ? HW : 1];
    const int64_t so = (static_cast<int64_t>(n) * p.C + c0) * HW;
    if (HW > 0) {
        float sv[NV4 > 0 ? 4 * NV4 : 4];
#pragma unroll
        for (int v = 0; v < NV4; ++v) {
            const float4 f = p.initial_state ? reinterpret_cast<const float4 *>(p.initial_state + so)[v]
                                             : make_float4(0.f, 0.f, 0.f, 0.f);
            sv[4 * v] = f.x; sv[4 * v + 1] = f.y; sv[4 * v + 2] = f.z; sv[4 * v + 3] = f.w;
        }
#pragma unroll
        for (int c = 0; c < CONV_CPT; ++c)
#pragma unroll
            for (int j = 0; j < HW; ++j) win[c][j] = sv[c * HW + j];
    }
    for (int t = 0; t < p.T; ++t) {
        const int64_t row = (static_cast<int64_t>(n) * p.T + t) * p.C + c0;
        const typename vec8<TI>::raw xr = vec8<TI>::ld(x + row);
        float out[CONV_CPT];
#pragma unroll
        for (int c = 0; c < CONV_CPT; ++c) {
            const float xc = vec8<TI>::get(xr, c);
            float acc = bias[c];
#pragma unroll
            for (int j = 0; j < HW; ++j) acc += w[c][j] * win[c][j];
            acc += w[c][W - 1] * xc;
            if (p.silu) acc = acc * sigmoid_f32(acc);
            out[c] = acc;
#pragma unroll
            for (int j = 0; j + 1 < HW; ++j) win[c][j] = win[c][j + 1];
            if (HW > 0) win[c][HW > 0 ? HW - 1 : 0] = xc;
        }
        vec8<TO>::st(y + row, out);
    }
    if (p.final_state && HW > 0) {
        float sv[NV4 > 0 ? 4 * NV4 : 4];
#pragma unroll
        for (int c = 0; c < CONV_CPT; ++c)
#pragma unroll
            for (int j = 0; j < HW; ++j) sv[c * HW + j] = win[c][j];
#pragma unroll
        for (int v = 0; v < NV4; ++v)
            reinterpret_cast<float4 *>(p.final_state + so)[v] = make_float4(sv[4 * v], sv[4 * v + 1], sv[4 * v + 2], sv[4 * v + 3]);
    }
}

namespace {
template <typename TI, typename TO, int W, int TT>
hipError_t launch_conv_tiles(const ConvParams &p, hipStream_t s) {
    const int64_t items = static_cast<int64_t>(p.C / CONV_CPT) * ((static_cast<int64_t>(p.B) * p.T + TT - 1) / TT);
    if (items == 0) return hipSuccess;
    const unsigned grid = static_cast<unsigned>((items + CONV_THREADS - 1) / CONV_THREADS);
    hipLaunchKernelGGL((short_conv_kernel<TI, TO, W, TT>), dim3(grid), dim3(CONV_THREADS), 0, s, p);
    return hipGetLastError();
}

template <typename TI, typename TO, int W>
hipError_t run_conv(const ConvParams &p, hipStream_t s) {
    if (!p.cu_seqlens && p.T <= 16) {  // batch rows of a few tokens: one kernel, state rolled in place
        const int64_t items = static_cast<int64_t>(p.B) * (p.C / CONV_CPT);
        hipLaunchKernelGGL((conv_rows_kernel<TI, TO, W>), dim3(static_cast<unsigned>((items + CONV_THREADS - 1) / CONV_THREADS)),
                           dim3(CONV_THREADS), 0, s, p);
        return hipGetLastError();
    }
    const int64_t ntok = static_cast<int64_t>(p.B) * p.T;
    const bool long_seqs = p.N > 0 && ntok / p.N >= 2 * CONV_TT_LONG;  // mean sequence length
    hipError_t e = long_seqs ? launch_conv_tiles<TI, TO, W, CONV_TT_LONG>(p, s) : launch_conv_tiles<TI, TO, W, 1>(p, s);
    if (e != hipSuccess) return e;
    if (p.final_state && W > 1) {
        const int64_t n = static_cast<int64_t>(p.N) * p.C;
        hipLaunchKernelGGL((conv_state_kernel<TI, W>), dim3(static_cast<unsigned>((n + CONV_THREADS - 1) / CONV_THREADS)),
                           dim3(CONV_THREADS), 0, s, p);
        return hipGetLastError();
    }
    return hipSuccess;
}

template <typename TI, typename TO>
hipError_t run_conv_w(const ConvParams &p, hipStream_t s) {
    switch (p.W) {
        case 1: return run_conv<TI, TO, 1>(p, s);
        case 2: return run_conv<TI, TO, 2>(p, s);
        case 3: return run_conv<TI, TO, 3>(p, s);
        case 4: return run_conv<TI, TO, 4>(p, s);
        case 5: return run_conv<TI, TO, 5>(p, s);
        case 6: return run_conv<TI, TO, 6>(p, s);
        case 7: return run_conv<TI, TO, 7>(p, s);
        default: return run_conv<TI, TO, 8>(p, s);
    }
}
}  // namespace

hipError_t launch_short_conv(const ConvParams &p, int in_dtype, int out_dtype, hipStream_t s) {
    if (in_dtype == 0 && out_dtype == 0) return run_conv_w<float, float>(p, s);
    if (in_dtype == 0 && out_dtype == 1) return run_conv_w<float, bf16_t>(p, s);
    if (in_dtype == 1 && out_dtype == 0) return run_conv_w<bf16_t, float>(p, s);
    return run_conv_w<bf16_t, bf16_t>(p, s);
}

}  // namespace kda
