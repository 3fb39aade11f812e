// Shared device helpers for the KDA kernels (gfx950 / CDNA4).
//
// Matrix-core conventions used throughout (v_mfma_f32_16x16x32_bf16, wave64):
//   A operand (16 x 32, M x K): lane l holds 8 bf16 of row (l % 16);
//   B operand (32 x 16, K x N): lane l holds 8 bf16 of column (l % 16);
//   C/D       (16 x 16 fp32):   lane l holds rows 4*(l/16) + j, j = 0..3,
//                               of column (l % 16).
// Within one instruction the k index of an A register slot and of the
// matching B register slot is the same function of (l / 16, slot); which
// function it is does not matter for a product as long as both operands are
// loaded with the same one.  Every operand here is loaded with KPERM below,
// chosen so that two C/D tiles stacked along M (rows 0-15 and 16-31 of a
// 32-row block) are, register for register, a B operand with K = 32:
//   slot j < 4  ->  k = 4*g + j          (first tile,  its register j)
//   slot j >= 4 ->  k = 16 + 4*g + j - 4 (second tile, its register j - 4)
// with g = l / 16.  A state or Delta held as accumulators therefore feeds the
// next product without passing through LDS.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef uint16_t bf16_t;  // storage type: raw bf16 bits

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- bf16 ----
__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// round to nearest, ties to even (the hardware conversion, v_cvt_pk_bf16_f32)
__device__ __forceinline__ bf16_t f32_to_bf16(float x) {
    return __builtin_bit_cast(bf16_t, static_cast<__bf16>(x));
}

__device__ __forceinline__ __bf16 bits_as_bf16(bf16_t b) {
    return __builtin_bit_cast(__bf16, b);
}

// x = hi + lo with hi = bf16(x), lo = bf16(x - hi): ~16 significant bits.
__device__ __forceinline__ void split_bf16(float x, bf16_t &hi, bf16_t &lo) {
    hi = f32_to_bf16(x);
    lo = f32_to_bf16(x - bf16_to_f32(hi));
}

template <typename T> struct io;
template <> struct io<float> {
    __device__ __forceinline__ static float ld(const float *p, int64_t i) { return p[i]; }
    __device__ __forceinline__ static void st(float *p, int64_t i, float x) { p[i] = x; }
};
template <> struct io<bf16_t> {
    __device__ __forceinline__ static float ld(const bf16_t *p, int64_t i) { return bf16_to_f32(p[i]); }
    __device__ __forceinline__ static void st(bf16_t *p, int64_t i, float x) { p[i] = f32_to_bf16(x); }
};

// --------------------------------------------------------------- MFMA ----
__device__ __forceinline__ f32x4 mfma16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// k offset (within a 32-wide K step) of register slot j for lane group g
__device__ __forceinline__ constexpr int kperm(int g, int j) {
    return j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4);
}

union frag8 {
    bf16x8 v;
    bf16_t s[8];
    uint4 u;
};

// two fp32 accumulator tiles (stacked along M) -> B operand, hi and lo parts
__device__ __forceinline__ void acc2_to_split(const f32x4 &t0, const f32x4 &t1, frag8 &hi, frag8 &lo) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        split_bf16(t0[j], hi.s[j], lo.s[j]);
        split_bf16(t1[j], hi.s[4 + j], lo.s[4 + j]);
    }
}
__device__ __forceinline__ void acc2_to_bf16(const f32x4 &t0, const f32x4 &t1, frag8 &hi) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        hi.s[j] = f32_to_bf16(t0[j]);
        hi.s[4 + j] = f32_to_bf16(t1[j]);
    }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ------------------------------------------------------------ prologue ----
// Stages that precede the recurrence in the executed sublayer (Module 04 —
// KDA II, §3 "The sublayer is bigger than the recurrence"), fused into the
// kernels when the matching bit is set; the argument then holds the
// pre-activation x.
constexpr uint32_t kProGate = 1u;    // log alpha = -softplus(x)
constexpr uint32_t kProBeta = 2u;    // beta = sigmoid(x)
constexpr uint32_t kProQKNorm = 4u;  // q, k / sqrt(sum x^2 + kQKNormEps)
constexpr float kQKNormEps = 1e-6f;

// log(1 + e^x) = max(x, 0) + ln 2 * log2(1 + 2^(-|x| log2 e)) on the hardware
// exp2 / log2: no overflow for any x; the absolute error is a few 1e-8 (the
// rounding of 1 + y), which is what a sum of log-decays accumulates.
__device__ __forceinline__ float softplus_f32(float x) {
    const float y = fast_exp2(-fabsf(x) * kLog2e);
    return fmaxf(x, 0.f) + __builtin_amdgcn_logf(1.f + y) * 0.6931471805599453f;
}

// 1 / (1 + e^-x) without overflow on either side
__device__ __forceinline__ float sigmoid_f32(float x) {
    const float e = fast_exp2(-fabsf(x) * kLog2e);
    const float r = 1.f / (1.f + e);
    return x >= 0.f ? r : e * r;
}

// Workgroup barrier that orders LDS only.  __syncthreads() is a
// workgroup-scope fence over all memory, so it waits for every outstanding
// global load and store of the wave (s_waitcnt vmcnt(0)); kernels whose
// waves exchange data only through LDS use this instead so that prefetched
// loads and workspace stores stay in flight across the barrier.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace kda
