// Hand-off of per-(chunk, head) blocks between the workgroups of one launch
// (the overlapped prefill launches): flags, bounded waits, error reporting.
#pragma once
#include "kda_prefill_common.hpp"

namespace kda {

// ------------------------------------------- overlapped launch hand-off --
// In the overlapped launch one workgroup writes a (chunk, head) block and
// another one of the same XCD reads it while the kernel still runs.  Within
// an XCD the L2 is the point of coherence: a store has reached it once the
// storing thread's vector memory counter is zero, and a load that misses the
// L1 reads it there.  The reader never touches a block before its flag is
// set, so the block's lines cannot be in the reader's L1 from earlier.  A
// flag holds 1 + the XCD of its writer; a reader on another XCD (which the
// launches' role assignment never makes) would take a device-wide acquire.
//
// The ready area of the workspace: kReadyTickets role counters (one per
// XCD, the rest padding), then one flag per (head, chunk).
constexpr int kReadyTickets = 64;

// Status code of an expired hand-off wait (KDA_ERR_DEVICE_WAIT).
constexpr int32_t kErrDeviceWait = 8;

__device__ __forceinline__ int xcc_id() {
    return __builtin_amdgcn_s_getreg((20) | (0 << 6) | (3 << 11));  // HW_REG_XCC_ID, bits [3:0]
}

// Waits until every vector memory access of this thread has completed.
__device__ __forceinline__ void wait_memory() { __builtin_amdgcn_s_waitcnt(0x0f70); }  // vmcnt(0)

// After the block's stores have completed (wait_memory by every thread and a
// barrier): flag = 1 + xcc.
__device__ __forceinline__ void publish_ready(int32_t *flag, int xcc) {
    __hip_atomic_store(flag, 1 + xcc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void report_device_error(const PrefillParams &p, int32_t code) {
    __hip_atomic_store(p.status, code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (p.user_status) __hip_atomic_store(p.user_status, code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A reader's view of one head's flags (flags[c] for chunk c < nch, one
// sequence): chunks below `known` are published.  ensure(j) returns once
// chunk j is; each poll reads the flags of the next 64 chunks at once (one
// per lane), so a reader behind its writers polls once per 64 chunks.
// Bounded: once the call's status word holds an error, or after
// p.wait_ticks of the 100 MHz real-time counter without progress, ensure
// returns anyway (recording kErrDeviceWait), so every wave still runs to its
// end; the call's results are then undefined and its status says so.
// Uniform per wave.
struct ReadyView {
    const int32_t *flags;
    int nch, known, xcc;
    __device__ __forceinline__ void ensure(int j, const PrefillParams &p) {
        if (j < known) return;
        const int lane = __lane_id();
        uint64_t t0 = 0;
        for (int spin = 0;; ++spin) {
            const int c = known + lane;
            const int f = c < nch ? __hip_atomic_load(flags + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 1 + xcc;
            const uint64_t unset = __builtin_amdgcn_ballot_w64(f == 0);
            const int m = unset ? __builtin_ctzll(unset) : 64;  // leading published chunks
            // a block written on another XCD is only visible after a device-wide acquire
            if (__builtin_amdgcn_ballot_w64(lane < m && f - 1 != xcc)) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            known += m;
            if (j < known) return;
            if (spin == 0) t0 = __builtin_amdgcn_s_memrealtime();
            if (m > 0) t0 = __builtin_amdgcn_s_memrealtime();
            if (__builtin_amdgcn_readfirstlane(
                    __hip_atomic_load(p.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) != 0) {
                known = nch;
                return;
            }
            if (__builtin_amdgcn_s_memrealtime() - t0 > p.wait_ticks) {
                report_device_error(p, kErrDeviceWait);
                known = nch;
                return;
            }
            __builtin_amdgcn_s_sleep(2);
        }
    }
};

// Flag of (chunk x, head h) in the overlapped launch: one sequence, flags
// of a head contiguous in chunk order.
__device__ __forceinline__ int ready_index(const PrefillParams &p, int x, int h) {
    return kReadyTickets + h * p.n_chunks_bound + x;
}

}  // namespace kda
