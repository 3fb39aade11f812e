// Chunk table and cu_seqlens validation (runs before every prefill).
#include "kda_launch.hpp"

namespace kda {

// Chunk table: chunk_off[n] = sum_{m < n} ceil(len_m / C), and per chunk x
// chunk_info[x] = (first token low 32 bits, high 32 bits, length, sequence)
// so that a kernel walking chunks reads its coordinates with one load.  With packed
// input also validates cu_seqlens (0 = cu[0] <= ... <= cu[N] = T) and writes
// the verdict to *status (and *user_status); every later kernel reads
// *status first and does nothing if it is non-zero, so malformed offsets are
// never used to address memory.  One workgroup of 1024 threads.
__global__ void __launch_bounds__(1024) chunk_table_kernel(PrefillParams p) {
    __shared__ int32_t s_sum[1024];
    __shared__ int32_t s_bad;
    const int tid = threadIdx.x;
    const int N = p.N;
    // the overlapped launch's role counters and hand-off flags start cleared
    if (p.ready)
        for (size_t i = tid; i < mfma_ready_words(p.n_chunks_bound, p.H); i += 1024) p.ready[i] = 0;
    if (tid == 0) s_bad = 0;
    __syncthreads();
    // each thread owns a contiguous block of sequences
    const int per = (N + 1023) / 1024;
    const int n0 = tid * per, n1 = min(N, n0 + per);
    int32_t local = 0;
    for (int n = n0; n < n1; ++n) {
        int32_t len;
        if (p.cu_seqlens) {
            const int32_t a = p.cu_seqlens[n], b = p.cu_seqlens[n + 1];
            if (b < a || a < 0 || b > p.T) s_bad = 1;  // benign race: any writer sets 1
            len = b - a;
        } else {
            len = p.T;
        }
        local += len > 0 ? (len + p.C - 1) / p.C : 0;
    }
    if (p.cu_seqlens && tid == 0 && (p.cu_seqlens[0] != 0 || p.cu_seqlens[N] != p.T)) s_bad = 1;
    s_sum[tid] = local;
    __syncthreads();
    // inclusive scan (Hillis-Steele) over the 1024 partial sums
    for (int off = 1; off < 1024; off <<= 1) {
        const int32_t x = tid >= off ? s_sum[tid - off] : 0;
        __syncthreads();
        s_sum[tid] += x;
        __syncthreads();
    }
    int32_t run = tid > 0 ? s_sum[tid - 1] : 0;
    int32_t *off = const_cast<int32_t *>(p.chunk_off);
    for (int n = n0; n < n1; ++n) {
        off[n] = run;
        int32_t len = p.cu_seqlens ? p.cu_seqlens[n + 1] - p.cu_seqlens[n] : p.T;
        run += len > 0 ? (len + p.C - 1) / p.C : 0;
    }
    if (tid == 1023) off[N] = s_sum[1023];
    const int32_t total = s_sum[1023];
    const bool bad = s_bad || total > p.n_chunks_bound;
    __syncthreads();  // chunk_off visible to the whole workgroup
    if (!bad) {
        int4 *info = const_cast<int4 *>(p.chunk_info);
        for (int x = tid; x < total; x += 1024) {
            const int n = chunk_to_seq(off, N, x);
            const SeqRange sr = seq_range(p, n);
            const int c = x - off[n];
            const int64_t t0 = sr.start + static_cast<int64_t>(c) * p.C;
            info[x] = make_int4(static_cast<int32_t>(t0 & 0xffffffff), static_cast<int32_t>(t0 >> 32),
                                min(p.C, sr.len - c * p.C), n);
        }
    }
    if (tid == 1023) {
        *p.status = bad ? 6 /* KDA_ERR_BAD_SEQLENS */ : 0;
        if (p.user_status) *p.user_status = bad ? 6 : 0;
    }
}

hipError_t launch_chunk_table(const PrefillParams &p, hipStream_t s) {
    hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(1024), 0, s, p);
    return hipGetLastError();
}

}  // namespace kda
