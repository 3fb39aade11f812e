// C ABI of libkda (declared in include/kda.h): host-side validation,
// workspace sizing and dispatch.  No kernel is launched before every
// argument has been checked; nothing here allocates or synchronises.
#include "../../include/kda.h"
#include "kda_launch.hpp"

#include <atomic>
#include <cstdlib>
#include <cstring>
#include <mutex>

using namespace kda;

namespace {

bool dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool chunk_ok(int c) { return c == 16 || c == 32 || c == 64; }
bool dtype_ok(int t) { return t == KDA_F32 || t == KDA_BF16; }
bool prologue_ok(uint32_t f) { return (f & ~static_cast<uint32_t>(KDA_PROLOGUE_ALL)) == 0; }

// shape / dtype / pointer checks that do not need the workspace
kda_status check_prefill(const kda_prefill_args *a, bool need_ptrs) {
    if (!a) return KDA_ERR_NULL_ARG;
    if (a->B < 1 || a->T < 0 || a->H < 1 || a->num_seqs < 0) return KDA_ERR_BAD_SHAPE;
    if (!dim_ok(a->d_k) || !dim_ok(a->d_v) || !chunk_ok(a->chunk_size)) {
        // sizes that are positive but not implemented are "unsupported"
        if (a->d_k < 1 || a->d_v < 1 || a->chunk_size < 1) return KDA_ERR_BAD_SHAPE;
        return KDA_ERR_UNSUPPORTED;
    }
    if (!dtype_ok(a->in_dtype) || !dtype_ok(a->out_dtype)) return KDA_ERR_UNSUPPORTED;
    if (!prologue_ok(a->prologue)) return KDA_ERR_UNSUPPORTED;
    if (a->cu_seqlens) {
        if (a->B != 1 || a->num_seqs < 1) return KDA_ERR_BAD_SHAPE;
    } else if (a->num_seqs != a->B) {
        return KDA_ERR_BAD_SHAPE;
    }
    if (a->cu_seqlens_host && !a->cu_seqlens) return KDA_ERR_BAD_SHAPE;
    // element counts must fit the kernels' 32-bit token indexing
    const int64_t tokens = static_cast<int64_t>(a->B) * a->T;
    if (tokens * a->H > (static_cast<int64_t>(1) << 31)) return KDA_ERR_UNSUPPORTED;
    if (a->cu_seqlens_host) {
        const int32_t *c = a->cu_seqlens_host;
        if (c[0] != 0 || c[a->num_seqs] != a->T) return KDA_ERR_BAD_SEQLENS;
        for (int n = 0; n < a->num_seqs; ++n)
            if (c[n + 1] < c[n]) return KDA_ERR_BAD_SEQLENS;
    }
    const bool any_tokens = tokens > 0;
    if (need_ptrs && any_tokens && (!a->q || !a->k || !a->v || !a->beta || !a->log_alpha || !a->o))
        return KDA_ERR_NULL_ARG;
    return KDA_OK;
}

int64_t max_chunks(const kda_prefill_args *a) {
    const int64_t per_row = (static_cast<int64_t>(a->T) + a->chunk_size - 1) / a->chunk_size;
    return a->cu_seqlens ? per_row + a->num_seqs : per_row * a->B;
}

bool use_mfma(const kda_prefill_args *a) {
    return a->in_dtype == KDA_BF16 && mfma_supported(a->d_k, a->d_v, a->chunk_size);
}

// the fp32 matrix-core path: fp32 inputs, and bf16 inputs whose head sizes
// the bf16 matrix-core path does not take.  Its per-(chunk,
// head) blocks have 64 rows whatever the chunk size, so chunk 16 takes this
// path only while they stay within 4 GiB.
bool use_f32mm(const kda_prefill_args *a) {
    if (use_mfma(a) || !f32mm_supported(a->d_k, a->d_v, a->chunk_size, a->prologue)) return false;
    const double blocks = static_cast<double>(max_chunks(a)) * a->H * cb_block_bytes(a->d_k);
    return a->chunk_size > 16 || blocks <= 4.0 * (1u << 30);
}

// shapes whose matrix-core prefill may run as one overlapped launch
bool overlap_shape(const kda_prefill_args *a) {
    return use_mfma(a) && mfma_overlap_shape(a->num_seqs, a->H, a->d_k, a->chunk_size);
}

size_t mfma_blocks_bytes(const kda_prefill_args *a) {
    return static_cast<size_t>(max_chunks(a)) * a->H * mfma_block_bytes(a->chunk_size, a->d_k);
}

// fp32 inputs on the fp32 matrix cores: shapes whose prep and scan may run
// as one overlapped launch
bool f32_overlap_shape(const kda_prefill_args *a) {
    return use_f32mm(a) && a->in_dtype == KDA_F32 && f32mm_overlap_shape(a->num_seqs, a->H, a->d_k, a->d_v);
}

size_t f32mm_blocks_bytes(const kda_prefill_args *a) {
    return static_cast<size_t>(max_chunks(a)) * a->H * cb_block_bytes(a->d_k);
}

size_t workspace_for(const kda_prefill_args *a) {
    size_t bytes = table_bytes(a->num_seqs, max_chunks(a));
    if (use_mfma(a)) {
        bytes += mfma_blocks_bytes(a);
        if (overlap_shape(a)) bytes += mfma_ready_bytes(max_chunks(a), a->H);
    }
    else if (use_f32mm(a)) {
        bytes += f32mm_blocks_bytes(a);
        if (f32_overlap_shape(a)) bytes += mfma_ready_bytes(max_chunks(a), a->H);
    }
    return bytes;
}

}  // namespace

extern "C" {

int32_t kda_abi_version(void) { return KDA_ABI_VERSION; }

const char *kda_status_string(int32_t s) {
    switch (s) {
        case KDA_OK: return "ok";
        case KDA_ERR_NULL_ARG: return "a required pointer is NULL";
        case KDA_ERR_BAD_SHAPE: return "sizes are inconsistent or out of range";
        case KDA_ERR_UNSUPPORTED: return "valid but unsupported size or dtype";
        case KDA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case KDA_ERR_HIP: return "HIP launch failed";
        case KDA_ERR_BAD_SEQLENS: return "cu_seqlens malformed";
        case KDA_ERR_SCRATCH_LIMIT: return "needs more scratch than the allocation-free entry point holds";
        case KDA_ERR_DEVICE_WAIT: return "a hand-off between workgroups of the overlapped prefill failed";
        default: return "unknown status";
    }
}

int64_t kda_prefill_max_chunks(const kda_prefill_args *a) {
    if (check_prefill(a, false) != KDA_OK) return 0;
    return max_chunks(a);
}

size_t kda_prefill_workspace_bytes(const kda_prefill_args *a) {
    if (check_prefill(a, false) != KDA_OK) return 0;
    return workspace_for(a);
}

}  // extern "C"

namespace {

constexpr int kMaxDevices = 64;

// The device that owns hip_stream (the current device for the null stream).
kda_status stream_device(void *hip_stream, int *dev) {
    int d = -1;
    if (hip_stream) {
        hipDevice_t sd = -1;
        if (hipStreamGetDevice(static_cast<hipStream_t>(hip_stream), &sd) != hipSuccess) return KDA_ERR_HIP;
        d = static_cast<int>(sd);
    } else if (hipGetDevice(&d) != hipSuccess) {
        return KDA_ERR_HIP;
    }
    if (d < 0 || d >= kMaxDevices) return KDA_ERR_UNSUPPORTED;
    *dev = d;
    return KDA_OK;
}

// The overlapped launch places one workgroup on each of the 256 CUs of the
// 8 XCDs; it is used on devices with that many CUs unless the environment
// sets KDA_PREFILL_OVERLAP=0.  CU counts are looked up once per device.
std::atomic<int> g_cu_count[kMaxDevices];

bool overlap_enabled(void *hip_stream) {
    const char *env = std::getenv("KDA_PREFILL_OVERLAP");
    if (env && std::strcmp(env, "0") == 0) return false;
    int dev = -1;
    if (stream_device(hip_stream, &dev) != KDA_OK) return false;
    int n = g_cu_count[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return false;
        g_cu_count[dev].store(n, std::memory_order_relaxed);
    }
    return n == 256;
}

// Bound of the overlapped launch's cross-workgroup waits, in ticks of the
// device's 100 MHz real-time counter: 1 s, or KDA_PREFILL_WAIT_TICKS from the
// environment (a small bound makes the waits expire: the failure path's test).
uint64_t overlap_wait_ticks() {
    const char *env = std::getenv("KDA_PREFILL_WAIT_TICKS");
    if (env && *env) {
        char *end = nullptr;
        const unsigned long long v = std::strtoull(env, &end, 10);
        if (end && *end == 0) return v;
    }
    return 100000000ull;
}

// The prefill after host validation, with its scratch at ws (ws_bytes long).
kda_status prefill_on(const kda_prefill_args *a, char *ws, size_t ws_bytes, void *hip_stream) {
    if (!ws) return KDA_ERR_NULL_ARG;
    if (reinterpret_cast<uintptr_t>(ws) % kAlign) return KDA_ERR_BAD_SHAPE;
    if (ws_bytes < workspace_for(a)) return KDA_ERR_WORKSPACE_TOO_SMALL;
    // the bf16 matrix-core path reads q, k, v and the gate as 128-bit vectors
    if (use_mfma(a))
        for (const void *ptr : {a->q, a->k, a->v, a->log_alpha})
            if (reinterpret_cast<uintptr_t>(ptr) % 16) return KDA_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);

    PrefillParams p{};
    p.q = a->q; p.k = a->k; p.v = a->v; p.beta = a->beta; p.log_alpha = a->log_alpha;
    p.o = a->o;
    p.initial_state = a->initial_state;
    p.final_state = a->final_state;
    p.chunk_states = a->chunk_states;
    p.cu_seqlens = a->cu_seqlens;
    p.status = reinterpret_cast<int32_t *>(ws);
    p.chunk_off = reinterpret_cast<int32_t *>(ws + kAlign);
    p.chunk_info = reinterpret_cast<const int4 *>(ws + kAlign + chunk_off_bytes(a->num_seqs));
    p.user_status = a->device_status;
    p.B = a->B; p.T = a->T; p.H = a->H; p.dk = a->d_k; p.dv = a->d_v;
    p.N = a->num_seqs; p.C = a->chunk_size;
    p.n_chunks_bound = static_cast<int32_t>(max_chunks(a));
    p.prologue = a->prologue;
    p.ready = nullptr;
    p.wait_ticks = overlap_wait_ticks();
    if (overlap_shape(a) && overlap_enabled(hip_stream))
        p.ready = reinterpret_cast<int32_t *>(ws + table_bytes(p.N, p.n_chunks_bound) + mfma_blocks_bytes(a));
    else if (f32_overlap_shape(a) && overlap_enabled(hip_stream))
        p.ready = reinterpret_cast<int32_t *>(ws + table_bytes(p.N, p.n_chunks_bound) + f32mm_blocks_bytes(a));

    if (p.N == 0) return KDA_OK;
    hipEvent_t *ev = static_cast<hipEvent_t *>(a->timing_events);
    hipError_t e = ev ? hipEventRecord(ev[0], s) : hipSuccess;
    if (e == hipSuccess) e = launch_chunk_table(p, s);
    if (e == hipSuccess) {
        if (use_mfma(a))
            e = launch_prefill_mfma(p, ws + table_bytes(p.N, p.n_chunks_bound), a->out_dtype, s,
                                    ev ? ev[1] : nullptr);
        else if (use_f32mm(a))
            e = launch_prefill_f32mm(p, reinterpret_cast<float *>(ws + table_bytes(p.N, p.n_chunks_bound)),
                                     a->in_dtype, a->out_dtype, s, ev ? ev[1] : nullptr);
        else {
            e = launch_prefill_f32(p, a->in_dtype, a->out_dtype, s);
            if (e == hipSuccess && ev) e = hipEventRecord(ev[1], s);
        }
    }
    if (e == hipSuccess && ev) e = hipEventRecord(ev[2], s);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

// Scratch of the allocation-free prefill: one copy of this array per GPU,
// allocated when the library's code object is loaded on that GPU and held
// until the process ends.  In host code its name is only a stand-in for the
// device symbol, never an address: host code uses the per-device address
// that scratch_address() looks up.
static __device__ __align__(256) char scratch[KDA_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the device that owns hip_stream (the
// current device for the null stream), looked up once per device with that
// device current.
kda_status scratch_address(void *hip_stream, char **out) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return KDA_ERR_HIP;
    int dev = cur;
    const kda_status st = stream_device(hip_stream, &dev);
    if (st != KDA_OK) return st;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        if (dev != cur && hipSetDevice(dev) != hipSuccess) return KDA_ERR_HIP;
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (dev != cur && hipSetDevice(cur) != hipSuccess) return KDA_ERR_HIP;
        if (e != hipSuccess || ptr == nullptr) return KDA_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = static_cast<char *>(g_scratch_ptr[dev]);
    return KDA_OK;
}

}  // namespace

extern "C" {

kda_status kda_prefill_chunked(const kda_prefill_args *a, void *hip_stream) {
    kda_status st = check_prefill(a, true);
    if (st != KDA_OK) return st;
    return prefill_on(a, static_cast<char *>(a->workspace), a->workspace_bytes, hip_stream);
}

kda_status kda_prefill_chunked_noalloc(const kda_prefill_args *a, void *hip_stream) {
    kda_status st = check_prefill(a, true);
    if (st != KDA_OK) return st;
    if (workspace_for(a) > KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_SCRATCH_LIMIT;
    char *ws = nullptr;
    st = scratch_address(hip_stream, &ws);
    if (st != KDA_OK) return st;
    return prefill_on(a, ws, KDA_NOALLOC_SCRATCH_BYTES, hip_stream);
}

kda_status kda_decode_step(int32_t B, int32_t H, int32_t d_k, int32_t d_v, int32_t in_dtype,
                           int32_t out_dtype, const void *q, const void *k, const void *v,
                           const void *beta, const void *log_alpha, float *state, void *o,
                           void *hip_stream) {
    kda_decode_args a{};
    a.B = B; a.H = H; a.d_k = d_k; a.d_v = d_v; a.n_tokens = 1;
    a.in_dtype = in_dtype; a.out_dtype = out_dtype; a.prologue = 0;
    a.q = q; a.k = k; a.v = v; a.beta = beta; a.log_alpha = log_alpha;
    a.initial_state = state; a.final_state = state; a.token_states = nullptr; a.o = o;
    return kda_decode(&a, hip_stream);
}

kda_status kda_decode(const kda_decode_args *a, void *hip_stream) {
    if (!a) return KDA_ERR_NULL_ARG;
    if (a->B < 0 || a->H < 1 || a->n_tokens < 1) return KDA_ERR_BAD_SHAPE;
    if (!dim_ok(a->d_k) || !dim_ok(a->d_v)) return (a->d_k < 1 || a->d_v < 1) ? KDA_ERR_BAD_SHAPE : KDA_ERR_UNSUPPORTED;
    if (!dtype_ok(a->in_dtype) || !dtype_ok(a->out_dtype)) return KDA_ERR_UNSUPPORTED;
    if (!prologue_ok(a->prologue)) return KDA_ERR_UNSUPPORTED;
    if (static_cast<int64_t>(a->B) * a->n_tokens * a->H > (static_cast<int64_t>(1) << 31) - 1)
        return KDA_ERR_UNSUPPORTED;
    if (a->B == 0) return KDA_OK;
    if (!a->q || !a->k || !a->v || !a->beta || !a->log_alpha || !a->initial_state || !a->o)
        return KDA_ERR_NULL_ARG;
    // the kernel moves state rows as 128-bit vectors
    for (const float *ptr : {a->initial_state, static_cast<const float *>(a->final_state),
                             static_cast<const float *>(a->token_states)})
        if (reinterpret_cast<uintptr_t>(ptr) % 16) return KDA_ERR_UNSUPPORTED;
    hipError_t e = launch_decode(a->B, a->H, a->n_tokens, a->d_k, a->d_v, a->in_dtype, a->out_dtype, a->prologue,
                                 a->q, a->k, a->v, a->beta, a->log_alpha, a->initial_state, a->final_state,
                                 a->token_states, a->o, static_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_short_conv(const kda_conv_args *a, void *hip_stream) {
    if (!a) return KDA_ERR_NULL_ARG;
    if (a->B < 1 || a->T < 0 || a->C < 1 || a->W < 1 || a->num_seqs < 0) return KDA_ERR_BAD_SHAPE;
    if (a->W > 8 || a->C % 8 != 0) return KDA_ERR_UNSUPPORTED;
    if (!dtype_ok(a->in_dtype) || !dtype_ok(a->out_dtype)) return KDA_ERR_UNSUPPORTED;
    if (a->activation != KDA_CONV_NONE && a->activation != KDA_CONV_SILU) return KDA_ERR_UNSUPPORTED;
    if (a->cu_seqlens) {
        if (a->B != 1 || a->num_seqs < 1) return KDA_ERR_BAD_SHAPE;
    } else if (a->num_seqs != a->B) {
        return KDA_ERR_BAD_SHAPE;
    }
    if (static_cast<int64_t>(a->B) * a->T * a->C > (static_cast<int64_t>(1) << 31) - 1) return KDA_ERR_UNSUPPORTED;
    const bool any_tokens = static_cast<int64_t>(a->B) * a->T > 0;
    if (!a->weight || (any_tokens && (!a->x || !a->y))) return KDA_ERR_NULL_ARG;
    // rows and states are moved as 16-byte vectors
    for (const void *ptr : {a->x, static_cast<const void *>(a->y), static_cast<const void *>(a->initial_state),
                            static_cast<const void *>(a->final_state)})
        if (reinterpret_cast<uintptr_t>(ptr) % 16) return KDA_ERR_UNSUPPORTED;
    ConvParams p{};
    p.x = a->x; p.weight = a->weight; p.bias = a->bias; p.cu_seqlens = a->cu_seqlens;
    p.initial_state = a->initial_state; p.final_state = a->final_state; p.y = a->y;
    p.B = a->B; p.T = a->T; p.C = a->C; p.W = a->W; p.N = a->num_seqs;
    p.silu = a->activation == KDA_CONV_SILU;
    hipError_t e = launch_short_conv(p, a->in_dtype, a->out_dtype, static_cast<hipStream_t>(hip_stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

namespace {
// backward: the checks that do not need the workspace
kda_status check_backward(const kda_backward_args *a, bool need_ptrs) {
    if (!a) return KDA_ERR_NULL_ARG;
    if (a->B < 1 || a->T < 0 || a->H < 1 || a->num_seqs < 0) return KDA_ERR_BAD_SHAPE;
    if (!dim_ok(a->d_k) || !dim_ok(a->d_v)) return (a->d_k < 1 || a->d_v < 1) ? KDA_ERR_BAD_SHAPE : KDA_ERR_UNSUPPORTED;
    if (!dtype_ok(a->in_dtype)) return KDA_ERR_UNSUPPORTED;
    if (a->in_dtype == KDA_BF16 ? !chunk_ok(a->chunk_size) : a->chunk_size != 16) {
        if (a->chunk_size < 1) return KDA_ERR_BAD_SHAPE;
        return KDA_ERR_UNSUPPORTED;
    }
    if (a->cu_seqlens) {
        if (a->B != 1 || a->num_seqs < 1) return KDA_ERR_BAD_SHAPE;
    } else if (a->num_seqs != a->B) {
        return KDA_ERR_BAD_SHAPE;
    }
    const int64_t tokens = static_cast<int64_t>(a->B) * a->T;
    if (tokens * a->H * (a->d_k > a->d_v ? a->d_k : a->d_v) > (static_cast<int64_t>(1) << 31) - 1)
        return KDA_ERR_UNSUPPORTED;
    if (need_ptrs && tokens > 0 &&
        (!a->q || !a->k || !a->v || !a->beta || !a->log_alpha || !a->checkpoints || !a->d_o || !a->dq ||
         !a->dk || !a->dv || !a->dbeta || !a->dlog_alpha))
        return KDA_ERR_NULL_ARG;
    return KDA_OK;
}
int64_t backward_chunks(const kda_backward_args *a) {
    const int64_t per_row = (static_cast<int64_t>(a->T) + a->chunk_size - 1) / a->chunk_size;
    return a->cu_seqlens ? per_row + a->num_seqs : per_row * a->B;
}
// bf16: chunk table, the per-(chunk, head) blocks, the dS entering every chunk
size_t backward_blocks_bytes(const kda_backward_args *a) {
    if (a->in_dtype != KDA_BF16) return 0;
    const size_t items = static_cast<size_t>(backward_chunks(a)) * a->H;
    return align_up(items * cb_block_bytes(a->d_k)) + align_up(items * a->d_k * a->d_v * sizeof(float));
}
}  // namespace

size_t kda_backward_workspace_bytes(const kda_backward_args *a) {
    if (check_backward(a, false) != KDA_OK) return 0;
    return table_bytes(a->num_seqs, backward_chunks(a)) + backward_blocks_bytes(a);
}

kda_status kda_backward(const kda_backward_args *a, void *hip_stream) {
    kda_status st = check_backward(a, true);
    if (st != KDA_OK) return st;
    if (!a->workspace) return KDA_ERR_NULL_ARG;
    if (reinterpret_cast<uintptr_t>(a->workspace) % kAlign) return KDA_ERR_BAD_SHAPE;
    if (a->workspace_bytes < kda_backward_workspace_bytes(a)) return KDA_ERR_WORKSPACE_TOO_SMALL;
    if (a->in_dtype == KDA_BF16 &&
        (reinterpret_cast<uintptr_t>(a->d_o) % 16 || reinterpret_cast<uintptr_t>(a->checkpoints) % 16))
        return KDA_ERR_UNSUPPORTED;  // the chunked kernels read them as float4
    if (a->num_seqs == 0) return KDA_OK;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    char *ws = static_cast<char *>(a->workspace);
    // the chunk table of chunk_size-token chunks (validates cu_seqlens on the device)
    PrefillParams tp{};
    tp.cu_seqlens = a->cu_seqlens;
    tp.status = reinterpret_cast<int32_t *>(ws);
    tp.chunk_off = reinterpret_cast<int32_t *>(ws + kAlign);
    tp.chunk_info = reinterpret_cast<const int4 *>(ws + kAlign + chunk_off_bytes(a->num_seqs));
    tp.B = a->B; tp.T = a->T; tp.H = a->H; tp.dk = a->d_k; tp.dv = a->d_v;
    tp.N = a->num_seqs; tp.C = a->chunk_size;
    tp.n_chunks_bound = static_cast<int32_t>(backward_chunks(a));
    hipError_t e = launch_chunk_table(tp, s);
    if (e != hipSuccess) return KDA_ERR_HIP;
    if (a->in_dtype == KDA_BF16) {
        char *wb = ws + table_bytes(a->num_seqs, backward_chunks(a));
        const size_t items = static_cast<size_t>(backward_chunks(a)) * a->H;
        CbParams c{};
        c.q = a->q; c.k = a->k; c.v = a->v; c.beta = a->beta; c.log_alpha = a->log_alpha;
        c.d_o = a->d_o; c.d_final = a->d_final_state; c.checkpoints = a->checkpoints;
        c.blocks = reinterpret_cast<float *>(wb);
        c.dS_right = reinterpret_cast<float *>(wb + align_up(items * cb_block_bytes(a->d_k)));
        c.gq = a->dq; c.gk = a->dk; c.gv = a->dv; c.gbeta = a->dbeta; c.gg = a->dlog_alpha;
        c.d_initial = a->d_initial_state;
        c.chunk_off = tp.chunk_off; c.chunk_info = tp.chunk_info; c.status = tp.status;
        c.N = a->num_seqs; c.H = a->H; c.dk = a->d_k; c.dv = a->d_v;
        // the chunk count is only known on the device: the per-chunk kernels
        // are launched over the bound and items beyond the table's total
        // return at once (their chunk_info is never read)
        e = launch_backward_chunked(c, static_cast<int>(items), s);
        return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
    }
    BackwardParams p{};
    p.q = a->q; p.k = a->k; p.v = a->v; p.beta = a->beta; p.log_alpha = a->log_alpha;
    p.d_o = a->d_o; p.d_final = a->d_final_state; p.checkpoints = a->checkpoints;
    p.gq = a->dq; p.gk = a->dk; p.gv = a->dv; p.gbeta = a->dbeta; p.gg = a->dlog_alpha;
    p.d_initial = a->d_initial_state;
    p.cu_seqlens = a->cu_seqlens; p.chunk_off = tp.chunk_off; p.status = tp.status;
    p.B = a->B; p.T = a->T; p.H = a->H; p.dk = a->d_k; p.dv = a->d_v; p.N = a->num_seqs;
    e = launch_backward(p, a->in_dtype, s);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // extern "C"
