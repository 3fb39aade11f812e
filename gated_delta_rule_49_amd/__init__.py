"""KDA gated delta-rule recurrence on AMD Instinct MI355X (gfx950).

Thin Python binding over ``libkda.so`` (C ABI in ``include/kda.h``): it only
marshals torch tensors into pointers and sizes, allocates outputs and the
workspace with torch, and passes torch's current HIP stream.  Every step of
the computation runs in the library's HIP kernels; there is no CPU fallback —
if the library is missing or the tensors are not on the GPU these functions
raise.

    o, S = prefill(q, k, v, beta, log_alpha, initial_state=None,
                   cu_seqlens=None, chunk_size=64)
    o = decode_step(q, k, v, beta, log_alpha, state)     # state updated in place
    o, S, per_token = decode(q, k, v, beta, log_alpha, state)   # m tokens per sequence
    y, conv_state = short_conv(x, weight, conv_state)            # rolling causal conv
    dq, dk, dv, dbeta, dlog_alpha, dS0 = backward(q, k, v, beta, log_alpha, d_o)

``prologue`` (prefill and decode) fuses the stages that precede the
recurrence: PROLOGUE_GATE_SOFTPLUS (log_alpha holds x, log alpha =
-softplus(x)), PROLOGUE_BETA_SIGMOID (beta holds x, beta = sigmoid(x)),
PROLOGUE_QK_L2NORM (q, k divided by sqrt(sum x^2 + 1e-6)), or PROLOGUE_ALL.

The recurrence (per sequence and head, S is d_k x d_v fp32):
    S_t = (I - beta_t k_t k_t^T) Diag(exp(log_alpha_t)) S_{t-1} + beta_t k_t v_t^T
    o_t = S_t^T q_t
("GLM-5.3-Flash Architecture Mastery", course index, Course Outcomes;
Module 04 — KDA II, §2: prefill and decode are separate kernel families.)
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["prefill", "prefill_noalloc", "NOALLOC_SCRATCH_BYTES", "decode_step", "decode", "short_conv", "backward", "workspace_bytes", "max_chunks",
           "lib", "KDAError", "PrefillArgs", "DecodeArgs", "ConvArgs", "BackwardArgs", "KDA_F32", "KDA_BF16", "PROLOGUE_GATE_SOFTPLUS",
           "PROLOGUE_BETA_SIGMOID", "PROLOGUE_QK_L2NORM", "PROLOGUE_ALL"]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")

KDA_F32, KDA_BF16 = 0, 1
PROLOGUE_GATE_SOFTPLUS, PROLOGUE_BETA_SIGMOID, PROLOGUE_QK_L2NORM = 1, 2, 4
PROLOGUE_ALL = 7
_STATUS_BAD_SEQLENS = 6
# fixed per-GPU scratch of kda_prefill_chunked_noalloc (KDA_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 256 << 20


class KDAError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: status {status} ({_status_string(status)})")


class PrefillArgs(ctypes.Structure):
    """Mirror of ``kda_prefill_args`` (include/kda.h)."""
    _fields_ = [
        ("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
        ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32), ("num_seqs", ctypes.c_int32),
        ("chunk_size", ctypes.c_int32), ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("beta", ctypes.c_void_p), ("log_alpha", ctypes.c_void_p),
        ("cu_seqlens", ctypes.c_void_p), ("cu_seqlens_host", ctypes.c_void_p),
        ("initial_state", ctypes.c_void_p), ("final_state", ctypes.c_void_p),
        ("chunk_states", ctypes.c_void_p), ("o", ctypes.c_void_p),
        ("device_status", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("timing_events", ctypes.c_void_p),
        ("prologue", ctypes.c_uint32),
    ]


class DecodeArgs(ctypes.Structure):
    """Mirror of ``kda_decode_args`` (include/kda.h)."""
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
        ("n_tokens", ctypes.c_int32), ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
        ("prologue", ctypes.c_uint32),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("beta", ctypes.c_void_p), ("log_alpha", ctypes.c_void_p),
        ("initial_state", ctypes.c_void_p), ("final_state", ctypes.c_void_p),
        ("token_states", ctypes.c_void_p), ("o", ctypes.c_void_p),
    ]


class ConvArgs(ctypes.Structure):
    """Mirror of ``kda_conv_args`` (include/kda.h)."""
    _fields_ = [
        ("B", ctypes.c_int32), ("T", ctypes.c_int32), ("C", ctypes.c_int32), ("W", ctypes.c_int32),
        ("num_seqs", ctypes.c_int32), ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
        ("activation", ctypes.c_int32),
        ("x", ctypes.c_void_p), ("weight", ctypes.c_void_p), ("bias", ctypes.c_void_p),
        ("cu_seqlens", ctypes.c_void_p), ("initial_state", ctypes.c_void_p),
        ("final_state", ctypes.c_void_p), ("y", ctypes.c_void_p),
    ]


class BackwardArgs(ctypes.Structure):
    """Mirror of ``kda_backward_args`` (include/kda.h)."""
    _fields_ = [
        ("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
        ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32), ("num_seqs", ctypes.c_int32),
        ("in_dtype", ctypes.c_int32), ("chunk_size", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("beta", ctypes.c_void_p), ("log_alpha", ctypes.c_void_p), ("cu_seqlens", ctypes.c_void_p),
        ("checkpoints", ctypes.c_void_p), ("d_o", ctypes.c_void_p), ("d_final_state", ctypes.c_void_p),
        ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p),
        ("dbeta", ctypes.c_void_p), ("dlog_alpha", ctypes.c_void_p), ("d_initial_state", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
    ]


_lib = None


def lib():
    """The loaded ``libkda.so`` with argument types declared."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                               "(or gated_delta_rule_49_amd/build.py) first")
        L = ctypes.CDLL(LIB_PATH)
        P, I32 = ctypes.c_void_p, ctypes.c_int32
        AP = ctypes.POINTER(PrefillArgs)
        L.kda_prefill_workspace_bytes.argtypes = [AP]
        L.kda_prefill_workspace_bytes.restype = ctypes.c_size_t
        L.kda_prefill_max_chunks.argtypes = [AP]
        L.kda_prefill_max_chunks.restype = ctypes.c_int64
        L.kda_prefill_chunked.argtypes = [AP, P]
        L.kda_prefill_chunked.restype = I32
        L.kda_prefill_chunked_noalloc.argtypes = [AP, P]
        L.kda_prefill_chunked_noalloc.restype = I32
        L.kda_decode_step.argtypes = [I32, I32, I32, I32, I32, I32, P, P, P, P, P, P, P, P]
        L.kda_decode_step.restype = I32
        L.kda_decode.argtypes = [ctypes.POINTER(DecodeArgs), P]
        L.kda_decode.restype = I32
        L.kda_short_conv.argtypes = [ctypes.POINTER(ConvArgs), P]
        L.kda_short_conv.restype = I32
        BP = ctypes.POINTER(BackwardArgs)
        L.kda_backward_workspace_bytes.argtypes = [BP]
        L.kda_backward_workspace_bytes.restype = ctypes.c_size_t
        L.kda_backward.argtypes = [BP, P]
        L.kda_backward.restype = I32
        L.kda_status_string.argtypes = [I32]
        L.kda_status_string.restype = ctypes.c_char_p
        L.kda_abi_version.restype = I32
        _lib = L
    return _lib


def _status_string(s: int) -> str:
    try:
        return lib().kda_status_string(int(s)).decode()
    except Exception:  # pragma: no cover
        return "?"


def _dt(t: torch.dtype) -> int:
    if t == torch.float32:
        return KDA_F32
    if t == torch.bfloat16:
        return KDA_BF16
    raise TypeError(f"unsupported dtype {t} (float32 or bfloat16)")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_dev(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU (no CPU path exists)")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("tensors are on different devices")
    return dev


def _check_buffer(t, name, shape, dtypes):
    """A caller-supplied output or scratch buffer must have exactly the shape
    and one of the dtypes the kernels will write (they write through raw
    pointers: a smaller or narrower buffer would be overrun)."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must be " + " or ".join(str(d) for d in dtypes) + f", got {t.dtype}")


def _host_chunk_count(B, T, cu_seqlens, chunk_size):
    """Number of chunk_size-token chunks over all sequences (one host copy of
    cu_seqlens when packed)."""
    if cu_seqlens is None:
        return B * ((T + chunk_size - 1) // chunk_size)
    lens = (cu_seqlens[1:] - cu_seqlens[:-1]).cpu().long()
    if bool((lens < 0).any()):
        raise KDAError(_STATUS_BAD_SEQLENS, "cu_seqlens")
    return int(((lens + chunk_size - 1) // chunk_size).sum())


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _make_args(q, k, v, beta, log_alpha, cu_seqlens, chunk_size, out_dtype, cu_host=None, prologue=0):
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    a = PrefillArgs()
    a.B, a.T, a.H, a.d_k, a.d_v = B, T, H, dk, dv
    a.num_seqs = B if cu_seqlens is None else cu_seqlens.numel() - 1
    a.chunk_size = chunk_size
    a.in_dtype = _dt(q.dtype)
    a.out_dtype = _dt(out_dtype)
    a.q, a.k, a.v, a.beta, a.log_alpha = (_ptr(x) for x in (q, k, v, beta, log_alpha))
    a.cu_seqlens = _ptr(cu_seqlens)
    if cu_host is not None:
        a.cu_seqlens_host = cu_host.ctypes.data_as(ctypes.c_void_p)
    a.prologue = int(prologue)
    return a


def workspace_bytes(q, k, v, beta, log_alpha, cu_seqlens=None, chunk_size=64,
                    out_dtype=torch.float32) -> int:
    """Bytes of scratch a prefill call with these inputs needs."""
    return int(lib().kda_prefill_workspace_bytes(
        ctypes.byref(_make_args(q, k, v, beta, log_alpha, cu_seqlens, chunk_size, out_dtype))))


def max_chunks(q, k, v, beta, log_alpha, cu_seqlens=None, chunk_size=64) -> int:
    return int(lib().kda_prefill_max_chunks(
        ctypes.byref(_make_args(q, k, v, beta, log_alpha, cu_seqlens, chunk_size, torch.float32))))


def prefill(q, k, v, beta, log_alpha, initial_state=None, output_final_state=True,
            cu_seqlens=None, chunk_size=64, out_dtype=None, chunk_states=False,
            workspace=None, final_state=None, o=None, check_seqlens=True, timing_events=None,
            prologue=0, device_status=None):
    """Chunked prefill.

    q, k, log_alpha [B,T,H,d_k]; v [B,T,H,d_v]; beta [B,T,H]; all float32 or
    all bfloat16 on one GPU.  ``cu_seqlens`` (int32 [N+1], B == 1) packs N
    documents along T.  ``initial_state`` fp32 [N,H,d_k,d_v] or None (zeros).
    Returns (o, final_state or None) or, with ``chunk_states=True``,
    (o, final_state, chunk_states) where chunk_states[c] is the state entering
    global chunk c (documents in order).

    ``o`` / ``final_state`` / ``workspace``: optional preallocated buffers
    ([B,T,H,d_v] float32 or bfloat16 — the output dtype is taken from ``o``
    when given —, [N,H,d_k,d_v] float32, and at least workspace_bytes()
    bytes); a buffer of another shape or dtype is rejected before launch.
    ``out_dtype`` (default float32) is the dtype of an allocated ``o``.

    ``check_seqlens`` (packed input only, default True) validates cu_seqlens
    on the host (one device-to-host copy) and raises on a device-side
    rejection (one synchronisation).  With ``check_seqlens=False`` nothing
    synchronises; malformed cu_seqlens are still caught on the device, where
    they stop every kernel before it writes, so o and final_state then keep
    whatever their buffers held (uninitialised memory when allocated here):
    the results are UNDEFINED and no error is raised.

    ``timing_events`` (a ctypes pointer to three hipEvent_t) is passed
    through to the library's profiling hook.  ``prologue``: PROLOGUE_* bits
    (which inputs are pre-activations).  ``device_status`` (int32 [1] on the
    device, optional) receives the call's device-side status (0 or a
    kda_status code) without a synchronisation; with packed input and
    ``check_seqlens`` it is read back and raised on as above."""
    dev = _check_dev(q, k, v, beta, log_alpha, initial_state, cu_seqlens, workspace, final_state, o, device_status)
    if not (q.dtype == k.dtype == v.dtype == beta.dtype == log_alpha.dtype):
        raise TypeError("q, k, v, beta, log_alpha must share one dtype")
    if q.dim() != 4 or k.shape != q.shape or log_alpha.shape != q.shape:
        raise ValueError("q, k, log_alpha must be [B,T,H,d_k]")
    B, T, H, dk = q.shape
    if v.dim() != 4 or v.shape[:3] != q.shape[:3] or beta.shape != q.shape[:3]:
        raise ValueError("v must be [B,T,H,d_v] and beta [B,T,H]")
    dv = v.shape[-1]
    if cu_seqlens is not None and cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if initial_state is not None:
        if initial_state.dtype != torch.float32 or tuple(initial_state.shape) != (N, H, dk, dv):
            raise ValueError(f"initial_state must be float32 [{N},{H},{dk},{dv}]")
    if o is not None:
        _check_buffer(o, "o", (B, T, H, dv), (torch.float32, torch.bfloat16))
        if out_dtype is not None and out_dtype != o.dtype:
            raise TypeError(f"out_dtype {out_dtype} disagrees with o.dtype {o.dtype}")
        out_dtype = o.dtype
    elif out_dtype is None:
        out_dtype = torch.float32
    _check_buffer(final_state, "final_state", (N, H, dk, dv), (torch.float32,))
    cu_host = None
    if cu_seqlens is not None and check_seqlens:
        cu_host = cu_seqlens.cpu().numpy()
    a = _make_args(q, k, v, beta, log_alpha, cu_seqlens, chunk_size, out_dtype, cu_host, prologue)
    L = lib()
    need = int(L.kda_prefill_workspace_bytes(ctypes.byref(a)))
    if need == 0:
        st = L.kda_prefill_chunked(ctypes.byref(a), None)  # reports why
        raise KDAError(st, "kda_prefill_chunked")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=out_dtype, device=dev)
    if final_state is None and output_final_state:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    cs = None
    if chunk_states:
        nmax = int(L.kda_prefill_max_chunks(ctypes.byref(a)))
        cs = torch.zeros((nmax, H, dk, dv), dtype=torch.float32, device=dev)
    status = device_status
    if device_status is not None:
        _check_buffer(device_status, "device_status", (1,), (torch.int32,))
    elif check_seqlens and cu_seqlens is not None:
        status = torch.zeros(1, dtype=torch.int32, device=dev)
    a.o = _ptr(o)
    a.initial_state = _ptr(initial_state)
    a.final_state = _ptr(final_state)
    a.chunk_states = _ptr(cs)
    a.device_status = _ptr(status)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = workspace.numel() * workspace.element_size()
    a.timing_events = timing_events
    st = L.kda_prefill_chunked(ctypes.byref(a), _stream(dev))
    if st != 0:
        raise KDAError(st, "kda_prefill_chunked")
    if check_seqlens and cu_seqlens is not None and int(status.item()) != 0:
        raise KDAError(int(status.item()), "kda_prefill_chunked (device check)")
    if chunk_states:
        return o, final_state, cs[:_host_chunk_count(B, T, cu_seqlens, chunk_size)]
    return o, final_state


def prefill_noalloc(q, k, v, beta, log_alpha, o, final_state=None, initial_state=None, cu_seqlens=None,
                    chunk_size=64, prologue=0):
    """Chunked prefill through ``kda_prefill_chunked_noalloc``: the library
    takes its scratch from a fixed per-GPU array (NOALLOC_SCRATCH_BYTES)
    instead of a workspace, and this wrapper allocates nothing either — the
    caller passes ``o`` ([B,T,H,d_v] float32 or bfloat16, which sets the
    output dtype) and, if wanted, ``final_state`` (float32 [N,H,d_k,d_v]).
    cu_seqlens are validated on the device only (no host copy, no
    synchronisation): malformed offsets leave o and final_state unwritten.
    Calls that overlap in time on one GPU race on the shared scratch.
    Raises KDAError (status 7) when the call needs more scratch than the
    array holds.  Returns (o, final_state)."""
    dev = _check_dev(q, k, v, beta, log_alpha, initial_state, cu_seqlens, final_state, o)
    if not (q.dtype == k.dtype == v.dtype == beta.dtype == log_alpha.dtype):
        raise TypeError("q, k, v, beta, log_alpha must share one dtype")
    if q.dim() != 4 or k.shape != q.shape or log_alpha.shape != q.shape:
        raise ValueError("q, k, log_alpha must be [B,T,H,d_k]")
    B, T, H, dk = q.shape
    if v.dim() != 4 or v.shape[:3] != q.shape[:3] or beta.shape != q.shape[:3]:
        raise ValueError("v must be [B,T,H,d_v] and beta [B,T,H]")
    dv = v.shape[-1]
    if cu_seqlens is not None and cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if o is None:
        raise ValueError("prefill_noalloc needs the output buffer o")
    _check_buffer(o, "o", (B, T, H, dv), (torch.float32, torch.bfloat16))
    _check_buffer(initial_state, "initial_state", (N, H, dk, dv), (torch.float32,))
    _check_buffer(final_state, "final_state", (N, H, dk, dv), (torch.float32,))
    a = _make_args(q, k, v, beta, log_alpha, cu_seqlens, chunk_size, o.dtype, None, prologue)
    a.o, a.initial_state, a.final_state = _ptr(o), _ptr(initial_state), _ptr(final_state)
    st = lib().kda_prefill_chunked_noalloc(ctypes.byref(a), _stream(dev))
    if st != 0:
        raise KDAError(st, "kda_prefill_chunked_noalloc")
    return o, final_state


def decode_step(q, k, v, beta, log_alpha, state, out_dtype=torch.float32, o=None):
    """One fused decode step: q, k, log_alpha [B,H,d_k]; v [B,H,d_v];
    beta [B,H]; state fp32 [B,H,d_k,d_v] updated in place.  Returns o [B,H,d_v]."""
    dev = _check_dev(q, k, v, beta, log_alpha, state, o)
    if not (q.dtype == k.dtype == v.dtype == beta.dtype == log_alpha.dtype):
        raise TypeError("q, k, v, beta, log_alpha must share one dtype")
    B, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or log_alpha.shape != q.shape or v.shape[:2] != (B, H) or beta.shape != (B, H):
        raise ValueError("shape mismatch")
    if state.dtype != torch.float32 or tuple(state.shape) != (B, H, dk, dv):
        raise ValueError(f"state must be float32 [{B},{H},{dk},{dv}]")
    _check_buffer(o, "o", (B, H, dv), (torch.float32, torch.bfloat16))
    if o is None:
        o = torch.empty((B, H, dv), dtype=out_dtype, device=dev)
    st = lib().kda_decode_step(B, H, dk, dv, _dt(q.dtype), _dt(o.dtype), _ptr(q), _ptr(k), _ptr(v),
                               _ptr(beta), _ptr(log_alpha), _ptr(state), _ptr(o), _stream(dev))
    if st != 0:
        raise KDAError(st, "kda_decode_step")
    return o


def decode(q, k, v, beta, log_alpha, state, out_dtype=torch.float32, update_state=True,
           token_states=False, prologue=0, o=None, final_state=None):
    """m consecutive tokens per sequence in one launch (multi-token decode /
    speculative verification).

    q, k, log_alpha [B,m,H,d_k]; v [B,m,H,d_v]; beta [B,m,H]; state fp32
    [B,H,d_k,d_v], the state before the first token.  With ``update_state``
    the state after the last token is written back into ``state`` (else into
    ``final_state`` if given, else nowhere, keeping ``state`` for a rollback).
    ``token_states=True`` also returns the state after every token,
    [B,m,H,d_k,d_v].  Returns (o [B,m,H,d_v], final state or None,
    token states or None)."""
    dev = _check_dev(q, k, v, beta, log_alpha, state, o, final_state)
    if not (q.dtype == k.dtype == v.dtype == beta.dtype == log_alpha.dtype):
        raise TypeError("q, k, v, beta, log_alpha must share one dtype")
    if q.dim() != 4 or k.shape != q.shape or log_alpha.shape != q.shape:
        raise ValueError("q, k, log_alpha must be [B,m,H,d_k]")
    B, m, H, dk = q.shape
    if v.dim() != 4 or v.shape[:3] != q.shape[:3] or beta.shape != q.shape[:3]:
        raise ValueError("v must be [B,m,H,d_v] and beta [B,m,H]")
    dv = v.shape[-1]
    if state.dtype != torch.float32 or tuple(state.shape) != (B, H, dk, dv):
        raise ValueError(f"state must be float32 [{B},{H},{dk},{dv}]")
    _check_buffer(o, "o", (B, m, H, dv), (torch.float32, torch.bfloat16))
    _check_buffer(final_state, "final_state", (B, H, dk, dv), (torch.float32,))
    if update_state and final_state is not None and final_state.data_ptr() != state.data_ptr():
        raise ValueError("update_state writes the final state into `state`; do not pass final_state too")
    if o is None:
        o = torch.empty((B, m, H, dv), dtype=out_dtype, device=dev)
    if update_state:
        final_state = state
    ts = torch.empty((B, m, H, dk, dv), dtype=torch.float32, device=dev) if token_states else None
    a = DecodeArgs()
    a.B, a.H, a.d_k, a.d_v, a.n_tokens = B, H, dk, dv, m
    a.in_dtype, a.out_dtype, a.prologue = _dt(q.dtype), _dt(o.dtype), int(prologue)
    a.q, a.k, a.v, a.beta, a.log_alpha = (_ptr(x) for x in (q, k, v, beta, log_alpha))
    a.initial_state, a.final_state, a.token_states, a.o = _ptr(state), _ptr(final_state), _ptr(ts), _ptr(o)
    st = lib().kda_decode(ctypes.byref(a), _stream(dev))
    if st != 0:
        raise KDAError(st, "kda_decode")
    return o, final_state, ts


def short_conv(x, weight, initial_state=None, bias=None, cu_seqlens=None, silu=False,
               out_dtype=None, final_state=None, update_state=False, y=None):
    """Short causal depthwise convolution with a rolling state.

    x [B,T,C] (float32 or bfloat16, C a multiple of 8); weight fp32 [C,W]
    (taps oldest input first, W <= 8); bias fp32 [C] or None; initial_state
    fp32 [N,C,W-1] or None (zeros).  ``cu_seqlens`` (int32 [N+1], B == 1)
    packs N documents along T.  With ``update_state`` the final state is
    written back into ``initial_state`` (decode); else into ``final_state``
    (allocated when None).  Returns (y [B,T,C], final_state)."""
    dev = _check_dev(x, weight, initial_state, bias, cu_seqlens, final_state, y)
    if x.dim() != 3:
        raise ValueError("x must be [B,T,C]")
    B, T, C = x.shape
    if weight.dtype != torch.float32 or weight.dim() != 2 or weight.shape[0] != C:
        raise ValueError(f"weight must be float32 [{C},W]")
    W = weight.shape[1]
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if initial_state is not None and (initial_state.dtype != torch.float32
                                      or tuple(initial_state.shape) != (N, C, W - 1)):
        raise ValueError(f"initial_state must be float32 [{N},{C},{W - 1}]")
    _check_buffer(final_state, "final_state", (N, C, W - 1), (torch.float32,))
    if y is not None:
        _check_buffer(y, "y", (B, T, C), (torch.float32, torch.bfloat16))
        if out_dtype is not None and out_dtype != y.dtype:
            raise TypeError(f"out_dtype {out_dtype} disagrees with y.dtype {y.dtype}")
    if update_state:
        if initial_state is None:
            raise ValueError("update_state needs an initial_state to update")
        if final_state is not None and final_state.data_ptr() != initial_state.data_ptr():
            raise ValueError("update_state writes the final state into initial_state; do not pass final_state too")
        final_state = initial_state
    elif final_state is None:
        final_state = torch.empty((N, C, W - 1), dtype=torch.float32, device=dev)
    if y is None:
        y = torch.empty((B, T, C), dtype=out_dtype or x.dtype, device=dev)
    a = ConvArgs()
    a.B, a.T, a.C, a.W, a.num_seqs = B, T, C, W, N
    a.in_dtype, a.out_dtype, a.activation = _dt(x.dtype), _dt(y.dtype), 1 if silu else 0
    a.x, a.weight, a.bias, a.cu_seqlens = _ptr(x), _ptr(weight), _ptr(bias), _ptr(cu_seqlens)
    a.initial_state, a.final_state, a.y = _ptr(initial_state), _ptr(final_state), _ptr(y)
    st = lib().kda_short_conv(ctypes.byref(a), _stream(dev))
    if st != 0:
        raise KDAError(st, "kda_short_conv")
    return y, final_state


def backward(q, k, v, beta, log_alpha, d_o, initial_state=None, d_final_state=None, cu_seqlens=None,
             checkpoints=None, chunk_size=None, device_status=None):
    """Gradients of the recurrence: (dq, dk, dv, dbeta, dlog_alpha,
    d_initial_state), all float32, from d_o [B,T,H,d_v] fp32 (and
    d_final_state fp32 [N,H,d_k,d_v] or None).  ``checkpoints`` are the
    states entering every chunk of ``chunk_size`` tokens (default 64 for
    bf16 inputs, 16 for fp32); when None they are produced here by a chunked
    prefill with that chunk size.  ``device_status`` (int32 [1] on the
    device, optional) receives the call's device-side status (the
    workspace's status word, copied on the stream: no synchronisation)."""
    dev = _check_dev(q, k, v, beta, log_alpha, d_o, initial_state, d_final_state, cu_seqlens, checkpoints,
                     device_status)
    _check_buffer(device_status, "device_status", (1,), (torch.int32,))
    if not (q.dtype == k.dtype == v.dtype == beta.dtype == log_alpha.dtype):
        raise TypeError("q, k, v, beta, log_alpha must share one dtype")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if d_o.dtype != torch.float32 or tuple(d_o.shape) != (B, T, H, dv):
        raise ValueError(f"d_o must be float32 [{B},{T},{H},{dv}]")
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if cu_seqlens is not None and cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    if chunk_size is None:
        chunk_size = 64 if q.dtype == torch.bfloat16 else 16
    for name, t in (("initial_state", initial_state), ("d_final_state", d_final_state)):
        _check_buffer(t, name, (N, H, dk, dv), (torch.float32,))
    if checkpoints is not None:
        # the kernels address checkpoints through the device chunk table of
        # chunk_size-token chunks: the buffer must hold exactly that many
        nch = _host_chunk_count(B, T, cu_seqlens, chunk_size)
        _check_buffer(checkpoints, "checkpoints", (nch, H, dk, dv), (torch.float32,))
    if checkpoints is None:
        _, _, checkpoints = prefill(q, k, v, beta, log_alpha, initial_state=initial_state,
                                    output_final_state=False, cu_seqlens=cu_seqlens, chunk_size=chunk_size,
                                    chunk_states=True)
    f32 = dict(dtype=torch.float32, device=dev)
    out = dict(dq=torch.empty((B, T, H, dk), **f32), dk=torch.empty((B, T, H, dk), **f32),
               dv=torch.empty((B, T, H, dv), **f32), dbeta=torch.empty((B, T, H), **f32),
               dlog_alpha=torch.empty((B, T, H, dk), **f32), d_initial_state=torch.empty((N, H, dk, dv), **f32))
    a = BackwardArgs()
    a.B, a.T, a.H, a.d_k, a.d_v, a.num_seqs, a.in_dtype = B, T, H, dk, dv, N, _dt(q.dtype)
    a.chunk_size = chunk_size
    a.q, a.k, a.v, a.beta, a.log_alpha = (_ptr(x) for x in (q, k, v, beta, log_alpha))
    a.cu_seqlens, a.checkpoints, a.d_o, a.d_final_state = (_ptr(cu_seqlens), _ptr(checkpoints), _ptr(d_o),
                                                           _ptr(d_final_state))
    for name, t in out.items():
        setattr(a, name, _ptr(t))
    L = lib()
    need = int(L.kda_backward_workspace_bytes(ctypes.byref(a)))
    if need == 0:
        raise KDAError(L.kda_backward(ctypes.byref(a), None), "kda_backward")
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    a.workspace, a.workspace_bytes = _ptr(ws), need
    st = L.kda_backward(ctypes.byref(a), _stream(dev))
    if st != 0:
        raise KDAError(st, "kda_backward")
    if device_status is not None:  # the workspace's first word is the call's status
        device_status.copy_(ws[:4].view(torch.int32))
    return out["dq"], out["dk"], out["dv"], out["dbeta"], out["dlog_alpha"], out["d_initial_state"]
