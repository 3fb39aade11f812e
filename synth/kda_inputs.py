"""Seeded synthetic inputs for the KDA gated delta-rule recurrence.

This module is shared by the CPU oracle's tests and the GPU path's tests and
benchmark.  It draws random numbers and shapes them into the inputs the
recurrence consumes; it performs none of the recurrence's own arithmetic.

Input preparation (the sublayer stages *before* the recurrence, Module 04 §3
"The sublayer is bigger than the recurrence": Q/K normalisation, decay gate,
write gate) is done here on the synthetic pre-activations:

* k is L2-normalised per (token, head) in fp32,
* beta = sigmoid(x),
* log_alpha = -softplus(x)  (so alpha = exp(log_alpha) lies in (0, 1)).

bf16 workloads are rounded to bf16 with round-to-nearest-even *after* these
steps; the arrays returned here hold the rounded values widened back to fp32
(exactly), so every consumer sees identical inputs.

Layouts (row-major, contiguous):
    q, k       [B, T, H, d_k]
    v          [B, T, H, d_v]
    beta       [B, T, H]
    log_alpha  [B, T, H, d_k]
    state      [N, H, d_k, d_v]   (N = number of sequences)
For packed workloads B == 1 and ``cu_seqlens`` (int32, [N+1]) delimits the
documents along T.

Random stream: torch's generator on the device given (``device="cpu"`` by
default; large workloads are drawn on the GPU, which is much faster — the
same seed gives different, equally valid, inputs on a different device
type).  Draws are made in fp32 in the order q, k, v, beta_raw, gate_raw,
then the initial state.  Long inputs are drawn in blocks of ``BLOCK_TOKENS``
tokens with seeds ``seed * 100003 + block`` so any block can be regenerated on
its own.  Results are returned as host numpy arrays.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

BLOCK_TOKENS = 8192


# ---------------------------------------------------------------- bf16 -----
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 -> bf16 (round to nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bits to fp32 exactly."""
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 array whose values are the bf16 (RNE) roundings of ``x``."""
    return bits_to_f32(bf16_bits(x))


# ------------------------------------------------------- activations -------
def _gen(seed: int, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _to_np(t):
    return t.detach().to("cpu").numpy()


# ---------------------------------------------------------- container ------
@dataclasses.dataclass
class KDAInputs:
    """One synthetic workload.  All float arrays are fp32 (bf16-exact if
    ``dtype == 'bf16'``)."""

    name: str
    dtype: str  # 'f32' or 'bf16' : the element type handed to the kernels
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    beta: np.ndarray
    log_alpha: np.ndarray
    initial_state: Optional[np.ndarray]  # fp32 [N,H,dk,dv] or None (zeros)
    cu_seqlens: Optional[np.ndarray]  # int32 [N+1] or None (B rows)
    chunk_size: int
    # non-zero: q, k, beta, log_alpha hold the raw pre-activations of the
    # stages before the recurrence (bit 1 gate, bit 2 beta, bit 4 q/k norm)
    prologue: int = 0

    @property
    def B(self) -> int:
        return self.q.shape[0]

    @property
    def T(self) -> int:
        return self.q.shape[1]

    @property
    def H(self) -> int:
        return self.q.shape[2]

    @property
    def d_k(self) -> int:
        return self.q.shape[3]

    @property
    def d_v(self) -> int:
        return self.v.shape[3]

    @property
    def num_seqs(self) -> int:
        return self.B if self.cu_seqlens is None else len(self.cu_seqlens) - 1

    def seq_bounds(self):
        """[(row, start, end)] of every sequence along (B, T)."""
        if self.cu_seqlens is None:
            return [(b, 0, self.T) for b in range(self.B)]
        c = self.cu_seqlens
        return [(0, int(c[n]), int(c[n + 1])) for n in range(len(c) - 1)]


# ------------------------------------------------------------ drawing ------
def _draw_tokens(g, B, T, H, dk, dv, gate_mean=0.0, device="cpu", bf16=False):
    """Token inputs as torch fp32 tensors on ``device``."""
    kw = dict(generator=g, device=device, dtype=torch.float32)
    q = torch.randn((B, T, H, dk), **kw)
    k = torch.randn((B, T, H, dk), **kw)
    v = torch.randn((B, T, H, dv), **kw)
    beta_raw = torch.randn((B, T, H), **kw)
    gate_raw = torch.randn((B, T, H, dk), **kw)
    if gate_mean:
        gate_raw += gate_mean
    k = k / torch.clamp(torch.linalg.vector_norm(k, dim=-1, keepdim=True), min=1e-12)
    beta = torch.sigmoid(beta_raw)
    log_alpha = -torch.nn.functional.softplus(gate_raw)
    out = [q, k, v, beta, log_alpha]
    if bf16:
        out = [t.to(torch.bfloat16).to(torch.float32) for t in out]
    return out


def _state(g, shape, std, device):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std


def make_uniform(seed: int, B: int, T: int, H: int, dk: int, dv: int, dtype: str,
                 chunk: int = 64, state_std: float = 0.0, gate_mean: float = 0.0,
                 name: str = "custom", device="cpu") -> KDAInputs:
    """B independent rows of T tokens, typical gates; optional N(0, std^2) state."""
    g = _gen(seed, device)
    q, k, v, beta, la = _draw_tokens(g, B, T, H, dk, dv, gate_mean, device, dtype == "bf16")
    state = _to_np(_state(g, (B, H, dk, dv), state_std, device)) if state_std else None
    return KDAInputs(name, dtype, *(_to_np(t) for t in (q, k, v, beta, la)), state, None, chunk)


def make_preact(seed: int, B: int, T: int, H: int, dk: int, dv: int, dtype: str,
                chunk: int = 64, state_std: float = 0.0, name: str = "preact",
                device="cpu", prologue: int = 7) -> KDAInputs:
    """Inputs for the fused prologue: q, k, v, beta_raw and gate_raw ~ N(0, 1)
    drawn in the same order as the other workloads.  The stages selected by
    ``prologue`` (bit 1 gate, bit 2 beta, bit 4 q/k norm) are left as raw
    pre-activations; the others are applied here as for the other workloads
    (k normalised, beta = sigmoid, log alpha = -softplus), so that the
    recurrence always sees keys of unit norm and gates in range."""
    g = _gen(seed, device)
    out = preact_tensors(g, B, T, H, dk, dv, dtype, device, prologue)
    if dtype == "bf16":
        out = [t.to(torch.float32) for t in out]
    state = _to_np(_state(g, (B, H, dk, dv), state_std, device)) if state_std else None
    return KDAInputs(name, dtype, *(_to_np(t) for t in out), state, None, chunk, prologue=prologue)


def preact_tensors(g, B, T, H, dk, dv, dtype="bf16", device="cpu", prologue=7):
    """The token draws of ``make_preact`` as torch tensors on ``device``
    (bf16 tensors for dtype 'bf16'), for benchmarks that keep them there."""
    kw = dict(generator=g, device=device, dtype=torch.float32)
    q, k, v, beta, la = (torch.randn((B, T, H, dk), **kw), torch.randn((B, T, H, dk), **kw),
                         torch.randn((B, T, H, dv), **kw), torch.randn((B, T, H), **kw),
                         torch.randn((B, T, H, dk), **kw))
    if not prologue & 4:
        k = k / torch.clamp(torch.linalg.vector_norm(k, dim=-1, keepdim=True), min=1e-12)
    if not prologue & 2:
        beta = torch.sigmoid(beta)
    if not prologue & 1:
        la = -torch.nn.functional.softplus(la)
    out = [q, k, v, beta, la]
    if dtype == "bf16":
        out = [t.to(torch.bfloat16) for t in out]
    return out


def make_packed(seed: int, lengths, H: int, dk: int, dv: int, dtype: str, chunk: int = 64,
                state_std: float = 0.02, name: str = "packed", device="cpu") -> KDAInputs:
    """Documents of the given lengths concatenated along T (B == 1)."""
    g = _gen(seed, device)
    T = int(np.sum(lengths))
    q, k, v, beta, la = _draw_tokens(g, 1, T, H, dk, dv, 0.0, device, dtype == "bf16")
    n = len(lengths)
    state = _to_np(_state(g, (n, H, dk, dv), state_std, device)) if state_std else None
    cu = np.zeros(n + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return KDAInputs(name, dtype, *(_to_np(t) for t in (q, k, v, beta, la)), state, cu, chunk)


def _extreme_block(g, T, H, dk, device):
    """Per token: Bernoulli(0.1) selects the token (all heads); selected
    tokens get log_alpha ~ U[-20, -10] per (head, channel) and beta drawn
    from {1e-4, 1 - 1e-4} with probability 1/2 each per (token, head)."""
    kw = dict(generator=g, device=device, dtype=torch.float32)
    sel = torch.rand((T,), **kw) < 0.1
    la = torch.rand((T, H, dk), **kw) * 10.0 - 20.0
    bsel = torch.rand((T, H), **kw) < 0.5
    b = torch.where(bsel, torch.tensor(1e-4, device=device), torch.tensor(1.0 - 1e-4, device=device))
    return sel, la, b


def long_tensors(seed: int, T: int, H: int, dk: int, dv: int, dtype: str = "bf16",
                 extreme: bool = True, device="cpu"):
    """[q, k, v, beta, log_alpha] of one long row as torch fp32 tensors on
    ``device`` (bf16-exact if dtype == 'bf16'), drawn in BLOCK_TOKENS blocks
    with seed ``seed * 100003 + block``; with ``extreme`` the stress pattern
    of :func:`_extreme_block` is applied per block."""
    shapes = [(1, T, H, dk), (1, T, H, dk), (1, T, H, dv), (1, T, H), (1, T, H, dk)]
    out = [torch.empty(sh, dtype=torch.float32, device=device) for sh in shapes]
    nblk = (T + BLOCK_TOKENS - 1) // BLOCK_TOKENS
    for i in range(nblk):
        t0, t1 = i * BLOCK_TOKENS, min(T, (i + 1) * BLOCK_TOKENS)
        g = _gen(seed * 100003 + i, device)
        bq, bk, bv, bb, bla = _draw_tokens(g, 1, t1 - t0, H, dk, dv, 0.0, device, False)
        if extreme:
            sel, xla, xb = _extreme_block(g, t1 - t0, H, dk, device)
            bla[0, sel] = xla[sel]
            bb[0, sel] = xb[sel]
        parts = [bq, bk, bv, bb, bla]
        if dtype == "bf16":
            parts = [t.to(torch.bfloat16).to(torch.float32) for t in parts]
        for dst, src in zip(out, parts):
            dst[:, t0:t1] = src
    return out


def make_long(seed: int, T: int, H: int, dk: int, dv: int, dtype: str = "bf16",
              chunk: int = 64, extreme: bool = True, name: str = "long", device="cpu") -> KDAInputs:
    """One long row (see :func:`long_tensors`) as host arrays."""
    ts = long_tensors(seed, T, H, dk, dv, dtype, extreme, device)
    arrs = []
    while ts:
        arrs.append(_to_np(ts.pop(0)))  # frees each device tensor as it is copied
    return KDAInputs(name, dtype, *arrs, None, None, chunk)


# -------------------------------------------------- the five workloads ----
C4_DOCS = 8


def c4_lengths(seed: int = 4):
    """8 lengths uniform on [512, 8192] (numpy PCG64, so identical on every host)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(512, 8193, size=C4_DOCS).tolist()


def workload(idx: int, device="cpu", **over) -> KDAInputs:
    """The five named workloads (seed = workload index):

    1  tiny fp32: B=1 H=1 T=64 d=16, chunk 16, zero state
    2  prefill:   B=1 H=16 T=4096 d=128 bf16, chunk 64, zero state
    3  decode:    see :func:`decode_workload`
    4  packed:    8 docs, lengths U[512, 8192], H=32 d=128 bf16, chunk 64,
                  per-document N(0, 0.02^2) state
    5  long:      B=1 H=32 T=131072 d=128 bf16, chunk 64, 10% extreme gates
    """
    if idx == 1:
        return make_uniform(1, 1, 64, 1, 16, 16, "f32", chunk=16, name="tiny_f32_T64_d16",
                            device=device)
    if idx == 2:
        return make_uniform(2, 1, over.get("T", 4096), over.get("H", 16), 128, 128, "bf16",
                            chunk=64, name="prefill_T4096_H16_d128", device=device)
    if idx == 4:
        lens = over.get("lengths", c4_lengths(4))
        return make_packed(4, lens, over.get("H", 32), 128, 128, "bf16", chunk=64,
                           name="packed_8docs_H32_d128", device=device)
    if idx == 5:
        return make_long(5, over.get("T", 131072), over.get("H", 32), 128, 128, "bf16",
                         chunk=64, name="long_T131072_H32_d128_extreme", device=device)
    raise ValueError(f"workload {idx}: use decode_workload() for 3")


@dataclasses.dataclass
class DecodeInputs:
    """``steps`` single-token steps for B sequences (q,k,v,beta,log_alpha have a
    leading step axis: [steps, B, H, d] / [steps, B, H])."""

    name: str
    dtype: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    beta: np.ndarray
    log_alpha: np.ndarray
    initial_state: np.ndarray  # fp32 [B,H,dk,dv]


def decode_workload(B: int = 256, H: int = 32, dk: int = 128, dv: int = 128,
                    steps: int = 64, seed: int = 3, dtype: str = "bf16",
                    state_std: float = 0.02, name: str = "decode_B256_H32_d128",
                    device="cpu") -> DecodeInputs:
    """Workload 3: per step fresh q,k,v,beta,alpha (as in workload 1, rounded
    to bf16); initial state N(0, 0.02^2) fp32, drawn after the token inputs."""
    g = _gen(seed, device)
    # steps play the role of T with one token per sequence: [steps, B, H, d]
    q, k, v, beta, la = _draw_tokens(g, steps, B, H, dk, dv, 0.0, device, dtype == "bf16")
    state = _state(g, (B, H, dk, dv), state_std, device)
    return DecodeInputs(name, dtype, *(_to_np(t) for t in (q, k, v, beta, la, state)))


def slow_decay(seed: int, B: int, T: int, H: int, dk: int, dv: int, dtype: str = "bf16",
               chunk: int = 64, state_std: float = 0.02, device="cpu") -> KDAInputs:
    """Supplementary case: log_alpha = -softplus(N(-5, 1)) (alpha ~ 0.99), so
    state carried across chunk boundaries dominates the outputs."""
    return make_uniform(seed, B, T, H, dk, dv, dtype, chunk=chunk, state_std=state_std,
                        gate_mean=-5.0, name="slow_decay", device=device)
