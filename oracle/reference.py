"""CPU oracle for the KDA gated delta-rule recurrence (numpy, fp64).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link anything under ``oracle/``; only the test suite, the smoke check and the
benchmark's CPU-baseline leg do.  It shares no code with the HIP path.

What is computed (per sequence n and head h; S is d_k x d_v, fp64):

    S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
    o_t = S_t^T q_t

* The closed form and the operator order (I - beta k k^T) D, not
  D (I - beta k k^T): "GLM-5.3-Flash Architecture Mastery" course index,
  Course Outcomes (the closed form) and Exit Criteria (five lines expanded to
  the closed form); Module 11 — Correctness as Architecture Mastery, §2 "The
  full correctness matrix", KDA row (operator order); Module 12 — Capstone,
  §1 (ordering errors diverge silently).
* The five named operations are not printed on the pages (their Module 03 is
  not among them).  Reading taken: decay, predict, error, write, read — the
  plainest expansion that multiplies out to the closed form above:
      S'  = Diag(alpha_t) S_{t-1}          decay
      p   = S'^T k_t                       predict
      e   = v_t - p                        error
      S_t = S' + beta_t k_t e^T            write
      o_t = S_t^T q_t                      read (post-update state)
  (S' + beta k (v - S'^T k)^T = (I - beta k k^T) S' + beta k v^T.)
* alpha_t = exp(log_alpha_t) is per key channel: D acts on the rows of S.
* No query scale is applied (the pages show none).
* The affine form S_{t+1} = A_{t+1} S_t + B_{t+1} and its composition
  (A2 A1, A2 B1 + B2): Module 04 — KDA II, §1 "The recurrence has affine form".
* Chunked execution agrees with the recurrence on outputs, final state and
  the state at every chunk boundary: Module 04, §4 "The correctness
  invariant".  Packed documents never share state: Module 11, §2, row
  "Padding / packing".

Inputs are taken as given (bf16 inputs arrive widened exactly to fp32) and
computed on in fp64.
"""
from __future__ import annotations

import numpy as np

f64 = np.float64


# ---------------------------------------------------------- prologue ----
# The stages that run just before the recurrence in the executed sublayer:
# Q/K normalisation, a decay gate that produces alpha and a write gate that
# produces beta (Module 04 — KDA II, §3 "The sublayer is bigger than the
# recurrence").  The pages name the stages but give no formulas; the forms
# below are the ones the workload descriptions use for their inputs (k "then
# L2-normalised", beta = sigmoid(x), alpha = exp(-softplus(x))).  Reading for
# the norm: x / sqrt(sum x^2 + eps) with eps = 1e-6, so a zero vector stays
# zero instead of becoming NaN.
PRO_GATE_SOFTPLUS = 1   # log_alpha holds x; the gate is log alpha = -softplus(x)
PRO_BETA_SIGMOID = 2    # beta holds x; beta = sigmoid(x)
PRO_QK_L2NORM = 4       # q and k are L2-normalised over d_k per (token, head)
QK_NORM_EPS = 1e-6


def softplus(x):
    """log(1 + e^x), evaluated without overflow: max(x, 0) + log1p(e^-|x|)."""
    x = np.asarray(x, f64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def sigmoid(x):
    """1 / (1 + e^-x), evaluated without overflow on either side."""
    x = np.asarray(x, f64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def l2norm(x, eps=QK_NORM_EPS):
    """x / sqrt(sum over the last axis of x^2 + eps)."""
    x = np.asarray(x, f64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def prologue(q, k, beta, log_alpha, flags):
    """Apply the selected pre-recurrence stages (flags: PRO_* bits) in fp64.
    Returns (q, k, beta, log_alpha) as the recurrence consumes them."""
    q, k, beta, log_alpha = (np.asarray(a, f64) for a in (q, k, beta, log_alpha))
    if flags & PRO_QK_L2NORM:
        q, k = l2norm(q), l2norm(k)
    if flags & PRO_BETA_SIGMOID:
        beta = sigmoid(beta)
    if flags & PRO_GATE_SOFTPLUS:
        log_alpha = -softplus(log_alpha)
    return q, k, beta, log_alpha


# ---------------------------------------------------- short convolution --
# The short causal convolution of the executed sublayer, a small local mixing
# step on q, k and/or v before the recurrence (Module 04 — KDA II, §3 "The
# sublayer is bigger than the recurrence"); its rolling state is part of the
# serving state a rollback must restore (Module 11, §2, row "Serving state").
# The pages give neither the width nor the form.  Reading: depthwise (one
# filter per channel), causal, width W, taps ordered oldest input first:
#     y_t[c] = sum_{j=0}^{W-1} w[c, j] * x_{t-W+1+j}[c]  (+ bias[c]),
# optionally followed by SiLU (y * sigmoid(y)); inputs before a sequence's
# first token come from its conv state (the W-1 inputs that preceded it,
# oldest first), or are zero.
def short_conv(x, weight, cu_seqlens=None, initial_state=None, bias=None, silu=False):
    """x [B, T, C]; weight [C, W]; initial_state [N, C, W-1] or None (zeros);
    bias [C] or None.  Sequences are the B rows, or with ``cu_seqlens``
    (B == 1) the documents packed along T.  Returns (y [B, T, C] fp64,
    final_state [N, C, W-1] fp64: the last W-1 inputs of each sequence, taken
    from its initial state where the sequence is shorter)."""
    x = np.asarray(x, f64)
    w = np.asarray(weight, f64)
    B, T, Cc = x.shape
    W = w.shape[1]
    if cu_seqlens is None:
        seqs = [(b, 0, T) for b in range(B)]
    else:
        seqs = [(0, int(cu_seqlens[n]), int(cu_seqlens[n + 1])) for n in range(len(cu_seqlens) - 1)]
    y = np.zeros_like(x)
    final = np.zeros((len(seqs), Cc, W - 1), f64)
    for n, (b, t0, t1) in enumerate(seqs):
        hist = (np.zeros((W - 1, Cc)) if initial_state is None
                else np.asarray(initial_state[n], f64).T)           # [W-1, C], oldest first
        xp = np.concatenate([hist, x[b, t0:t1]], axis=0)             # [W-1+L, C]
        L = t1 - t0
        acc = np.zeros((L, Cc))
        for j in range(W):
            acc += w[:, j] * xp[j:j + L]
        if bias is not None:
            acc += np.asarray(bias, f64)
        if silu:
            acc = acc * sigmoid(acc)
        y[b, t0:t1] = acc
        final[n] = xp[L:L + W - 1].T
    return y, final


# ------------------------------------------------------- one token ------
def step(S, q, k, v, beta, log_alpha):
    """One token of the recurrence, batched over any leading axes.

    S [..., dk, dv]; q, k, log_alpha [..., dk]; v [..., dv]; beta [...].
    Returns (S_t, o_t)."""
    S = np.exp(log_alpha)[..., :, None] * S                 # decay
    p = np.einsum("...kv,...k->...v", S, k)                  # predict
    e = v - p                                                # error
    S = S + beta[..., None, None] * k[..., :, None] * e[..., None, :]  # write
    o = np.einsum("...kv,...k->...v", S, q)                  # read
    return S, o


def recurrent(q, k, v, beta, log_alpha, S0=None, snap_every=0):
    """Token-by-token recurrence for ONE sequence.

    q, k, log_alpha [T, H, dk]; v [T, H, dv]; beta [T, H]; S0 [H, dk, dv] or None.
    Returns (o [T, H, dv], S_T [H, dk, dv], snaps) where ``snaps`` lists the
    state entering tokens 0, c, 2c, ... (c = snap_every) if snap_every > 0."""
    q, k, v, beta, log_alpha = (np.asarray(a, dtype=f64) for a in (q, k, v, beta, log_alpha))
    T, H, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((H, dk, dv), f64) if S0 is None else np.array(S0, dtype=f64)
    o = np.zeros((T, H, dv), f64)
    snaps = []
    for t in range(T):
        if snap_every and t % snap_every == 0:
            snaps.append(S.copy())
        S, o[t] = step(S, q[t], k[t], v[t], beta[t], log_alpha[t])
    return o, S, snaps


def prefill(q, k, v, beta, log_alpha, cu_seqlens=None, initial_state=None, snap_every=0, prologue_flags=0):
    """Batched / packed driver.  Layouts as the kernels': q [B,T,H,dk] ...;
    with ``cu_seqlens`` (B == 1) every document starts from its own state
    (``initial_state[n]`` or zeros) and shares nothing with its neighbours.
    ``prologue_flags`` (PRO_* bits) says which inputs are pre-activations.

    Returns (o [B,T,H,dv] fp64, final [N,H,dk,dv] fp64, snaps) where snaps is
    the concatenation over documents of the state entering each chunk."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    q, k, beta, log_alpha = prologue(q, k, beta, log_alpha, prologue_flags)
    if cu_seqlens is None:
        seqs = [(b, 0, T) for b in range(B)]
    else:
        seqs = [(0, int(cu_seqlens[n]), int(cu_seqlens[n + 1])) for n in range(len(cu_seqlens) - 1)]
    o = np.zeros((B, T, H, dv), f64)
    final = np.zeros((len(seqs), H, dk, dv), f64)
    snaps = []
    for n, (b, t0, t1) in enumerate(seqs):
        S0 = None if initial_state is None else initial_state[n]
        on, Sn, sn = recurrent(q[b, t0:t1], k[b, t0:t1], v[b, t0:t1], beta[b, t0:t1],
                               log_alpha[b, t0:t1], S0, snap_every)
        o[b, t0:t1] = on
        final[n] = Sn
        snaps.extend(sn)
    return o, final, snaps


# ------------------------------------------------------------ backward --
# Gradients of the recurrence.  The pages call the affine composition the
# argument for parallel training (course index, module list, the Module 04
# entry) but derive no backward pass; this is reverse-mode differentiation of
# the five operations of one token, applied from the last token to the first:
#   read   o = S_t^T q           dS_t += q do^T          dq = S_t do
#   write  S_t = S' + b k e^T    dS' = dS_t, u = dS_t^T k, de = b u,
#                                db = u.e, dk += b dS_t e
#   error  e = v - p             dv = de, dp = -de
#   predict p = S'^T k           dS' += k dp^T, dk += S' dp
#   decay  S' = Diag(a) S        dS_{t-1} = Diag(a) dS', d(log a) = a * rowsum(dS' * S)
def recurrent_backward(q, k, v, beta, log_alpha, d_o, S0=None, dS_T=None):
    """One sequence: q, k, log_alpha [T, H, dk]; v, d_o [T, H, dv]; beta [T, H];
    S0, dS_T [H, dk, dv] or None (zeros).  Returns the gradients
    (dq, dk, dv, dbeta, dlog_alpha, dS0) of the scalar loss whose gradients
    with respect to o and S_T are d_o and dS_T."""
    q, k, v, beta, log_alpha, d_o = (np.asarray(a, dtype=f64) for a in (q, k, v, beta, log_alpha, d_o))
    T, H, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((H, dk, dv), f64) if S0 is None else np.array(S0, dtype=f64)
    states = [S]                                   # S_0 .. S_T
    for t in range(T):
        S, _ = step(S, q[t], k[t], v[t], beta[t], log_alpha[t])
        states.append(S)
    dS = np.zeros((H, dk, dv), f64) if dS_T is None else np.array(dS_T, dtype=f64)
    g = {n: np.zeros_like(a) for n, a in (("q", q), ("k", k), ("v", v), ("b", beta), ("g", log_alpha))}
    for t in range(T - 1, -1, -1):
        a = np.exp(log_alpha[t])                              # [H, dk]
        Sp = a[..., None] * states[t]                         # S'
        p = np.einsum("hkv,hk->hv", Sp, k[t])
        e = v[t] - p
        St = states[t + 1]
        dS = dS + q[t][..., None] * d_o[t][:, None, :]         # read
        g["q"][t] = np.einsum("hkv,hv->hk", St, d_o[t])
        u = np.einsum("hkv,hk->hv", dS, k[t])                   # write
        de = beta[t][:, None] * u
        g["b"][t] = np.sum(u * e, axis=-1)
        dk_t = beta[t][:, None] * np.einsum("hkv,hv->hk", dS, e)
        g["v"][t] = de                                          # error
        dp = -de
        dSp = dS + k[t][..., None] * dp[:, None, :]             # predict
        dk_t = dk_t + np.einsum("hkv,hv->hk", Sp, dp)
        g["k"][t] = dk_t
        g["g"][t] = a * np.sum(dSp * states[t], axis=-1)        # decay
        dS = a[..., None] * dSp
    return g["q"], g["k"], g["v"], g["b"], g["g"], dS


# -------------------------------------------- dense affine form ---------
def transition(k, beta, log_alpha, v):
    """Explicit dense affine step for one head and token:
    A_t = (I - beta k k^T) Diag(alpha),  B_t = beta k v^T."""
    k = np.asarray(k, f64)
    dk = k.shape[0]
    A = (np.eye(dk) - beta * np.outer(k, k)) @ np.diag(np.exp(np.asarray(log_alpha, f64)))
    Bm = beta * np.outer(k, np.asarray(v, f64))
    return A, Bm


def compose(later, earlier):
    """Affine composition: applying ``earlier`` then ``later`` equals
    (A_l A_e, A_l B_e + B_l)."""
    A2, B2 = later
    A1, B1 = earlier
    return A2 @ A1, A2 @ B1 + B2


def recurrent_dense(q, k, v, beta, log_alpha, S0=None):
    """One head, one sequence: S <- A_t S + B_t with dense A_t, o_t = S_t^T q_t.
    q, k, log_alpha [T, dk]; v [T, dv]; beta [T]."""
    T, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((dk, dv), f64) if S0 is None else np.array(S0, f64)
    o = np.zeros((T, dv), f64)
    for t in range(T):
        A, Bm = transition(k[t], beta[t], log_alpha[t], v[t])
        S = A @ S + Bm
        o[t] = S.T @ np.asarray(q[t], f64)
    return o, S


def chunked_affine(q, k, v, beta, log_alpha, chunk, S0=None):
    """One head: the chunked execution the pages describe, in dense form.

    Each chunk's transitions are composed into one (A, B) independently of
    the incoming state; chunks are then applied in order.  Outputs inside a
    chunk use the prefix composition up to that token.  Dense d_k x d_k
    matrices: tiny inputs only.  Returns (o, S_T, boundary states)."""
    T, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((dk, dv), f64) if S0 is None else np.array(S0, f64)
    o = np.zeros((T, dv), f64)
    bounds = []
    for c0 in range(0, T, chunk):
        bounds.append(S.copy())
        acc = (np.eye(dk), np.zeros((dk, dv)))
        prefix = []
        for t in range(c0, min(T, c0 + chunk)):
            acc = compose(transition(k[t], beta[t], log_alpha[t], v[t]), acc)
            prefix.append(acc)
        for j, (A, Bm) in enumerate(prefix):
            o[c0 + j] = (A @ S + Bm).T @ np.asarray(q[c0 + j], f64)
        A, Bm = prefix[-1]
        S = A @ S + Bm
    return o, S, bounds


# ----------------------------------------------------- the metric -------
def rel_err(x, ref):
    """max |x - ref| / RMS(ref).  If RMS(ref) == 0 the comparison requires
    exact zeros: 0.0 when x is all zero, else inf."""
    x = np.asarray(x, f64)
    ref = np.asarray(ref, f64)
    rms = np.sqrt(np.mean(ref * ref)) if ref.size else 0.0
    d = np.max(np.abs(x - ref)) if ref.size else 0.0
    if rms > 0:
        return d / rms
    return 0.0 if d == 0 else float("inf")
