"""Pins for the CPU oracle, against facts that do not come from the oracle.

* hand-computed cases (tests/golden/hand_cases.json, each with its citation);
* special cases with closed forms: overwrite at alpha = 1, beta = 1, k = e_i;
  pure decay at beta = 0; causal linear attention at alpha = 1 with
  orthonormal keys (one masked matrix product);
* brute force: the explicit dense A_t = (I - beta k k^T) Diag(alpha) product
  (Module 04 — KDA II, §1 "The recurrence has affine form");
* the affine-composition identity and linearity in the initial state;
* invariants: prefix split / continuation (Module 11, §3), packed documents
  share nothing (Module 11, §2 "Padding / packing"), exact power-of-two
  homogeneity, the contraction bound for unit keys and beta in [0, 1];
* mutation tests: plausible mistakes planted in a copy of the oracle's token
  step must each fail at least one of the pins above.

Both oracle forms (numpy and C) are pinned.
"""
import json
import os

import numpy as np
import pytest

from oracle import native, reference as R
import synth

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")))


# ------------------------------------------------------------ helpers ----
def run_numpy(q, k, v, beta, la, S0=None):
    """one sequence, one head: q [T, dk] ... -> (o [T, dv], S_T)"""
    o, S, _ = R.recurrent(q[:, None], k[:, None], v[:, None], beta[:, None], la[:, None],
                          None if S0 is None else np.asarray(S0)[None])
    return o[:, 0], S[0]


def run_c(q, k, v, beta, la, S0=None):
    f = lambda a: np.asarray(a, np.float32)[None, :, None]  # noqa: E731
    o, S, _ = native.prefill(f(q), f(k), f(v), f(beta), f(la),
                             initial_state=None if S0 is None else np.asarray(S0, np.float64)[None, None])
    return o[0, :, 0], S[0, 0]


IMPLS = {"numpy": run_numpy, "c": run_c}


def run_with_step(step, q, k, v, beta, la, S0=None):
    """Token loop over an arbitrary single-token step (used by the mutation tests)."""
    T, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, np.float64)
    o = np.zeros((T, dv))
    for t in range(T):
        S, o[t] = step(S, q[t].astype(np.float64), k[t].astype(np.float64),
                       v[t].astype(np.float64), np.float64(beta[t]), la[t].astype(np.float64))
    return o, S


def arr(x):
    return np.asarray(x, np.float32)


# ----------------------------------------------------- hand cases -------
def check_h1(run):
    c = GOLD["H1_operator_order"]
    o, S = run(arr([c["q"]]), arr([c["k"]]), arr([c["v"]]), arr([c["beta"]]),
               arr([c["log_alpha"]]), np.array(c["S0"]))
    ok = np.allclose(S, c["S1"], atol=c["tol"], rtol=0) and np.allclose(o[0], c["o1"], atol=c["tol"], rtol=0)
    return ok


def check_h2(run):
    c = GOLD["H2_scalar_three_steps"]
    col = lambda x: arr(x)[:, None]  # noqa: E731
    o, S = run(col(c["q"]), col(c["k"]), col(c["v"]), arr(c["beta"]), col(c["log_alpha"]))
    return (np.allclose(o[:, 0], c["o"], atol=c["tol"], rtol=0)
            and abs(S[0, 0] - c["S_final"]) <= c["tol"])


@pytest.mark.parametrize("impl", IMPLS)
def test_h1_operator_order(impl):
    assert check_h1(IMPLS[impl])
    # and the wrong order really is different on this case
    c = GOLD["H1_operator_order"]
    assert not np.allclose(c["S1"], c["S1_wrong_order"])


@pytest.mark.parametrize("impl", IMPLS)
def test_h2_scalar(impl):
    assert check_h2(IMPLS[impl])


def check_h3(run, seed=0):
    """alpha = 1, beta = 1, k = e_i: row i of S becomes v^T, other rows stay."""
    rng = np.random.default_rng(seed)
    dk, dv, i = 5, 3, 2
    S0 = rng.standard_normal((dk, dv))
    k = np.zeros(dk, np.float32)
    k[i] = 1
    v = arr(rng.standard_normal(dv))
    q = arr(rng.standard_normal(dk))
    o, S = run(q[None], k[None], v[None], arr([1.0]), np.zeros((1, dk), np.float32), S0)
    expect = S0.copy()
    expect[i] = v
    return np.allclose(S, expect, atol=1e-12, rtol=0) and np.allclose(o[0], expect.T @ q, atol=1e-12)


@pytest.mark.parametrize("impl", IMPLS)
def test_h3_overwrite(impl):
    assert check_h3(IMPLS[impl])


def check_h4(run, seed=1):
    """beta = 0: S_T = Diag(exp(sum g)) S_0 (decay on the key rows), o_t = S_t^T q_t."""
    rng = np.random.default_rng(seed)
    T, dk, dv = 6, 4, 3
    S0 = rng.standard_normal((dk, dv))
    la = arr(-rng.random((T, dk)))
    q = arr(rng.standard_normal((T, dk)))
    k = arr(rng.standard_normal((T, dk)))
    v = arr(rng.standard_normal((T, dv)))
    o, S = run(q, k, v, np.zeros(T, np.float32), la, S0)
    G = np.cumsum(la.astype(np.float64), axis=0)
    ok = np.allclose(S, np.exp(G[-1])[:, None] * S0, atol=1e-12, rtol=1e-12)
    for t in range(T):
        ok &= np.allclose(o[t], (np.exp(G[t])[:, None] * S0).T @ q[t], atol=1e-12, rtol=1e-12)
    return bool(ok)


@pytest.mark.parametrize("impl", IMPLS)
def test_h4_pure_decay(impl):
    assert check_h4(IMPLS[impl])


def check_h5(run, seed=2):
    """alpha = 1, S_0 = 0, orthonormal keys: the delta rule reduces to causal
    linear attention o = ((Q K^T) * M_inclusive) Diag(beta) V."""
    rng = np.random.default_rng(seed)
    T, dk, dv = 7, 8, 5
    Kq, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    K = arr(Kq[:T])                      # rows orthonormal (to fp32 rounding)
    Q = arr(rng.standard_normal((T, dk)))
    V = arr(rng.standard_normal((T, dv)))
    beta = arr(rng.random(T))
    o, S = run(Q, K, V, beta, np.zeros((T, dk), np.float32))
    K64, Q64, V64 = (a.astype(np.float64) for a in (K, Q, V))
    M = np.tril(np.ones((T, T)))
    expect = ((Q64 @ K64.T) * M) @ (beta.astype(np.float64)[:, None] * V64)
    return np.allclose(o, expect, atol=2e-6, rtol=0)


@pytest.mark.parametrize("impl", IMPLS)
def test_h5_linear_attention(impl):
    assert check_h5(IMPLS[impl])


# ---------------------------------------------- brute force / affine ----
def tiny(seed=3, T=12, dk=6, dv=4, state=True):
    rng = np.random.default_rng(seed)
    q = arr(rng.standard_normal((T, dk)))
    k = rng.standard_normal((T, dk)).astype(np.float32)
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = arr(rng.standard_normal((T, dv)))
    beta = arr(1 / (1 + np.exp(-rng.standard_normal(T))))
    la = arr(-np.log1p(np.exp(rng.standard_normal((T, dk)))))
    S0 = rng.standard_normal((dk, dv)) * 0.3 if state else None
    return q, k, v, beta, la, S0


def check_dense(run, seed=3):
    q, k, v, beta, la, S0 = tiny(seed)
    o, S = run(q, k, v, beta, la, S0)
    od, Sd = R.recurrent_dense(q, k, v, beta, la, S0)
    return np.allclose(o, od, atol=1e-12, rtol=0) and np.allclose(S, Sd, atol=1e-12, rtol=0)


@pytest.mark.parametrize("impl", IMPLS)
def test_brute_force_dense_transition(impl):
    assert check_dense(IMPLS[impl])


def test_dense_transition_is_the_closed_form():
    """The dense matrix is (I - beta k k^T) D, checked entrywise by its
    definition on a 2x2 case (and differs from D (I - beta k k^T))."""
    k = np.array([0.6, 0.8])
    A, Bm = R.transition(k, 0.5, np.log([0.9, 0.4]), np.array([1.0, -2.0]))
    D = np.diag([0.9, 0.4])
    for i in range(2):
        for j in range(2):
            assert abs(A[i, j] - ((i == j) - 0.5 * k[i] * k[j]) * D[j, j]) < 1e-15
    assert not np.allclose(A, D @ (np.eye(2) - 0.5 * np.outer(k, k)))
    assert np.allclose(Bm, 0.5 * np.outer(k, [1.0, -2.0]))


def check_affine(run, seed=4):
    """S_T = A S_0 + B with (A, B) accumulated by (A_t A, A_t B + B_t); and
    run(S_0) - run(0) = A S_0 (linearity in the initial state)."""
    q, k, v, beta, la, S0 = tiny(seed)
    dk, dv = k.shape[1], v.shape[1]
    A, Bm = np.eye(dk), np.zeros((dk, dv))
    for t in range(len(q)):
        A, Bm = R.compose(R.transition(k[t], beta[t], la[t], v[t]), (A, Bm))
    _, S = run(q, k, v, beta, la, S0)
    _, S_zero = run(q, k, v, beta, la, None)
    return (np.allclose(S, A @ S0 + Bm, atol=1e-12, rtol=0)
            and np.allclose(S - S_zero, A @ S0, atol=1e-12, rtol=0))


@pytest.mark.parametrize("impl", IMPLS)
def test_affine_composition(impl):
    assert check_affine(IMPLS[impl])


@pytest.mark.parametrize("chunk", [1, 3, 4, 5, 12, 13])
def test_chunked_affine_matches_recurrence(chunk):
    """Module 04 §4 test design on the oracle's own chunked (dense, composed)
    form: outputs, final state and every boundary state, for chunk sizes that
    do and do not divide T."""
    q, k, v, beta, la, S0 = tiny(5, T=12)
    o, S, snaps = R.recurrent(q[:, None], k[:, None], v[:, None], beta[:, None], la[:, None],
                              S0[None], snap_every=chunk)
    oc, Sc, bounds = R.chunked_affine(q, k, v, beta, la, chunk, S0)
    assert np.allclose(oc, o[:, 0], atol=1e-12, rtol=0)
    assert np.allclose(Sc, S[0], atol=1e-12, rtol=0)
    assert len(bounds) == len(snaps)
    for b, s in zip(bounds, snaps):
        assert np.allclose(b, s[0], atol=1e-12, rtol=0)


# ------------------------------------------------------- invariants -----
def test_prefix_split_continuation():
    """One pass == two passes with the state carried (Module 11, §3)."""
    x = synth.make_uniform(11, 1, 40, 3, 8, 6, "bf16", state_std=0.1)
    o, S, _ = native.prefill(x.q, x.k, x.v, x.beta, x.log_alpha, initial_state=x.initial_state)
    for a in (1, 17, 39):
        o1, S1, _ = native.prefill(x.q[:, :a], x.k[:, :a], x.v[:, :a], x.beta[:, :a],
                                   x.log_alpha[:, :a], initial_state=x.initial_state)
        o2, S2, _ = native.prefill(x.q[:, a:], x.k[:, a:], x.v[:, a:], x.beta[:, a:],
                                   x.log_alpha[:, a:], initial_state=S1)
        assert np.array_equal(np.concatenate([o1, o2], axis=1), o)
        assert np.array_equal(S2, S)


def test_packed_equals_separate():
    """No state crosses a document boundary: packed == separate calls, and a
    change inside one document leaves every other document's results bitwise
    unchanged (Module 11, §2, "Padding / packing")."""
    lens = [5, 0, 9, 1, 14]
    x = synth.make_packed(12, lens, 2, 8, 4, "bf16", state_std=0.1)
    o, S, _ = native.prefill(x.q, x.k, x.v, x.beta, x.log_alpha, x.cu_seqlens, x.initial_state)
    cu = x.cu_seqlens
    for n in range(len(lens)):
        t0, t1 = cu[n], cu[n + 1]
        on, Sn, _ = native.prefill(x.q[:, t0:t1], x.k[:, t0:t1], x.v[:, t0:t1], x.beta[:, t0:t1],
                                   x.log_alpha[:, t0:t1], initial_state=x.initial_state[n:n + 1])
        assert np.array_equal(on, o[:, t0:t1])
        assert np.array_equal(Sn, S[n:n + 1])
    # zero-length document: final = initial
    assert np.array_equal(S[1], x.initial_state[1].astype(np.float64))
    # perturb document 2 only
    v2 = x.v.copy()
    v2[:, cu[2]:cu[3]] += 1.0
    o2, S2, _ = native.prefill(x.q, x.k, v2, x.beta, x.log_alpha, cu, x.initial_state)
    keep = np.ones(x.T, bool)
    keep[cu[2]:cu[3]] = False
    assert np.array_equal(o2[:, keep], o[:, keep])
    assert np.array_equal(np.delete(S2, 2, 0), np.delete(S, 2, 0))
    assert not np.array_equal(S2[2], S[2])


def test_power_of_two_homogeneity_bitwise():
    x = synth.make_uniform(13, 2, 30, 2, 8, 8, "f32", state_std=0.5)
    o, S, _ = native.prefill(x.q, x.k, x.v, x.beta, x.log_alpha, initial_state=x.initial_state)
    o2, S2, _ = native.prefill(x.q, x.k, 2 * x.v, x.beta, x.log_alpha,
                               initial_state=2 * x.initial_state)
    assert np.array_equal(o2, 2 * o) and np.array_equal(S2, 2 * S)


def test_output_linear_in_q():
    x = synth.make_uniform(14, 1, 20, 2, 8, 8, "f32")
    # dyadic values so that q1 + q2 is exact in fp32
    q1 = np.round(x.q * 64).astype(np.float32) / 64
    q2 = np.round(np.random.default_rng(0).standard_normal(x.q.shape) * 64).astype(np.float32) / 64
    o1, _, _ = native.prefill(q1, x.k, x.v, x.beta, x.log_alpha)
    o2, _, _ = native.prefill(q2, x.k, x.v, x.beta, x.log_alpha)
    o3, _, _ = native.prefill(q1 + q2, x.k, x.v, x.beta, x.log_alpha)
    assert np.allclose(o3, o1 + o2, atol=1e-12 * (1 + np.abs(o3).max()))


def test_contraction_bound():
    """Unit keys and beta in [0, 1] make every A_t a contraction in the
    spectral norm, so ||S_t||_2 <= ||S_{t-1}||_2 + beta_t ||v_t||."""
    q, k, v, beta, la, S0 = tiny(6, T=25, dk=8, dv=8)
    S = S0.copy()
    for t in range(len(q)):
        A, _ = R.transition(k[t], beta[t], la[t], v[t])
        assert np.linalg.norm(A, 2) <= 1 + 1e-12
        _, S_next = run_c(q[t:t + 1], k[t:t + 1], v[t:t + 1], beta[t:t + 1], la[t:t + 1], S)
        assert np.linalg.norm(S_next, 2) <= np.linalg.norm(S, 2) + beta[t] * np.linalg.norm(v[t]) + 1e-12
        S = S_next


def test_c_and_numpy_agree_on_a_workload():
    x = synth.make_packed(15, [33, 64, 7], 3, 16, 16, "bf16")
    o1, S1, c1 = native.prefill(x.q, x.k, x.v, x.beta, x.log_alpha, x.cu_seqlens,
                                x.initial_state, chunk=16, want_chunk_states=True)
    o2, S2, c2 = R.prefill(x.q, x.k, x.v, x.beta, x.log_alpha, x.cu_seqlens, x.initial_state,
                           snap_every=16)
    assert np.allclose(o1, o2, atol=1e-12) and np.allclose(S1, S2, atol=1e-12)
    assert np.allclose(c1, np.stack(c2), atol=1e-12)


def test_metric():
    ref = np.array([3.0, -4.0])               # RMS = sqrt(12.5)
    assert abs(R.rel_err(ref + [0.0, 0.5], ref) - 0.5 / np.sqrt(12.5)) < 1e-15
    assert R.rel_err(np.zeros(3), np.zeros(3)) == 0.0
    assert R.rel_err(np.array([0, 1e-30, 0]), np.zeros(3)) == float("inf")


# ------------------------------------------------------- mutations ------
def _good(S, q, k, v, b, g):
    S = np.exp(g)[:, None] * S
    e = v - S.T @ k
    S = S + b * np.outer(k, e)
    return S, S.T @ q


def _wrong_order(S, q, k, v, b, g):            # D (I - beta k k^T) S + beta k v^T
    S = S - b * np.outer(k, k @ S)
    S = np.exp(g)[:, None] * S + b * np.outer(k, v)
    return S, S.T @ q


def _read_before_write(S, q, k, v, b, g):      # o from the pre-write state
    S = np.exp(g)[:, None] * S
    o = S.T @ q
    S = S + b * np.outer(k, v - S.T @ k)
    return S, o


def _predict_before_decay(S, q, k, v, b, g):   # p = S_{t-1}^T k
    e = v - S.T @ k
    S = np.exp(g)[:, None] * S + b * np.outer(k, e)
    return S, S.T @ q


def _decay_on_value_axis(S, q, k, v, b, g):    # D applied to columns
    S = S * np.exp(g)[None, : S.shape[1]] if S.shape[0] == S.shape[1] else S * np.exp(g[0])
    S = S + b * np.outer(k, v - S.T @ k)
    return S, S.T @ q


def _transposed_read(S, q, k, v, b, g):        # o = S q instead of S^T q
    S, _ = _good(S, q, k, v, b, g)
    return S, (S @ q[: S.shape[1]] if S.shape[0] == S.shape[1] else S[: len(q)].T @ q)


def _dropped_beta(S, q, k, v, b, g):
    return _good(S, q, k, v, 1.0, g)


def _sign_error(S, q, k, v, b, g):             # e = p - v
    S = np.exp(g)[:, None] * S
    S = S + b * np.outer(k, S.T @ k - v)
    return S, S.T @ q


def _no_exp(S, q, k, v, b, g):                 # alpha taken as log_alpha
    S = g[:, None] * S
    S = S + b * np.outer(k, v - S.T @ k)
    return S, S.T @ q


MUTANTS = [_wrong_order, _read_before_write, _predict_before_decay, _decay_on_value_axis,
           _transposed_read, _dropped_beta, _sign_error, _no_exp]


def _pins_pass(step):
    run = lambda *a: run_with_step(step, *a)  # noqa: E731
    return all([check_h1(run), check_h2(run), check_h3(run), check_h4(run), check_h5(run),
                check_dense(run), check_affine(run)])


def test_unmutated_step_passes_pins():
    assert _pins_pass(_good)


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda f: f.__name__)
def test_mutation_is_caught(mutant):
    assert not _pins_pass(mutant)
