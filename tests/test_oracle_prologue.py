"""Pins for the oracle's prologue: the pre-recurrence stages of the executed
sublayer (Q/K normalisation, the decay gate producing alpha, the write gate
producing beta; Module 04 — KDA II, §3 "The sublayer is bigger than the
recurrence").

* library routines: -softplus(x) = log(sigmoid(-x)) (scipy's log_expit) and
  exp(-softplus(x)) = sigmoid(-x), sigmoid = scipy's expit, over a grid that
  includes values where a naive formula overflows;
* closed forms: softplus(x) - softplus(-x) = x, the 3-4-5 triangle for the
  norm, zero stays zero;
* a hand-computed scalar trajectory (tests/golden, H6) run through both
  oracle forms with every prologue stage on;
* mutation tests: a sign flip or a dropped stage planted in a copy of the
  prologue fails the hand case.
"""
import json
import os

import numpy as np
import pytest
import scipy.special as sp

from oracle import native, reference as R
import synth

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")))
ALL = R.PRO_GATE_SOFTPLUS | R.PRO_BETA_SIGMOID | R.PRO_QK_L2NORM
GRID = np.concatenate([np.linspace(-30, 30, 601), [-745.0, -700.0, -88.0, 88.0, 700.0, 745.0, 1e4, -1e4]])


def test_gate_matches_library_log_sigmoid():
    np.testing.assert_allclose(-R.softplus(GRID), sp.log_expit(-GRID), rtol=1e-15, atol=1e-300)
    np.testing.assert_allclose(np.exp(-R.softplus(GRID)), sp.expit(-GRID), rtol=1e-14, atol=1e-300)


def test_softplus_closed_forms():
    assert R.softplus(0.0) == pytest.approx(np.log(2.0), rel=1e-16)
    x = GRID[np.abs(GRID) < 700]
    np.testing.assert_allclose(R.softplus(x) - R.softplus(-x), x, rtol=1e-13, atol=1e-13)
    assert np.all(R.softplus(GRID) >= 0) and np.all(np.isfinite(R.softplus(GRID)))


def test_sigmoid_matches_library():
    np.testing.assert_allclose(R.sigmoid(GRID), sp.expit(GRID), rtol=1e-15, atol=1e-300)
    assert R.sigmoid(np.log(3.0)) == pytest.approx(0.75, rel=1e-15)


def test_l2norm_closed_forms():
    y = R.l2norm(np.array([3.0, 4.0]))
    np.testing.assert_allclose(y, [0.6, 0.8], rtol=0, atol=2e-8)   # eps shifts by 1.2e-8
    assert np.all(R.l2norm(np.zeros(8)) == 0.0)
    x = np.random.default_rng(0).standard_normal((50, 128))
    n = np.linalg.norm(R.l2norm(x), axis=-1)
    np.testing.assert_allclose(n, 1.0, rtol=0, atol=1e-7)
    # direction is kept: the normalised vector is a positive multiple of x
    cos = np.sum(R.l2norm(x) * x, -1) / np.linalg.norm(x, axis=-1)
    np.testing.assert_allclose(cos, 1.0, rtol=0, atol=1e-7)


def _h6(run_prologue):
    c = GOLD["H6_prologue_scalar"]
    col = lambda a: np.asarray(a, np.float64)[:, None]  # noqa: E731
    q, k, beta, la = run_prologue(col(c["q"]), col(c["k"]), np.asarray(c["beta_x"], np.float64),
                                  col(c["gate_x"]))
    o, S, _ = R.recurrent(q[:, None], k[:, None], col(c["v"])[:, None], beta[:, None], la[:, None],
                          np.array([[[c["S0"]]]]))
    return (np.allclose(o[:, 0, 0], c["o"], atol=c["tol"], rtol=0)
            and abs(S[0, 0, 0] - c["S_final"]) <= c["tol"])


def test_hand_case_numpy():
    assert _h6(lambda q, k, b, g: R.prologue(q, k, b, g, ALL))


def test_hand_case_c():
    c = GOLD["H6_prologue_scalar"]
    f = lambda a: np.asarray(a, np.float32).reshape(1, 3, 1, 1)  # noqa: E731
    o, S, _ = native.prefill(f(c["q"]), f(c["k"]), f(c["v"]), np.asarray(c["beta_x"], np.float32).reshape(1, 3, 1),
                             f(c["gate_x"]), initial_state=np.full((1, 1, 1, 1), c["S0"]), prologue_flags=ALL)
    np.testing.assert_allclose(o[0, :, 0, 0], c["o"], atol=c["tol"], rtol=0)
    assert abs(S[0, 0, 0, 0] - c["S_final"]) <= c["tol"]


MUTANTS = {
    "gate_sign": lambda q, k, b, g: (R.l2norm(q), R.l2norm(k), R.sigmoid(b), -R.softplus(-g)),
    "beta_sign": lambda q, k, b, g: (R.l2norm(q), R.l2norm(k), R.sigmoid(-b), -R.softplus(g)),
    "no_k_norm": lambda q, k, b, g: (R.l2norm(q), k, R.sigmoid(b), -R.softplus(g)),
    "no_q_norm": lambda q, k, b, g: (q, R.l2norm(k), R.sigmoid(b), -R.softplus(g)),
    "gate_not_negated": lambda q, k, b, g: (R.l2norm(q), R.l2norm(k), R.sigmoid(b), R.softplus(g)),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_prologue_mutation_is_caught(name):
    assert not _h6(MUTANTS[name])


@pytest.mark.parametrize("flags", [1, 2, 4, 7])
def test_c_and_numpy_prologue_agree(flags):
    x = synth.make_uniform(11, 2, 40, 3, 16, 8, "f32", state_std=0.1)
    rng = np.random.default_rng(5)
    # pre-activations: raw gate / beta draws, unnormalised q and k
    q = rng.standard_normal(x.q.shape).astype(np.float32) * 3
    k = rng.standard_normal(x.k.shape).astype(np.float32) * 3
    b = rng.standard_normal(x.beta.shape).astype(np.float32) * 2
    g = rng.standard_normal(x.log_alpha.shape).astype(np.float32) * 2
    on, Sn, _ = R.prefill(q, k, x.v, b, g, initial_state=x.initial_state, prologue_flags=flags)
    oc, Sc, _ = native.prefill(q, k, x.v, b, g, initial_state=x.initial_state, prologue_flags=flags)
    assert R.rel_err(oc, on) < 1e-12 and R.rel_err(Sc, Sn) < 1e-12


def test_prologue_off_is_identity():
    x = synth.make_uniform(12, 1, 20, 2, 16, 16, "f32")
    a = native.prefill(x.q, x.k, x.v, x.beta, x.log_alpha)
    b = native.prefill(x.q, x.k, x.v, x.beta, x.log_alpha, prologue_flags=0)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
