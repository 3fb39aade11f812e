"""Pins for the oracle's short causal convolution (Module 04 — KDA II, §3
"The sublayer is bigger than the recurrence"; its rolling state is serving
state, Module 11, §2, row "Serving state").

* a hand-computed impulse response and a continuation from a given state
  (tests/golden, C1), which fix the tap order;
* a library routine: each channel equals scipy.signal.lfilter with the taps
  reversed (an FIR filter) on zero state;
* invariants: splitting a sequence and carrying the state equals one pass,
  packed documents equal separate calls, a width-1 filter is a per-channel
  scale, SiLU equals y * scipy's expit(y);
* mutation tests: a reversed tap order or a dropped state fails a pin.
"""
import json
import os

import numpy as np
import pytest
import scipy.signal as sig
import scipy.special as sp

from oracle import reference as R

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")))


def _hand(conv):
    c = GOLD["C1_conv_impulse"]
    w = np.array([c["w"]])
    y, fin = conv(np.array(c["x"])[None, :, None], w, None)
    y2, fin2 = conv(np.array(c["x2"])[None, :, None], w, np.array(c["state2"])[None, None])
    return (np.array_equal(y[0, :, 0], c["y"]) and np.array_equal(fin[0, 0], c["final"])
            and np.array_equal(y2[0, :, 0], c["y2"]) and np.array_equal(fin2[0, 0], c["final2"]))


def test_hand_impulse_and_continuation():
    assert _hand(lambda x, w, s: R.short_conv(x, w, initial_state=s))


MUTANTS = {
    "reversed_taps": lambda x, w, s: R.short_conv(x, w[:, ::-1], initial_state=s),
    "state_dropped": lambda x, w, s: R.short_conv(x, w, initial_state=None),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_conv_mutation_is_caught(name):
    assert not _hand(MUTANTS[name])


@pytest.mark.parametrize("W", [1, 2, 3, 4, 8])
def test_matches_fir_filter(W):
    rng = np.random.default_rng(W)
    x = rng.standard_normal((2, 50, 6))
    w = rng.standard_normal((6, W))
    y, _ = R.short_conv(x, w)
    for b in range(2):
        for c in range(6):
            ref = sig.lfilter(w[c, ::-1], [1.0], x[b, :, c])
            np.testing.assert_allclose(y[b, :, c], ref, rtol=1e-13, atol=1e-13)


def test_width_one_is_a_scale():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((1, 9, 5))
    w = rng.standard_normal((5, 1))
    y, fin = R.short_conv(x, w)
    assert np.array_equal(y, x * w[:, 0]) and fin.shape == (1, 5, 0)


@pytest.mark.parametrize("W", [2, 4])
def test_split_with_state_equals_one_pass(W):
    rng = np.random.default_rng(10 + W)
    x = rng.standard_normal((1, 40, 7))
    w = rng.standard_normal((7, W))
    s0 = rng.standard_normal((1, 7, W - 1))
    y, fin = R.short_conv(x, w, initial_state=s0)
    for cut in (1, 2, 17, 39):
        ya, sa = R.short_conv(x[:, :cut], w, initial_state=s0)
        yb, sb = R.short_conv(x[:, cut:], w, initial_state=sa)
        np.testing.assert_allclose(np.concatenate([ya, yb], 1), y, rtol=0, atol=1e-14)
        np.testing.assert_allclose(sb, fin, rtol=0, atol=0)


def test_short_sequences_take_the_state_from_before():
    """A sequence shorter than W - 1 keeps the tail of its incoming state."""
    w = np.ones((1, 4))
    s0 = np.array([[[1.0, 2.0, 3.0]]])
    y, fin = R.short_conv(np.array([[[10.0]]]), w, initial_state=s0)
    assert y[0, 0, 0] == 16.0 and np.array_equal(fin[0, 0], [2.0, 3.0, 10.0])
    y0, fin0 = R.short_conv(np.zeros((1, 0, 1)), w, initial_state=s0)
    assert np.array_equal(fin0, s0)


def test_packed_equals_separate():
    rng = np.random.default_rng(3)
    lens = [5, 0, 1, 12]
    cu = np.concatenate([[0], np.cumsum(lens)])
    x = rng.standard_normal((1, cu[-1], 3))
    w = rng.standard_normal((3, 3))
    s0 = rng.standard_normal((4, 3, 2))
    y, fin = R.short_conv(x, w, cu_seqlens=cu, initial_state=s0)
    for n in range(4):
        yn, fn = R.short_conv(x[:, cu[n]:cu[n + 1]], w, initial_state=s0[n:n + 1])
        assert np.array_equal(y[:, cu[n]:cu[n + 1]], yn) and np.array_equal(fin[n], fn[0])


def test_bias_and_silu():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((1, 20, 4))
    w = rng.standard_normal((4, 3))
    bias = rng.standard_normal(4)
    lin, _ = R.short_conv(x, w, bias=bias)
    nob, _ = R.short_conv(x, w)
    np.testing.assert_allclose(lin - nob, np.broadcast_to(bias, lin.shape), rtol=0, atol=1e-14)
    act, _ = R.short_conv(x, w, bias=bias, silu=True)
    np.testing.assert_allclose(act, lin * sp.expit(lin), rtol=1e-15, atol=1e-15)
