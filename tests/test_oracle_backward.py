"""Pins for the oracle's backward pass (reverse-mode through the five
operations of a token; the pages derive none, so the pins are independent
of any formula: central finite differences of the fp64 forward oracle).

* every gradient (q, k, v, beta, log_alpha, the initial state) against
  central differences of L = sum(R * o) + sum(Q * S_T) for random R, Q, at
  several heads and sizes, with per-channel gates;
* closed form: with beta = 0 the state only decays, so dL/dS0 =
  Diag(exp(sum g)) Q plus the contributions of the outputs, checked in the
  scalar case by hand;
* mutation tests: a dropped decay chain rule, a dropped predict term, a
  sign error in dp and the read taken before the write, each planted in a
  copy, fail the finite-difference pin (the unplanted copy passes).
"""
import numpy as np
import pytest

from oracle import reference as R


def loss(x, Rm, Qm, S0):
    o, S, _ = R.recurrent(x["q"], x["k"], x["v"], x["b"], x["g"], S0)
    return float(np.sum(Rm * o) + np.sum(Qm * S))


def draw(seed, T, H, dk, dv):
    rng = np.random.default_rng(seed)
    x = dict(q=rng.standard_normal((T, H, dk)), k=rng.standard_normal((T, H, dk)) / np.sqrt(dk),
             v=rng.standard_normal((T, H, dv)), b=rng.uniform(0.1, 0.9, (T, H)),
             g=-rng.uniform(0.05, 1.0, (T, H, dk)))
    S0 = rng.standard_normal((H, dk, dv)) * 0.5
    return x, S0, rng.standard_normal((T, H, dv)), rng.standard_normal((H, dk, dv))


def finite_diff(x, Rm, Qm, S0, eps=1e-6):
    grads = {}
    for n in ("q", "k", "v", "b", "g"):
        gr = np.zeros_like(x[n])
        it = np.nditer(x[n], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = {m: a.copy() for m, a in x.items()}
            xm = {m: a.copy() for m, a in x.items()}
            xp[n][idx] += eps
            xm[n][idx] -= eps
            gr[idx] = (loss(xp, Rm, Qm, S0) - loss(xm, Rm, Qm, S0)) / (2 * eps)
        grads[n] = gr
    gS = np.zeros_like(S0)
    it = np.nditer(S0, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        Sp, Sm = S0.copy(), S0.copy()
        Sp[idx] += eps
        Sm[idx] -= eps
        gS[idx] = (loss(x, Rm, Qm, Sp) - loss(x, Rm, Qm, Sm)) / (2 * eps)
    grads["S0"] = gS
    return grads


def analytic(x, Rm, Qm, S0, fn=R.recurrent_backward):
    dq, dk, dv, db, dg, dS0 = fn(x["q"], x["k"], x["v"], x["b"], x["g"], Rm, S0, Qm)
    return dict(q=dq, k=dk, v=dv, b=db, g=dg, S0=dS0)


@pytest.mark.parametrize("seed,T,H,dk,dv", [(1, 5, 1, 3, 2), (2, 7, 2, 4, 3), (3, 4, 1, 6, 6)])
def test_gradients_match_finite_differences(seed, T, H, dk, dv):
    x, S0, Rm, Qm = draw(seed, T, H, dk, dv)
    fd = finite_diff(x, Rm, Qm, S0)
    an = analytic(x, Rm, Qm, S0)
    for n in fd:
        scale = max(np.max(np.abs(fd[n])), 1e-3)
        assert np.max(np.abs(an[n] - fd[n])) / scale < 1e-7, n


def test_pure_decay_scalar_closed_form():
    """d = 1, beta = 0: S_t = a_1..a_t S0, o_t = q_t S_t.  With L = sum_t r_t o_t
    + Q S_T: dL/dS0 = sum_t r_t q_t prod_{i<=t} a_i + Q prod_i a_i, and
    dL/dv = 0 (nothing is written)."""
    a = np.array([0.5, 0.25, 0.8])
    qv = np.array([1.0, 2.0, -1.0])
    r = np.array([3.0, -1.0, 2.0])
    Q = 0.7
    x = dict(q=qv[:, None, None], k=np.ones((3, 1, 1)), v=np.array([1.0, 2.0, 3.0])[:, None, None],
             b=np.zeros((3, 1)), g=np.log(a)[:, None, None])
    an = analytic(x, r[:, None, None], np.array([[[Q]]]), np.array([[[1.5]]]))
    cum = np.cumprod(a)
    want = np.sum(r * qv * cum) + Q * cum[-1]
    assert abs(an["S0"][0, 0, 0] - want) < 1e-14
    assert np.all(an["v"] == 0.0)


def _planted(mistake):
    """A copy of the oracle's backward with one plausible mistake planted."""
    def bwd(q, k, v, beta, log_alpha, d_o, S0=None, dS_T=None):
        T, H, dk = q.shape
        dv = v.shape[-1]
        S = np.array(S0, dtype=float)
        states = [S]
        for t in range(T):
            S, _ = R.step(S, q[t], k[t], v[t], beta[t], log_alpha[t])
            states.append(S)
        dS = np.array(dS_T, dtype=float)
        out = [np.zeros_like(q), np.zeros_like(k), np.zeros_like(v), np.zeros_like(beta), np.zeros_like(log_alpha)]
        for t in range(T - 1, -1, -1):
            a = np.exp(log_alpha[t])
            Sp = a[..., None] * states[t]
            e = v[t] - np.einsum("hkv,hk->hv", Sp, k[t])
            dS = dS + q[t][..., None] * d_o[t][:, None, :]
            St = states[t] if mistake == "read_before_write" else states[t + 1]
            out[0][t] = np.einsum("hkv,hv->hk", St, d_o[t])
            u = np.einsum("hkv,hk->hv", dS, k[t])
            de = beta[t][:, None] * u
            out[3][t] = np.sum(u * e, -1)
            dkt = beta[t][:, None] * np.einsum("hkv,hv->hk", dS, e)
            out[2][t] = de
            dp = de if mistake == "dp_sign" else -de
            dSp = dS + k[t][..., None] * dp[:, None, :]
            if mistake != "no_predict":
                dkt = dkt + np.einsum("hkv,hv->hk", Sp, dp)
            out[1][t] = dkt
            out[4][t] = (1.0 if mistake == "no_decay_chain" else a) * np.sum(dSp * states[t], -1)
            dS = a[..., None] * dSp
        return (*out, dS)
    return bwd


def test_planted_copy_without_mistake_passes():
    x, S0, Rm, Qm = draw(4, 4, 1, 3, 2)
    fd = finite_diff(x, Rm, Qm, S0)
    an = analytic(x, Rm, Qm, S0, fn=_planted("none"))
    assert all(np.max(np.abs(an[n] - fd[n])) / max(np.max(np.abs(fd[n])), 1e-3) < 1e-7 for n in fd)


@pytest.mark.parametrize("mistake", ["no_decay_chain", "no_predict", "dp_sign", "read_before_write"])
def test_backward_mutation_is_caught(mistake):
    x, S0, Rm, Qm = draw(4, 4, 1, 3, 2)
    fd = finite_diff(x, Rm, Qm, S0)
    an = analytic(x, Rm, Qm, S0, fn=_planted(mistake))
    assert any(np.max(np.abs(an[n] - fd[n])) / max(np.max(np.abs(fd[n])), 1e-3) > 1e-4 for n in fd)
