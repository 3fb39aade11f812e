"""Multi-token decode / speculative verification (Module 11 — Correctness as
Architecture Mastery, §2 "The full correctness matrix", row "Serving state":
speculative rollback must restore the recurrent state).  m tokens per
sequence in one launch against the fp64 oracle's token-by-token trajectory:
every token's output, every per-token state and the final state; a rollback
to an accepted prefix continues exactly like a run that never saw the
rejected tokens.  Called through the C ABI via the Python binding."""
import numpy as np
import pytest
import torch

import gated_delta_rule_49_amd as kda
import synth
from oracle import native
from kda_testutil import TOL, err, report, tdtype

pytestmark = pytest.mark.gpu


def draw(seed, B, m, H, dk, dv, dtype):
    """[B, m, H, d] tokens and an N(0, 0.02^2) state, as the decode workload draws them."""
    x = synth.decode_workload(B=B, H=H, dk=dk, dv=dv, steps=m, seed=seed, dtype=dtype, state_std=0.02)
    tok = [np.ascontiguousarray(np.swapaxes(a, 0, 1)) for a in (x.q, x.k, x.v, x.beta, x.log_alpha)]
    return tok, x.initial_state


def oracle(tok, S0, flags=0):
    """Per-token outputs, states after every token and the final state."""
    B, m = tok[0].shape[:2]
    o, fin, cs = native.prefill(*tok, initial_state=S0, chunk=1, want_chunk_states=True, prologue_flags=flags)
    cs = cs.reshape((B, m) + cs.shape[1:])   # state ENTERING token j of row b
    after = np.concatenate([cs[:, 1:], fin[:, None]], axis=1)
    return o, after, fin


@pytest.mark.parametrize("m", [1, 2, 4, 8])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_multi_token_parity(m, dtype):
    tok, S0 = draw(70 + m, 6, m, 4, 128, 128, dtype)
    args = [torch.from_numpy(a).cuda().to(tdtype(dtype)) for a in tok]
    S = torch.from_numpy(S0).cuda()
    o, fin, ts = kda.decode(*args, S, update_state=False, final_state=torch.empty_like(S), token_states=True)
    o_ref, after_ref, fin_ref = oracle(tok, S0)
    e = dict(o=err(o, o_ref), S=err(fin, fin_ref),
             tokens=max(err(ts[:, j], after_ref[:, j]) for j in range(m)))
    report(f"multi-token decode m={m} B=6 H=4 d=128 {dtype}", **e)
    assert max(e.values()) <= TOL[dtype]
    assert torch.equal(S.cpu(), torch.from_numpy(S0)), "update_state=False must leave the state alone"
    assert torch.equal(ts[:, -1], fin)


@pytest.mark.parametrize("B,m,H,dk,dv", [(150, 4, 4, 128, 128), (275, 3, 4, 64, 32), (130, 4, 5, 16, 16)])
def test_multi_token_states_persistent_walk_with_uneven_share(B, m, H, dk, dv):
    """With per-token states, m up to 4 (d=128) runs on the persistent grid of
    512 workgroups; 600, 1100 and 650 states give workgroups shares that end
    on either half of the prefetch walk."""
    tok, S0 = draw(75 + B, B, m, H, dk, dv, "bf16")
    args = [torch.from_numpy(a).cuda().to(torch.bfloat16) for a in tok]
    S = torch.from_numpy(S0).cuda()
    o, fin, ts = kda.decode(*args, S, token_states=True)     # in place
    o_ref, after_ref, fin_ref = oracle(tok, S0)
    e = dict(o=err(o, o_ref), S=err(fin, fin_ref),
             tokens=max(err(ts[:, j], after_ref[:, j]) for j in range(m)))
    report(f"multi-token decode m={m} B={B} H={H} d={dk}x{dv} bf16, token states", **e)
    assert max(e.values()) <= TOL["bf16"]
    assert fin is S and torch.equal(ts[:, -1], fin)


@pytest.mark.parametrize("m", [2, 3, 4])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("flags", [0, 7])
def test_multi_token_state_only(m, dtype, flags):
    """Launches without per-token states (the state updated in place), with
    and without the fused prologue: every output and the final state against
    the oracle.  150 x 4 = 600 states give the persistent workgroups an
    uneven share."""
    B, H = 150, 4
    x = synth.make_preact(95 + m + flags, B, m, H, 128, 128, dtype, state_std=0.02, prologue=flags)
    args = [torch.from_numpy(a).cuda().to(tdtype(dtype)) for a in (x.q, x.k, x.v, x.beta, x.log_alpha)]
    S = torch.from_numpy(x.initial_state).cuda()
    o, fin, ts = kda.decode(*args, S, prologue=flags)
    o_ref, S_ref, _ = native.prefill(x.q, x.k, x.v, x.beta, x.log_alpha, initial_state=x.initial_state,
                                     prologue_flags=flags)
    e = dict(o=err(o, o_ref), S=err(S, S_ref))
    report(f"state-only multi-token decode m={m} {dtype} prologue={flags}", **e)
    assert max(e.values()) <= TOL[dtype]
    assert fin is S and ts is None


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 128), (128, 16)])
def test_multi_token_head_sizes(dk, dv):
    tok, S0 = draw(80 + dk + dv, 3, 3, 2, dk, dv, "f32")
    args = [torch.from_numpy(a).cuda() for a in tok]
    S = torch.from_numpy(S0).cuda()
    o, fin, ts = kda.decode(*args, S, token_states=True)     # in place
    o_ref, after_ref, fin_ref = oracle(tok, S0)
    e = dict(o=err(o, o_ref), S=err(S, fin_ref), tokens=max(err(ts[:, j], after_ref[:, j]) for j in range(3)))
    report(f"multi-token decode d={dk}x{dv} f32", **e)
    assert max(e.values()) <= TOL["f32"]
    assert fin is S


def test_single_token_matches_decode_step_bitwise():
    tok, S0 = draw(90, 8, 1, 4, 128, 128, "bf16")
    args = [torch.from_numpy(a).cuda().to(torch.bfloat16) for a in tok]
    S1 = torch.from_numpy(S0).cuda()
    S2 = S1.clone()
    o1, _, _ = kda.decode(*args, S1)
    o2 = kda.decode_step(*(a[:, 0] for a in args), S2)
    assert torch.equal(o1[:, 0], o2) and torch.equal(S1, S2)


def test_multi_token_equals_repeated_steps():
    """m tokens in one launch vs m single-token launches: same arithmetic per
    token, so equal within fp32 rounding (reported: bitwise or not)."""
    tok, S0 = draw(91, 5, 6, 3, 128, 128, "bf16")
    args = [torch.from_numpy(a).cuda().to(torch.bfloat16) for a in tok]
    S1 = torch.from_numpy(S0).cuda()
    S2 = S1.clone()
    o1, _, _ = kda.decode(*args, S1)
    o2 = torch.stack([kda.decode_step(*(a[:, j].contiguous() for a in args), S2) for j in range(6)], 1)
    d = dict(o=err(o1, o2.double().cpu().numpy()), S=err(S1, S2.double().cpu().numpy()))
    report(f"multi vs repeated (bitwise={torch.equal(o1, o2) and torch.equal(S1, S2)})", **d)
    assert max(d.values()) <= 1e-6


def test_speculative_rollback():
    """Verify m = 4 drafted tokens, accept the first j per sequence, restore
    the state after token j - 1 (or the untouched state for j = 0), then
    decode 2 more tokens: equal to the oracle run on the accepted tokens only."""
    B, m, H, d = 6, 4, 3, 128
    tok, S0 = draw(92, B, m, H, d, d, "bf16")
    nxt, _ = draw(93, B, 2, H, d, d, "bf16")
    accept = np.array([0, 1, 2, 3, 4, 2])
    dev = [torch.from_numpy(a).cuda().to(torch.bfloat16) for a in tok]
    S = torch.from_numpy(S0).cuda()
    _, _, ts = kda.decode(*dev, S, update_state=False, token_states=True)
    for b in range(B):
        if accept[b] > 0:
            S[b] = ts[b, accept[b] - 1]
    o2, _, _ = kda.decode(*(torch.from_numpy(a).cuda().to(torch.bfloat16) for a in nxt), S)
    # oracle: per sequence, the accepted drafted tokens then the 2 new ones
    worst_o = worst_s = 0.0
    for b in range(B):
        j = accept[b]
        seq = [np.concatenate([t[b:b + 1, :j], n[b:b + 1]], axis=1) for t, n in zip(tok, nxt)]
        o_ref, fin_ref, _ = native.prefill(*seq, initial_state=S0[b:b + 1])
        worst_o = max(worst_o, err(o2[b:b + 1], o_ref[:, j:]))
        worst_s = max(worst_s, err(S[b:b + 1], fin_ref))
    report("speculative rollback", o=worst_o, S=worst_s)
    assert worst_o <= TOL["bf16"] and worst_s <= TOL["bf16"]
