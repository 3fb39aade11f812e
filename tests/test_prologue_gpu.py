"""Fused prologue parity: the pre-recurrence stages (Q/K normalisation, the
decay gate log alpha = -softplus(x), the write gate beta = sigmoid(x);
Module 04 — KDA II, §3 "The sublayer is bigger than the recurrence") applied
inside the prefill and decode kernels, against the fp64 oracle that applies
them itself.  Called through the C ABI via the Python binding."""
import numpy as np
import pytest
import torch

import gated_delta_rule_49_amd as kda
import synth
from oracle import native
from oracle import reference as R
from kda_testutil import TOL, dev_tensors, err, report, tdtype

pytestmark = pytest.mark.gpu

FLAG_SETS = [kda.PROLOGUE_GATE_SOFTPLUS, kda.PROLOGUE_BETA_SIGMOID, kda.PROLOGUE_QK_L2NORM, kda.PROLOGUE_ALL]


def check_prefill(x, flags, name, boundaries=True, tol=None):
    q, k, v, b, la, init, cu = dev_tensors(x)
    o, S, cs = kda.prefill(q, k, v, b, la, initial_state=init, cu_seqlens=cu, chunk_size=x.chunk_size,
                           chunk_states=True, prologue=flags)
    o_ref, S_ref, cs_ref = native.prefill(x.q, x.k, x.v, x.beta, x.log_alpha, x.cu_seqlens, x.initial_state,
                                          chunk=x.chunk_size, want_chunk_states=True, prologue_flags=flags)
    e = dict(o=err(o, o_ref), S=err(S, S_ref))
    if boundaries:
        e["bounds"] = max((err(cs[i], cs_ref[i]) for i in range(cs.shape[0])), default=0.0)
    report(f"prologue {name} flags={flags} T={x.T} H={x.H} d={x.d_k} C={x.chunk_size} {x.dtype}", **e)
    tol = tol or TOL[x.dtype]
    for key, val in e.items():
        assert val <= tol, f"{key}: {val:.3e} > {tol}"
    return o, S


def test_prefill_fp32_tiny_all_stages():
    """The tiny fp32 shape (T=64, d=16, chunk 16) from pre-activations: 1e-5."""
    x = synth.make_preact(1, 1, 64, 1, 16, 16, "f32", chunk=16)
    check_prefill(x, kda.PROLOGUE_ALL, "f32 tiny")


@pytest.mark.parametrize("flags", FLAG_SETS)
def test_prefill_fp32_each_stage(flags):
    x = synth.make_preact(2 + flags, 2, 70, 2, 32, 32, "f32", chunk=32, state_std=0.3, prologue=flags)
    check_prefill(x, flags, "f32")


@pytest.mark.parametrize("flags", FLAG_SETS)
def test_prefill_bf16_matrix_core_each_stage(flags):
    """d = 128, chunk 64 (matrix-core path), ragged tail, random state."""
    x = synth.make_preact(20 + flags, 1, 300, 4, 128, 128, "bf16", chunk=64, state_std=0.02, prologue=flags)
    check_prefill(x, flags, "bf16 mfma")


def test_prefill_bf16_d64_all_stages():
    x = synth.make_preact(31, 2, 200, 2, 64, 64, "bf16", chunk=32, state_std=0.02)
    check_prefill(x, kda.PROLOGUE_ALL, "bf16 d64")


def test_prefill_bf16_prefill_shape_all_stages():
    """B=1, H=16, T=4096, d=128, chunk 64: the prefill workload's shape, from
    pre-activations."""
    x = synth.make_preact(2, 1, 4096, 16, 128, 128, "bf16", chunk=64)
    check_prefill(x, kda.PROLOGUE_ALL, "bf16 T4096", boundaries=False)


def test_prefill_packed_all_stages():
    x0 = synth.make_packed(4, [100, 0, 257, 64, 33], 4, 128, 128, "bf16", chunk=64)
    x = synth.make_preact(44, 1, x0.T, 4, 128, 128, "bf16", chunk=64)
    x.cu_seqlens = x0.cu_seqlens
    x.initial_state = x0.initial_state
    check_prefill(x, kda.PROLOGUE_ALL, "bf16 packed")


def test_prefill_large_preactivations_stay_finite():
    """Gate pre-activations of +-60 (alpha ~ e^-60 and ~ 1) and beta
    pre-activations of +-40: no overflow, results within the contract."""
    x = synth.make_preact(45, 1, 256, 2, 128, 128, "bf16", chunk=64)
    rng = np.random.default_rng(1)
    x.log_alpha = synth.round_bf16((x.log_alpha * 30).astype(np.float32))
    x.beta = synth.round_bf16(np.where(rng.random(x.beta.shape) < 0.5, -40.0, 40.0).astype(np.float32))
    o, S = check_prefill(x, kda.PROLOGUE_ALL, "bf16 extreme pre-activations")
    assert torch.isfinite(o).all() and torch.isfinite(S).all()


def test_prologue_off_is_bitwise_unchanged():
    """prologue = 0 leaves the kernels' arithmetic as it was: equal to a
    call that never mentions the prologue."""
    x = synth.make_uniform(46, 1, 200, 2, 128, 128, "bf16", chunk=64, state_std=0.02)
    q, k, v, b, la, init, _ = dev_tensors(x)
    o1, S1 = kda.prefill(q, k, v, b, la, initial_state=init)
    o2, S2 = kda.prefill(q, k, v, b, la, initial_state=init, prologue=0)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_fused_equals_pretransformed_fp32():
    """fp32: fusing the stages equals feeding the oracle-transformed inputs
    (rounded to fp32) to the plain kernels, within the fp32 contract."""
    x = synth.make_preact(47, 1, 130, 2, 32, 32, "f32", chunk=32, state_std=0.2)
    q, k, v, b, la, init, _ = dev_tensors(x)
    o1, S1 = kda.prefill(q, k, v, b, la, initial_state=init, chunk_size=32, prologue=kda.PROLOGUE_ALL)
    qt, kt, bt, lat = (torch.from_numpy(a.astype(np.float32)).cuda()
                       for a in R.prologue(x.q, x.k, x.beta, x.log_alpha, R.PRO_QK_L2NORM | 3))
    o2, S2 = kda.prefill(qt, kt, v, bt, lat, initial_state=init, chunk_size=32)
    e = dict(o=err(o1, o2.double().cpu().numpy()), S=err(S1, S2.double().cpu().numpy()))
    report("fused vs pre-transformed f32", **e)
    assert e["o"] <= 1e-5 and e["S"] <= 1e-5


# --------------------------------------------------------------- decode ----
@pytest.mark.parametrize("flags", FLAG_SETS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_each_stage(flags, dtype):
    x = synth.make_preact(60 + flags, 5, 1, 3, 128, 128, dtype, state_std=0.02, prologue=flags)
    dt = tdtype(dtype)
    args = [torch.from_numpy(a).cuda().to(dt) for a in (x.q, x.k, x.v, x.beta, x.log_alpha)]
    S = torch.from_numpy(x.initial_state).cuda()
    o, S1, _ = kda.decode(*args, S, prologue=flags)
    o_ref, S_ref, _ = native.prefill(x.q, x.k, x.v, x.beta, x.log_alpha, initial_state=x.initial_state,
                                     prologue_flags=flags)
    e = dict(o=err(o, o_ref), S=err(S1, S_ref))
    report(f"decode prologue flags={flags} {dtype}", **e)
    assert max(e.values()) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_multi_token_decode_with_prologue(dtype):
    """4 tokens per sequence in one launch from pre-activations."""
    x = synth.make_preact(70, 5, 4, 3, 128, 128, dtype, state_std=0.02)
    dt = tdtype(dtype)
    args = [torch.from_numpy(a).cuda().to(dt) for a in (x.q, x.k, x.v, x.beta, x.log_alpha)]
    S = torch.from_numpy(x.initial_state).cuda()
    o, fin, ts = kda.decode(*args, S, prologue=kda.PROLOGUE_ALL, token_states=True)
    o_ref, S_ref, cs = native.prefill(x.q, x.k, x.v, x.beta, x.log_alpha, initial_state=x.initial_state,
                                      chunk=1, want_chunk_states=True, prologue_flags=7)
    after = np.concatenate([cs.reshape(5, 4, 3, 128, 128)[:, 1:], S_ref[:, None]], axis=1)
    e = dict(o=err(o, o_ref), S=err(fin, S_ref), tokens=err(ts, after))
    report(f"multi-token decode + prologue {dtype}", **e)
    assert max(e.values()) <= TOL[dtype]


def test_sublayer_conv_then_fused_prefill():
    """The stages composed as the sublayer runs them: a width-4 causal
    convolution of q, k and v (with states), then the prefill with every
    prologue stage fused, against the oracle's convolution and recurrence."""
    B, T, H, d, W = 1, 200, 4, 128, 4
    x = synth.make_preact(71, B, T, H, d, d, "bf16", chunk=64, state_std=0.02)
    rng = np.random.default_rng(72)
    ws = [(rng.standard_normal((H * d, W)) / 2).astype(np.float32) for _ in range(3)]
    cs = [rng.standard_normal((1, H * d, W - 1)).astype(np.float32) for _ in range(3)]
    conv_gpu, conv_ref = [], []
    for a, w, s0 in zip((x.q, x.k, x.v), ws, cs):
        y, _ = kda.short_conv(torch.from_numpy(a.reshape(B, T, H * d)).cuda().to(torch.bfloat16),
                              torch.from_numpy(w).cuda(), initial_state=torch.from_numpy(s0).cuda())
        conv_gpu.append(y.reshape(B, T, H, d))
        yr, _ = R.short_conv(a.reshape(B, T, H * d), w, initial_state=s0)
        conv_ref.append(yr.reshape(B, T, H, d))
    yq, yk, yv = conv_gpu
    for g, r in zip(conv_gpu, conv_ref):  # bf16 outputs: within their own rounding
        gv = g.float().cpu().numpy()
        assert np.all(np.abs(gv - r) <= 2.0 ** -8 * np.abs(r) + 1e-6 * np.sqrt(np.mean(r ** 2)))
    b, la = (torch.from_numpy(a).cuda().to(torch.bfloat16) for a in (x.beta, x.log_alpha))
    init = torch.from_numpy(x.initial_state).cuda()
    o, S = kda.prefill(yq, yk, yv, b, la, initial_state=init, prologue=kda.PROLOGUE_ALL)
    # oracle on the GPU's bf16 convolution outputs (rounding at the bf16
    # boundary is shared), from the same pre-activations
    gq, gk, gv = (t.float().cpu().numpy() for t in conv_gpu)
    o_ref, S_ref, _ = native.prefill(gq, gk, gv, x.beta, x.log_alpha, initial_state=x.initial_state,
                                     prologue_flags=7)
    e = dict(o=err(o, o_ref), S=err(S, S_ref))
    report("sublayer conv -> fused prefill", **e)
    assert max(e.values()) <= TOL["bf16"]
