"""Backward-pass parity: the HIP backward (reverse mode, states recomputed
from 16-token checkpoints of the chunked prefill) against the oracle's fp64
reverse-mode gradients, which are pinned by finite differences of the
forward oracle.  Called through the C ABI via the Python binding."""
import numpy as np
import pytest
import torch

import gated_delta_rule_49_amd as kda
import synth
from oracle import reference as R
from kda_testutil import TOL, dev_tensors, err, report

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dbeta", "dlog_alpha", "dS0")


def oracle_grads(x, d_o, d_fin):
    """Per sequence: fp64 reverse-mode gradients, laid out like the inputs."""
    out = {n: None for n in NAMES}
    out["dq"] = np.zeros(x.q.shape)
    out["dk"] = np.zeros(x.k.shape)
    out["dv"] = np.zeros(x.v.shape)
    out["dbeta"] = np.zeros(x.beta.shape)
    out["dlog_alpha"] = np.zeros(x.log_alpha.shape)
    out["dS0"] = np.zeros((x.num_seqs, x.H, x.d_k, x.d_v))
    for n, (b, t0, t1) in enumerate(x.seq_bounds()):
        S0 = None if x.initial_state is None else x.initial_state[n]
        g = R.recurrent_backward(x.q[b, t0:t1], x.k[b, t0:t1], x.v[b, t0:t1], x.beta[b, t0:t1],
                                 x.log_alpha[b, t0:t1], d_o[b, t0:t1], S0,
                                 None if d_fin is None else d_fin[n])
        for name, val in zip(NAMES[:5], g[:5]):
            out[name][b, t0:t1] = val
        out["dS0"][n] = g[5]
    return out


def check(x, name, with_final=True, tol=None, chunk_size=None):
    rng = np.random.default_rng(len(name) + x.T)
    d_o = rng.standard_normal((x.B, x.T, x.H, x.d_v)).astype(np.float32)
    d_fin = rng.standard_normal((x.num_seqs, x.H, x.d_k, x.d_v)).astype(np.float32) if with_final else None
    q, k, v, b, la, init, cu = dev_tensors(x)
    got = kda.backward(q, k, v, b, la, torch.from_numpy(d_o).cuda(), initial_state=init,
                       d_final_state=None if d_fin is None else torch.from_numpy(d_fin).cuda(), cu_seqlens=cu,
                       chunk_size=chunk_size)
    ref = oracle_grads(x, d_o, d_fin)
    e = {n: err(g, ref[n]) for n, g in zip(NAMES, got)}
    report(f"backward {name} T={x.T} H={x.H} d={x.d_k}x{x.d_v} {x.dtype}", **e)
    tol = tol or TOL[x.dtype]
    for n, val in e.items():
        assert val <= tol, f"{n}: {val:.3e} > {tol}"


@pytest.mark.parametrize("T", [1, 15, 16, 37])
def test_fp32_lengths(T):
    x = synth.make_uniform(400 + T, 2, T, 2, 32, 32, "f32", chunk=16, state_std=0.3)
    check(x, "f32")


@pytest.mark.parametrize("dk,dv", [(16, 16), (64, 32), (128, 128)])
def test_fp32_head_sizes(dk, dv):
    x = synth.make_uniform(410 + dk + dv, 1, 50, 2, dk, dv, "f32", chunk=16, state_std=0.2)
    check(x, "f32 sizes")


def test_fp32_without_final_gradient_and_state():
    x = synth.make_uniform(420, 1, 40, 1, 32, 32, "f32", chunk=16)
    check(x, "f32 zero state", with_final=False)


def test_fp32_slow_decay():
    x = synth.slow_decay(421, 1, 90, 2, 32, 32, "f32", chunk=16)
    check(x, "f32 slow decay")


def test_fp32_packed():
    x = synth.make_packed(422, [17, 0, 33, 1], 2, 32, 32, "f32", chunk=16)
    check(x, "f32 packed")


def test_bf16_d128():
    x = synth.make_uniform(430, 1, 300, 2, 128, 128, "bf16", chunk=16, state_std=0.02)
    check(x, "bf16")


def test_bf16_packed_d128():
    x = synth.make_packed(431, [100, 3, 0, 200], 2, 128, 128, "bf16", chunk=16)
    check(x, "bf16 packed")


def test_bf16_prefill_shape_heads_sampled():
    """T=1024 slice of the prefill workload's shape (H=16, d=128), all heads
    on the GPU, two heads checked against the oracle."""
    x = synth.make_uniform(2, 1, 1024, 16, 128, 128, "bf16", chunk=16)
    rng = np.random.default_rng(3)
    d_o = rng.standard_normal((1, 1024, 16, 128)).astype(np.float32)
    q, k, v, b, la, _, _ = dev_tensors(x)
    got = kda.backward(q, k, v, b, la, torch.from_numpy(d_o).cuda())
    worst = {}
    for h in (0, 15):
        g = R.recurrent_backward(x.q[0, :, h:h + 1], x.k[0, :, h:h + 1], x.v[0, :, h:h + 1],
                                 x.beta[0, :, h:h + 1], x.log_alpha[0, :, h:h + 1], d_o[0, :, h:h + 1])
        for n, gpu, ref in zip(NAMES, got, g):
            sl = gpu[:, h:h + 1] if n == "dS0" else gpu[0, :, h:h + 1]
            worst[n] = max(worst.get(n, 0.0), err(sl, ref))
    report("backward T=1024 H=16 d=128 bf16 heads 0,15", **worst)
    assert max(worst.values()) <= TOL["bf16"]


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_bf16_chunk_sizes_ragged(chunk):
    """The chunked backward at every chunk size, ragged tail, random state."""
    x = synth.make_uniform(440 + chunk, 2, 150, 2, 128, 128, "bf16", chunk=chunk, state_std=0.02)
    check(x, f"bf16 chunked C={chunk}", chunk_size=chunk)


@pytest.mark.parametrize("dk,dv", [(64, 64), (16, 32), (32, 128)])
def test_bf16_head_sizes(dk, dv):
    x = synth.make_uniform(450 + dk + dv, 1, 100, 2, dk, dv, "bf16", chunk=64, state_std=0.05)
    check(x, "bf16 chunked sizes")


def test_bf16_slow_decay():
    x = synth.slow_decay(460, 1, 300, 2, 128, 128, "bf16", chunk=64)
    check(x, "bf16 chunked slow decay")


def test_bf16_extreme_gates():
    x = synth.make_long(461, 512, 2, 128, 128, "bf16")
    check(x, "bf16 chunked extreme gates")


@pytest.mark.parametrize("gate_mean", [2.5, 4.0, 10.0])
def test_bf16_strong_decay(gate_mean):
    """log alpha ~ -softplus(N(gate_mean, 1)) on every token: a 16-token block
    decays by ~40, ~64 and ~160 nats, so the pair sums of the diagonal blocks
    take the split around the block's midpoint, a mix, and the pair-by-pair
    sum."""
    x = synth.make_uniform(470 + int(gate_mean), 1, 200, 2, 128, 128, "bf16", chunk=64, state_std=0.3,
                           gate_mean=gate_mean)
    check(x, f"bf16 chunked strong decay {gate_mean}")


def test_bf16_unaligned_inputs_match_aligned():
    """q, k, v, beta and log alpha passed to the backward as views that start
    one element into their allocation (2-byte aligned, not 16-byte aligned):
    the chunk prep and gradient kernels take their scalar staging paths and
    must give the same gradients, bit for bit, as with aligned tensors."""
    x = synth.make_uniform(480, 1, 130, 2, 128, 128, "bf16", chunk=64, state_std=0.05)
    q, k, v, b, la, init, cu = dev_tensors(x)
    d_o = torch.from_numpy(np.random.default_rng(7).standard_normal((x.B, x.T, x.H, x.d_v)).astype(np.float32)).cuda()

    def shifted(t):
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
        view = buf[1:].view(t.shape)
        view.copy_(t)
        assert view.data_ptr() % 16 != 0
        return view

    # the chunk-entry states from the prefill on the aligned inputs (the
    # prefill's matrix-core path takes 16-byte aligned inputs only)
    _, _, ck = kda.prefill(q, k, v, b, la, initial_state=init, output_final_state=False, chunk_size=64,
                           chunk_states=True)
    ref = kda.backward(q, k, v, b, la, d_o, initial_state=init, checkpoints=ck, chunk_size=64)
    got = kda.backward(*(shifted(t) for t in (q, k, v, b, la)), d_o, initial_state=init, checkpoints=ck,
                       chunk_size=64)
    for n, a, c in zip(NAMES, ref, got):
        assert torch.equal(a, c), n
