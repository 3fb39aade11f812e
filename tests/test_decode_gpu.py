"""Decode-step parity: the fused HIP decode kernel against the fp64 oracle's
own token-by-token trajectory, checked after every step (outputs and state).
Called through the C ABI via the Python binding."""
import numpy as np
import pytest
import torch

import gated_delta_rule_49_amd as kda
import synth
from oracle import native
from kda_testutil import TOL, err, report, tdtype

pytestmark = pytest.mark.gpu


def state_err(S_gpu, S_ref):
    """err(S) = max|S - S_ref| / RMS(S_ref) over the whole state, in fp64,
    in blocks of rows so that the temporaries stay small."""
    x = S_gpu.detach().cpu().numpy().reshape(-1, S_gpu.shape[-1])
    r = S_ref.reshape(-1, S_ref.shape[-1])
    d, ss = 0.0, 0.0
    for i in range(0, x.shape[0], 1 << 16):
        xs, rs = x[i:i + (1 << 16)], r[i:i + (1 << 16)]
        d = max(d, float(np.max(np.abs(xs - rs))))
        ss += float(np.einsum("ij,ij->", rs, rs))
    rms = np.sqrt(ss / r.size)
    return d / rms if rms > 0 else (0.0 if d == 0 else float("inf"))


def run_case(x):
    """Every step: the GPU decode step against the oracle's own fp64
    trajectory (never re-synchronised to the GPU state), outputs and the
    full state compared after every step."""
    steps, B, H, dk = x.q.shape
    dt = tdtype(x.dtype)
    S = torch.from_numpy(x.initial_state).cuda()
    S_ref = x.initial_state.astype(np.float64)
    worst_o = worst_s = 0.0
    for s in range(steps):
        args = [torch.from_numpy(a[s]).cuda().to(dt) for a in (x.q, x.k, x.v, x.beta, x.log_alpha)]
        o = kda.decode_step(*args, S)
        o_ref, S_ref, _ = native.prefill(x.q[s][None], x.k[s][None], x.v[s][None], x.beta[s][None],
                                         x.log_alpha[s][None], cu_seqlens=np.arange(B + 1),
                                         initial_state=S_ref)
        eo = err(o, o_ref[0])
        es = state_err(S, S_ref)
        worst_o, worst_s = max(worst_o, eo), max(worst_s, es)
        assert eo <= TOL[x.dtype], f"step {s}: err(o) = {eo:.3e}"
        assert es <= TOL[x.dtype], f"step {s}: err(S) = {es:.3e}"
    return worst_o, worst_s


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 32), (128, 128), (128, 16), (16, 128)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_small(dk, dv, dtype):
    x = synth.decode_workload(B=3, H=2, dk=dk, dv=dv, steps=6, seed=30 + dk + dv, dtype=dtype,
                              state_std=0.5)
    eo, es = run_case(x)
    report(f"decode B=3 H=2 d={dk}x{dv} {dtype}", o=eo, S=es)


@pytest.mark.parametrize("B,H,dk,dv,dtype", [(100, 16, 128, 128, "bf16"), (275, 4, 64, 32, "f32")])
def test_decode_persistent_walk_with_uneven_share(B, H, dk, dv, dtype):
    # B*H states over the persistent single-token grid (512 workgroups): with
    # 1600 and 1100 states some workgroups update one state more than others,
    # so both halves of the prefetch walk end a workgroup's share
    x = synth.decode_workload(B=B, H=H, dk=dk, dv=dv, steps=3, seed=47 + B, dtype=dtype, state_std=0.02)
    eo, es = run_case(x)
    report(f"decode B={B} H={H} d={dk}x{dv} {dtype}", o=eo, S=es)


def test_decode_bf16_output():
    x = synth.decode_workload(B=4, H=3, steps=1, seed=41, state_std=0.3)
    S = torch.from_numpy(x.initial_state).cuda()
    args = [torch.from_numpy(a[0]).cuda().to(torch.bfloat16) for a in (x.q, x.k, x.v, x.beta, x.log_alpha)]
    o = kda.decode_step(*args, S, out_dtype=torch.bfloat16)
    assert o.dtype == torch.bfloat16
    o_ref, _, _ = native.prefill(x.q[0][None], x.k[0][None], x.v[0][None], x.beta[0][None],
                                 x.log_alpha[0][None], cu_seqlens=np.arange(5),
                                 initial_state=x.initial_state)
    # elementwise: contract tolerance plus the bf16 rounding of o itself
    d = np.abs(o.float().cpu().numpy() - o_ref[0])
    rms = np.sqrt(np.mean(o_ref[0] ** 2))
    assert np.all(d <= 2e-2 * rms + 2.0 ** -8 * np.abs(o_ref[0]))


def test_decode_workload_b256_h32_64_steps():
    """B=256 sequences, H=32, d=128, 64 steps of fresh bf16 inputs from an
    N(0, 0.02^2) fp32 state: the outputs and the full 512 MiB state checked
    against the oracle's trajectory after every one of the 64 steps."""
    x = synth.decode_workload()
    eo, es = run_case(x)
    report("decode B=256 H=32 d=128 64 steps (full state every step)", o=eo, S=es)
