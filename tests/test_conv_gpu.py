"""Short causal convolution parity (Module 04 — KDA II, §3 "The sublayer is
bigger than the recurrence"; rolling conv state: Module 11, §2, row
"Serving state"): the HIP kernel against the fp64 oracle, prefill and
decode use, packed documents with empty and short ones, the final state.
Called through the C ABI via the Python binding."""
import numpy as np
import pytest
import torch

import gated_delta_rule_49_amd as kda
import synth
from oracle import reference as R
from kda_testutil import TOL, err, report

pytestmark = pytest.mark.gpu


def draw(seed, B, T, C, W, dtype, state=True, lens=None):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, T, C)).astype(np.float32)
    if dtype == "bf16":
        x = synth.round_bf16(x)
    w = (rng.standard_normal((C, W)) / np.sqrt(W)).astype(np.float32)
    bias = rng.standard_normal(C).astype(np.float32) * 0.1
    N = B if lens is None else len(lens)
    s0 = rng.standard_normal((N, C, W - 1)).astype(np.float32) if state else None
    return x, w, bias, s0


def tdt(dtype):
    return torch.float32 if dtype == "f32" else torch.bfloat16


def run(x, w, bias, s0, dtype, out_dtype, cu=None, silu=False):
    dev = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    y, fin = kda.short_conv(dev(x).to(tdt(dtype)), dev(w), initial_state=dev(s0), bias=dev(bias),
                            cu_seqlens=None if cu is None else dev(cu.astype(np.int32)), silu=silu,
                            out_dtype=out_dtype)
    return y, fin


def check(y, fin, y_ref, fin_ref, out_dtype, name):
    yv = y.float().cpu().numpy()
    if out_dtype == torch.float32:  # fp32 arithmetic: the fp32 contract
        e = err(y, y_ref)
        ok = e <= TOL["f32"]
    else:  # the bf16 rounding of y itself, elementwise
        e = float(np.max(np.abs(yv - y_ref) / (np.abs(y_ref) + 1e-30 + 1e-6 * np.sqrt(np.mean(y_ref ** 2)))))
        ok = np.all(np.abs(yv - y_ref) <= 2.0 ** -8 * np.abs(y_ref) + 1e-6 * np.sqrt(np.mean(y_ref ** 2)))
    report(name, y=e)
    assert ok, f"{name}: {e:.3e}"
    # the final state is a copy of inputs: exact
    np.testing.assert_array_equal(fin.cpu().numpy(), fin_ref.astype(np.float32))


@pytest.mark.parametrize("W", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("dtype,out", [("f32", torch.float32), ("bf16", torch.float32), ("bf16", torch.bfloat16)])
def test_widths_and_dtypes(W, dtype, out):
    x, w, bias, s0 = draw(W, 2, 37, 64, W, dtype)
    y, fin = run(x, w, bias, s0, dtype, out)
    y_ref, fin_ref = R.short_conv(x, w, initial_state=s0, bias=bias)
    check(y, fin, y_ref, fin_ref, out, f"conv W={W} {dtype}->{out}")


@pytest.mark.parametrize("T", [0, 1, 2, 15, 16, 17, 100])
def test_lengths_and_tiles(T):
    x, w, bias, s0 = draw(100 + T, 3, T, 24, 4, "bf16")
    y, fin = run(x, w, None, s0, "bf16", torch.float32)
    y_ref, fin_ref = R.short_conv(x, w, initial_state=s0)
    if T:
        check(y, fin, y_ref, fin_ref, torch.float32, f"conv T={T}")
    else:
        np.testing.assert_array_equal(fin.cpu().numpy(), s0)


def test_no_state_bias_silu():
    x, w, bias, _ = draw(7, 2, 50, 128, 4, "bf16", state=False)
    y, fin = run(x, w, bias, None, "bf16", torch.float32, silu=True)
    y_ref, fin_ref = R.short_conv(x, w, bias=bias, silu=True)
    check(y, fin, y_ref, fin_ref, torch.float32, "conv silu")


@pytest.mark.parametrize("lens", [[5, 0, 1, 2, 40, 16, 3], [100, 0, 3, 64, 1, 200, 2]],
                         ids=["short-docs", "long-docs"])
def test_packed_documents(lens):
    """Short documents (one token per thread) and long ones (16-token tiles
    that cross document starts)."""
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    x, w, bias, s0 = draw(8, 1, int(cu[-1]), 96, 4, "bf16", lens=lens)
    y, fin = run(x, w, bias, s0, "bf16", torch.float32, cu=cu)
    y_ref, fin_ref = R.short_conv(x, w, cu_seqlens=cu, initial_state=s0, bias=bias)
    check(y, fin, y_ref, fin_ref, torch.float32, "conv packed")


@pytest.mark.parametrize("W", [2, 4, 8])
def test_decode_steps_equal_one_pass_bitwise(W):
    """Rolling the state in place over single-token calls (the one-kernel
    path for rows of a few tokens) equals one call over all the tokens (the
    tiled path), bit for bit: the same arithmetic in the same order."""
    x, w, bias, s0 = draw(9 + W, 4, 40, 64, W, "bf16")
    xd = torch.from_numpy(x).cuda().to(torch.bfloat16)
    wd, bd = torch.from_numpy(w).cuda(), torch.from_numpy(bias).cuda()
    y1, fin1 = kda.short_conv(xd, wd, initial_state=torch.from_numpy(s0).cuda(), bias=bd, out_dtype=torch.float32)
    st = torch.from_numpy(s0).cuda()
    ys = [kda.short_conv(xd[:, t:t + 1].contiguous(), wd, initial_state=st, bias=bd, update_state=True,
                         out_dtype=torch.float32)[0] for t in range(40)]
    assert torch.equal(torch.cat(ys, 1), y1) and torch.equal(st, fin1)
    y_ref, fin_ref = R.short_conv(x, w, initial_state=s0, bias=bias)
    check(y1, fin1, y_ref, fin_ref, torch.float32, f"conv W={W} decode rolls vs one pass")


def test_prefill_shape_sampled():
    """The bench shape, x = q of the long workload flattened: [1, 131072,
    4096] bf16, W = 4: rows sampled across the sequence against the oracle
    on a window around them."""
    T, C, W = 131072, 4096, 4
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    x = torch.randn((1, T, C), generator=g, device="cuda").to(torch.bfloat16)
    rng = np.random.default_rng(11)
    w = torch.from_numpy((rng.standard_normal((C, W)) / 2).astype(np.float32)).cuda()
    y, fin = kda.short_conv(x, w, out_dtype=torch.float32)
    worst = 0.0
    for t in [0, 1, 2, 3, 15, 16, 4097, 65535, T - 1]:
        lo = max(0, t - W + 1)
        xw = x[:, lo:t + 1].float().cpu().numpy()
        yr, _ = R.short_conv(xw, w.cpu().numpy())
        worst = max(worst, err(y[:, t:t + 1], yr[:, -1:]))
    report("conv T=131072 C=4096 sampled", y=worst)
    assert worst <= TOL["f32"]
    np.testing.assert_array_equal(fin[0].cpu().numpy(), x[0, T - W + 1:].float().cpu().numpy().T)
