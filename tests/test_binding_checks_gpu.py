"""The binding rejects caller-supplied buffers that the kernels would overrun
or misread, before anything is launched: outputs of the wrong shape or
dtype, a chunk-checkpoint buffer sized for another chunk size, conflicting
output dtypes.  A bf16 ``o`` sets the output dtype by itself."""
import pytest
import torch

import gated_delta_rule_49_amd as kda
import synth
from kda_testutil import dev_tensors

pytestmark = pytest.mark.gpu


def _inputs(T=70, H=2, d=128, dtype="bf16", chunk=64):
    x = synth.make_uniform(61, 1, T, H, d, d, dtype, chunk=chunk, state_std=0.1)
    return x, dev_tensors(x)


def test_prefill_rejects_wrong_output_buffers():
    x, (q, k, v, b, la, init, _) = _inputs()
    B, T, H, d = q.shape
    with pytest.raises(ValueError):
        kda.prefill(q, k, v, b, la, o=torch.empty((B, T - 1, H, d), device="cuda"))
    with pytest.raises(TypeError):
        kda.prefill(q, k, v, b, la, o=torch.empty((B, T, H, d), dtype=torch.float16, device="cuda"))
    with pytest.raises(TypeError):
        kda.prefill(q, k, v, b, la, o=torch.empty((B, T, H, d), dtype=torch.bfloat16, device="cuda"),
                    out_dtype=torch.float32)
    with pytest.raises(ValueError):
        kda.prefill(q, k, v, b, la, final_state=torch.empty((1, H, d, d - 1), device="cuda"))
    with pytest.raises(TypeError):
        kda.prefill(q, k, v, b, la, final_state=torch.empty((1, H, d, d), dtype=torch.bfloat16, device="cuda"))


def test_prefill_output_dtype_follows_a_given_o():
    """A bf16 ``o`` given without out_dtype gets bf16 stores (not fp32 stores
    that would run past its end): the result is the default call's fp32
    output rounded to bf16."""
    x, (q, k, v, b, la, init, _) = _inputs()
    o32, S32 = kda.prefill(q, k, v, b, la, initial_state=init)
    ob = torch.full(o32.shape, 7.0, dtype=torch.bfloat16, device="cuda")
    o, S = kda.prefill(q, k, v, b, la, initial_state=init, o=ob)
    assert o is ob and o.dtype == torch.bfloat16
    assert torch.equal(S, S32)
    # the same fp32 accumulators, stored rounded to nearest even
    assert torch.equal(o, o32.to(torch.bfloat16))


def test_decode_and_conv_reject_wrong_buffers():
    x = synth.decode_workload(B=3, H=2, dk=64, dv=64, steps=2, seed=62, dtype="bf16", state_std=0.1)
    S = torch.from_numpy(x.initial_state).cuda()
    args = [torch.from_numpy(a[0]).cuda().to(torch.bfloat16) for a in (x.q, x.k, x.v, x.beta, x.log_alpha)]
    with pytest.raises(ValueError):
        kda.decode_step(*args, S, o=torch.empty((3, 2, 63), device="cuda"))
    margs = [a[:, None] for a in args]
    with pytest.raises(ValueError):
        kda.decode(*margs, S, o=torch.empty((3, 2, 2, 64), device="cuda"))
    with pytest.raises(ValueError):
        kda.decode(*margs, S, update_state=False, final_state=torch.empty((3, 2, 64, 32), device="cuda"))
    xc = torch.randn((1, 40, 64), device="cuda").to(torch.bfloat16)
    w = torch.randn((64, 4), device="cuda")
    with pytest.raises(ValueError):
        kda.short_conv(xc, w, y=torch.empty((1, 39, 64), device="cuda", dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        kda.short_conv(xc, w, final_state=torch.empty((1, 64, 2), device="cuda"))


def test_backward_rejects_checkpoints_of_another_chunk_size():
    """Checkpoints written at chunk 16 have 4x as many chunks as the chunk-64
    backward reads through its own chunk table; a buffer from chunk 64 used
    with chunk 16 would be read past its end: it is rejected, and the
    matching chunk size is accepted."""
    x, (q, k, v, b, la, init, _) = _inputs(T=200, H=2, d=64)
    d_o = torch.randn((1, 200, 2, 64), device="cuda")
    _, _, ck64 = kda.prefill(q, k, v, b, la, initial_state=init, chunk_size=64, chunk_states=True)
    with pytest.raises(ValueError):
        kda.backward(q, k, v, b, la, d_o, initial_state=init, checkpoints=ck64, chunk_size=16)
    # the matching chunk size is accepted
    g = kda.backward(q, k, v, b, la, d_o, initial_state=init, checkpoints=ck64, chunk_size=64)
    assert all(bool(torch.isfinite(t).all()) for t in g)
