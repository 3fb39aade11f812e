"""The allocation-free prefill (kda_prefill_chunked_noalloc, through the C
ABI) against the workspace entry point (kda_prefill_chunked) on the same
inputs: two calls in a row on the shared per-GPU scratch, the second smaller
than the first (so the second finds the first call's contents there), then a
third on the fp32 path and a fourth on its overlapped launch; outputs and final states must be identical (same
kernels, same scratch layout) and within the contract of the fp64 oracle.
A call beyond the scratch is refused before it writes anything."""
import pytest
import torch

import gated_delta_rule_49_amd as kda
import synth
from oracle import native
from kda_testutil import TOL, dev_tensors, err, report

pytestmark = pytest.mark.gpu


def _both(x, chunk):
    q, k, v, b, la, init, cu = dev_tensors(x)
    B, T, H, _ = q.shape
    N = B if cu is None else cu.numel() - 1
    o_ref, S_ref = kda.prefill(q, k, v, b, la, initial_state=init, cu_seqlens=cu, chunk_size=chunk)
    o = torch.full((B, T, H, x.d_v), float("nan"), dtype=torch.float32, device="cuda")
    S = torch.full((N, H, x.d_k, x.d_v), float("nan"), dtype=torch.float32, device="cuda")
    kda.prefill_noalloc(q, k, v, b, la, o, final_state=S, initial_state=init, cu_seqlens=cu, chunk_size=chunk)
    torch.cuda.synchronize()
    return o, S, o_ref, S_ref


def _oracle_check(x, o, S, name):
    o_or, S_or, _ = native.prefill(x.q, x.k, x.v, x.beta, x.log_alpha, x.cu_seqlens, x.initial_state)
    e = dict(o=err(o, o_or), S=err(S, S_or))
    report(name, **e)
    assert max(e.values()) <= TOL[x.dtype]


def test_noalloc_matches_the_workspace_entry_point_on_consecutive_calls():
    # 1: the T=4096, H=16 prefill workload (about half of the scratch)
    x1 = synth.workload(2)
    o, S, o_ref, S_ref = _both(x1, 64)
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
    _oracle_check(x1, o, S, "noalloc T=4096 H=16")
    # 2: smaller, packed, with empty and one-token documents and a state
    x2 = synth.make_packed(71, [70, 0, 1, 64, 129, 5], 3, 128, 128, "bf16", chunk=64)
    o, S, o_ref, S_ref = _both(x2, 64)
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
    _oracle_check(x2, o, S, "noalloc packed (second call, smaller)")
    # 3: fp32 inputs (the fp32 matrix-core path's blocks in the same scratch)
    x3 = synth.make_uniform(72, 2, 150, 2, 64, 64, "f32", chunk=32, state_std=0.2)
    o, S, o_ref, S_ref = _both(x3, 32)
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
    _oracle_check(x3, o, S, "noalloc fp32 (third call)")
    # 4: fp32 inputs, d = 128, one sequence with 4 heads: the overlapped fp32
    #    launch, whose flags live in the same scratch after the first three
    #    calls' contents (cleared by the call's own chunk-table kernel)
    x4 = synth.make_uniform(74, 1, 1000, 4, 128, 128, "f32", chunk=64, state_std=0.1)
    o, S, o_ref, S_ref = _both(x4, 64)
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
    _oracle_check(x4, o, S, "noalloc fp32 overlapped launch (fourth call)")


def test_noalloc_refuses_a_call_beyond_its_scratch():
    x = synth.make_uniform(73, 1, 16, 1, 128, 128, "bf16", chunk=64)
    q, k, v, b, la, _, _ = dev_tensors(x)
    # a long row whose chunk blocks exceed the fixed scratch (the first token
    # repeated): the host-side size check fails before any launch
    T = 8192
    H = 32
    big = lambda t: t[:, :1].expand(1, T, H, t.shape[-1]).contiguous()  # noqa: E731
    qb, kb, vb, lab = big(q), big(k), big(v), big(la)
    bb = b[:, :1].expand(1, T, H).contiguous()
    assert kda.workspace_bytes(qb, kb, vb, bb, lab) > kda.NOALLOC_SCRATCH_BYTES
    o = torch.full((1, T, H, 128), 7.0, device="cuda")
    with pytest.raises(kda.KDAError) as ei:
        kda.prefill_noalloc(qb, kb, vb, bb, lab, o)
    assert ei.value.status == 7
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())


def test_noalloc_prefill_replays_from_a_captured_graph():
    """The use the allocation-free entry point is for: captured once in a
    HIP graph (torch.cuda.graph; one eager call before the capture looks up
    the scratch address), the graph replays to the eager result every time,
    with other library calls on the same scratch and synchronisations
    between the replays."""
    x = synth.workload(2)   # the T=4096, H=16 prefill workload
    q, k, v, b, la, _, _ = dev_tensors(x)
    B, T, H, _ = q.shape
    o_ref = torch.empty((B, T, H, x.d_v), dtype=torch.float32, device="cuda")
    S_ref = torch.empty((B, H, x.d_k, x.d_v), dtype=torch.float32, device="cuda")
    kda.prefill_noalloc(q, k, v, b, la, o_ref, final_state=S_ref)
    torch.cuda.synchronize()
    o, S = torch.empty_like(o_ref), torch.empty_like(S_ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        kda.prefill_noalloc(q, k, v, b, la, o, final_state=S)
    y = synth.make_uniform(74, 1, 300, 2, 128, 128, "bf16", chunk=64, state_std=0.1)
    yq, yk, yv, yb, yla, yinit, _ = dev_tensors(y)
    yo = torch.empty((1, 300, 2, 128), dtype=torch.float32, device="cuda")
    for rep in range(4):
        o.fill_(float("nan"))
        S.fill_(float("nan"))
        kda.prefill_noalloc(yq, yk, yv, yb, yla, yo, initial_state=yinit)   # other contents in the scratch
        kda.prefill(yq, yk, yv, yb, yla, initial_state=yinit)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(S, S_ref), f"replay {rep}"
