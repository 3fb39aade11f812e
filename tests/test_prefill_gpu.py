"""Chunked-prefill parity against the fp64 recurrent oracle (Module 04 —
KDA II, §4 "The correctness invariant": outputs, final state and the state at
every chunk boundary; chunk sizes that do and do not divide the length).
Called through the C ABI via the Python binding."""
import numpy as np
import pytest
import torch

import gated_delta_rule_49_amd as kda
import synth
from oracle import native
from kda_testutil import TOL, dev_tensors, err, report

pytestmark = pytest.mark.gpu


def check(x, chunk=None, name="", tol=None, boundaries=True):
    chunk = chunk or x.chunk_size
    q, k, v, b, la, init, cu = dev_tensors(x)
    res = kda.prefill(q, k, v, b, la, initial_state=init, cu_seqlens=cu, chunk_size=chunk,
                      chunk_states=boundaries, check_seqlens=cu is not None)
    o, S, cs = res if boundaries else (*res, None)
    o_ref, S_ref, cs_ref = native.prefill(x.q, x.k, x.v, x.beta, x.log_alpha, x.cu_seqlens,
                                          x.initial_state, chunk=chunk, want_chunk_states=boundaries)
    tol = tol or TOL[x.dtype]
    e = dict(o=err(o, o_ref), S=err(S, S_ref))
    if boundaries:
        assert cs.shape == cs_ref.shape
        e["bounds"] = max((err(cs[i], cs_ref[i]) for i in range(cs.shape[0])), default=0.0)
    report(f"{name} T={x.T} H={x.H} d={x.d_k}x{x.d_v} C={chunk} {x.dtype}", **e)
    for key, val in e.items():
        assert val <= tol, f"{key}: {val:.3e} > {tol}"
    return o, S


def test_tiny_fp32_workload():
    """B=1 H=1 T=64 d=16 fp32, chunk 16, zero state: 1e-5."""
    check(synth.workload(1), name="tiny")


@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("T", [1, 37, 70, 128])
def test_fp32_chunks_and_ragged_tails(chunk, T):
    x = synth.make_uniform(100 + T, 2, T, 2, 32, 16, "f32", chunk=chunk, state_std=0.3)
    check(x, name="f32")


@pytest.mark.parametrize("dk,dv", [(16, 16), (64, 128), (128, 64), (128, 128)])
def test_fp32_head_sizes(dk, dv):
    x = synth.make_uniform(200 + dk + dv, 1, 100, 2, dk, dv, "f32", chunk=32, state_std=0.2)
    check(x, name="f32 sizes")


def test_fp32_slow_decay_boundaries():
    """alpha ~ 0.99: the carried state dominates, exposing boundary mistakes."""
    x = synth.slow_decay(7, 1, 150, 2, 32, 32, "f32", chunk=32)
    check(x, name="f32 slow decay")


def test_fp32_packed():
    x = synth.make_packed(8, [17, 0, 64, 1, 45], 2, 32, 32, "f32", chunk=16)
    check(x, name="f32 packed")


@pytest.mark.parametrize("dk,dv", [(16, 32), (32, 32)])
def test_bf16_small_heads_use_fp32_path(dk, dv):
    x = synth.make_uniform(300 + dk, 1, 90, 2, dk, dv, "bf16", chunk=16, state_std=0.2)
    check(x, name="bf16 small heads")


@pytest.mark.parametrize("dk,dv,chunk", [(16, 32, 32), (32, 32, 64), (128, 64, 64), (64, 16, 32)])
def test_bf16_small_or_unequal_heads_on_fp32_matrix_cores(dk, dv, chunk):
    """bf16 inputs with head sizes the bf16 matrix-core path does not take,
    at chunk 32 / 64: the chunk prep plus the fp32 matrix-core scan."""
    x = synth.make_uniform(310 + dk + dv, 2, 150, 2, dk, dv, "bf16", chunk=chunk, state_std=0.2)
    check(x, name="bf16 heads on fp32 matrix cores")


@pytest.mark.parametrize("chunk", [32, 64])
def test_fp32_packed_with_empty_and_tiny_documents(chunk):
    x = synth.make_packed(28, [70, 0, 1, 64, 129, 5], 3, 128, 128, "f32", chunk=chunk)
    check(x, name="f32 packed")


def test_fp32_bf16_output_and_extreme_gates():
    """fp32 inputs with 10 % extreme-gate tokens (log alpha in [-20, -10],
    beta in {1e-4, 1 - 1e-4}) and a bf16 output (checked elementwise against
    the contract plus bf16's own rounding)."""
    x = synth.make_long(29, 300, 2, 128, 128, "f32", chunk=64)
    q, k, v, b, la, init, _ = dev_tensors(x)
    o, S = kda.prefill(q, k, v, b, la, initial_state=init, chunk_size=64, out_dtype=torch.bfloat16)
    o_ref, S_ref, _ = native.prefill(x.q, x.k, x.v, x.beta, x.log_alpha, None, x.initial_state)
    d = np.abs(o.float().cpu().numpy() - o_ref)
    rms = np.sqrt(np.mean(o_ref ** 2))
    report("f32 extreme gates, bf16 output", o_max=float(d.max() / rms), S=err(S, S_ref))
    assert np.all(d <= 1e-5 * rms + 2.0 ** -8 * np.abs(o_ref))
    assert err(S, S_ref) <= 1e-5


@pytest.mark.parametrize("chunk", [16, 64])
def test_fp32_long_sequence_on_fp32_matrix_cores(chunk):
    """T=16384, H=4, d=128 fp32: 1024 or 256 chunks carried in sequence on
    the fp32 matrix-core path, every output and the final state within
    1e-5."""
    x = synth.make_uniform(34, 1, 16384, 4, 128, 128, "f32", chunk=chunk, state_std=0.1)
    q, k, v, b, la, init, _ = dev_tensors(x)
    assert kda.workspace_bytes(q, k, v, b, la, chunk_size=chunk) > (1 << 26)   # chunk blocks: this path
    o, S = kda.prefill(q, k, v, b, la, initial_state=init, chunk_size=chunk)
    o_ref, S_ref, _ = native.prefill(x.q, x.k, x.v, x.beta, x.log_alpha, None, x.initial_state)
    e = dict(o=err(o, o_ref), S=err(S, S_ref))
    report(f"f32 long T=16384 H=4 d=128 C={chunk} (fp32 matrix cores)", **e)
    assert max(e.values()) <= TOL["f32"]


@pytest.mark.parametrize("T,H,d", [(32768, 16, 128), (16384, 64, 16)])
def test_fp32_chunk16_beyond_the_block_budget_uses_the_vector_path(T, H, d):
    """A chunk-16 fp32 call whose 64-row chunk blocks would exceed 4 GiB
    (T/16 x H blocks of 209 KB at d = 128, 69 KB at d = 16) runs on the
    vector-ALU kernel: the workspace query shows no blocks, and the result
    meets the contract on every head."""
    x = synth.make_uniform(33, 1, T, H, d, d, "f32", chunk=16, state_std=0.1)
    q, k, v, b, la, init, _ = dev_tensors(x)
    assert kda.workspace_bytes(q, k, v, b, la, chunk_size=16) < (1 << 20)   # chunk table only
    assert kda.workspace_bytes(q, k, v, b, la, chunk_size=64) > (1 << 30)   # 64-token blocks
    o, S = kda.prefill(q, k, v, b, la, initial_state=init, chunk_size=16)
    o_ref, S_ref, _ = native.prefill(x.q, x.k, x.v, x.beta, x.log_alpha, None, x.initial_state)
    e = dict(o=err(o, o_ref), S=err(S, S_ref))
    report(f"f32 chunk 16, T={T} H={H} d={d} (vector-ALU path)", **e)
    assert max(e.values()) <= TOL["f32"]


def test_empty_sequences_keep_state():
    x = synth.make_packed(9, [0, 5, 0], 1, 16, 16, "f32", chunk=16)
    o, S = check(x, name="empty docs")
    assert torch.equal(S[0].cpu(), torch.from_numpy(x.initial_state[0]))
    assert torch.equal(S[2].cpu(), torch.from_numpy(x.initial_state[2]))


def test_malformed_seqlens_write_nothing():
    """Decreasing offsets: the host copy is rejected before launch; without a
    host copy the device check rejects them and no output is written."""
    import ctypes
    x = synth.make_packed(10, [20, 30], 1, 16, 16, "f32", chunk=16)
    q, k, v, b, la, init, _ = dev_tensors(x)
    cu = torch.tensor([0, 40, 30], dtype=torch.int32, device="cuda")
    with pytest.raises(kda.KDAError) as ei:
        kda.prefill(q, k, v, b, la, initial_state=init, cu_seqlens=cu, chunk_size=16,
                    check_seqlens=True)
    assert ei.value.status == 6
    o = torch.full((1, 50, 1, 16), 7.0, device="cuda")
    fs = torch.full((2, 1, 16, 16), 7.0, device="cuda")
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    ws = torch.empty(kda.workspace_bytes(q, k, v, b, la, cu, 16), dtype=torch.uint8, device="cuda")
    a = kda._make_args(q, k, v, b, la, cu, 16, torch.float32)
    a.o, a.final_state, a.initial_state = kda._ptr(o), kda._ptr(fs), kda._ptr(init)
    a.device_status, a.workspace = kda._ptr(status), kda._ptr(ws)
    a.workspace_bytes = ws.numel()
    assert kda.lib().kda_prefill_chunked(ctypes.byref(a), kda._stream(q.device)) == 0
    torch.cuda.synchronize()
    assert int(status.item()) == 6
    assert bool((o == 7.0).all()) and bool((fs == 7.0).all())


# --------------------------------------------------- matrix-core path ----
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("T", [1, 37, 100, 200])
def test_bf16_mfma_chunks_and_ragged_tails(D, chunk, T):
    x = synth.make_uniform(400 + T + D, 2, T, 2, D, D, "bf16", chunk=chunk, state_std=0.3)
    check(x, name="mfma")


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_bf16_mfma_slow_decay_boundaries(chunk):
    """alpha ~ 0.99 with an N(0, 0.02^2) state: carried state dominates, so a
    chunk-boundary mistake cannot hide behind fast forgetting."""
    x = synth.slow_decay(17, 1, 1000, 2, 128, 128, "bf16", chunk=chunk)
    check(x, name="mfma slow decay")


def test_bf16_mfma_extreme_gates():
    """10% of tokens with log alpha in [-20, -10] and beta in {1e-4, 1}:
    Gram blocks whose decay spans tens of powers of two, handled by the
    factorisation around each block's own reference points."""
    x = synth.make_long(55, 2048, 4, 128, 128, "bf16", chunk=64)
    check(x, name="mfma extreme")


def test_bf16_mfma_diagonal_blocks_beyond_the_factorisation_range():
    """Diagonal 16-token Gram blocks whose decay exceeds the midpoint
    factorisation's range (2^200 in some channel) are computed pair by pair.
    Forced here: log alpha = -20 on every token of some 16-token blocks (a
    block then decays by 16 x 20 nats = 462 powers of two) — in half of the
    channels of one block (so one channel half of the block takes the exact
    path and the other the factorised one), in all channels of another, and
    in a single channel of a third; the rest are typical gates."""
    x = synth.make_uniform(56, 1, 256, 2, 128, 128, "bf16", chunk=64, state_std=0.1)
    la = x.log_alpha.copy()
    la[0, 16:32, 0, :64] = -20.0     # head 0, chunk 0, block 1, channels 0..63
    la[0, 80:96, 1, :] = -20.0       # head 1, chunk 1, block 1, every channel
    la[0, 160:176, 0, 77] = -20.0    # head 0, chunk 2, block 2, one channel
    x.log_alpha = la                 # -20 is exact in bf16
    check(x, name="mfma diagonal beyond factorisation")


def test_bf16_mfma_packed_docs_with_empty_and_tiny():
    x = synth.make_packed(18, [70, 0, 1, 64, 129, 5], 3, 128, 128, "bf16", chunk=64)
    check(x, name="mfma packed")


def test_bf16_mfma_bf16_output():
    x = synth.make_uniform(19, 1, 300, 2, 128, 128, "bf16", chunk=64, state_std=0.1)
    q, k, v, b, la, init, _ = dev_tensors(x)
    o, S = kda.prefill(q, k, v, b, la, initial_state=init, out_dtype=torch.bfloat16)
    assert o.dtype == torch.bfloat16
    o_ref, S_ref, _ = native.prefill(x.q, x.k, x.v, x.beta, x.log_alpha, None, x.initial_state)
    d = np.abs(o.float().cpu().numpy() - o_ref)
    rms = np.sqrt(np.mean(o_ref ** 2))
    assert np.all(d <= 2e-2 * rms + 2.0 ** -8 * np.abs(o_ref))
    assert err(S, S_ref) <= 2e-2


def test_prefill_workload_T4096_H16():
    """B=1 H=16 T=4096 d=128 bf16, chunk 64, zero state: outputs, final state
    and all 64 boundary states per head."""
    check(synth.workload(2), name="prefill workload")


def test_packed_workload_8docs_H32():
    """8 documents, lengths U[512, 8192], H=32, d=128, per-document state:
    outputs, final states and the state entering every chunk of every
    document (the state must reset exactly at document boundaries)."""
    x = synth.workload(4, device="cuda")
    check(x, name="packed workload", boundaries=True)


def test_long_workload_T131072_H32_all_heads_and_continuation():
    """T=131072 H=32 d=128 with 10% extreme gates, every head.  The GPU runs
    the sequence in one pass and as 4 continuation calls of 32768 tokens
    passing the state; the two must be bitwise equal (the continuation
    boundaries are chunk boundaries, and a chunk's arithmetic does not depend
    on where the call started), and the single pass is compared with the
    fp64 oracle on the outputs and final state of all 32 heads, so the
    continuation is held to the oracle too."""
    x = synth.workload(5, device="cuda")
    q, k, v, b, la, _, _ = dev_tensors(x)
    o, S = kda.prefill(q, k, v, b, la)
    S_run = None
    outs = []
    for i in range(4):
        sl = slice(i * 32768, (i + 1) * 32768)
        oi, S_run = kda.prefill(q[:, sl].contiguous(), k[:, sl].contiguous(), v[:, sl].contiguous(),
                                b[:, sl].contiguous(), la[:, sl].contiguous(), initial_state=S_run)
        outs.append(oi)
    oc = torch.cat(outs, dim=1)
    del outs, q, k, v, b, la
    bitwise = bool(torch.equal(oc, o)) and bool(torch.equal(S_run, S))
    report("long continuation vs single pass", bitwise=float(bitwise))
    assert bitwise, "4 x 32768 continuation differs from the single pass"
    del oc, S_run
    torch.cuda.empty_cache()
    o_ref, S_ref, _ = native.prefill(x.q, x.k, x.v, x.beta, x.log_alpha)
    H = x.H
    oh = o.cpu().numpy()
    Sh = S.cpu().numpy()
    del o, S
    rms_o = float(np.sqrt(sum(float(np.dot(o_ref[0, :, h].ravel(), o_ref[0, :, h].ravel()))
                              for h in range(H)) / o_ref.size))
    rms_s = float(np.sqrt(np.mean(S_ref ** 2)))
    eo_h = [float(np.max(np.abs(oh[0, :, h] - o_ref[0, :, h]))) / rms_o for h in range(H)]
    es_h = [float(np.max(np.abs(Sh[0, h] - S_ref[0, h]))) / rms_s for h in range(H)]
    worst_o, worst_s = int(np.argmax(eo_h)), int(np.argmax(es_h))
    print("[parity] long T=131072 per head err(o): " + " ".join(f"{e:.2e}" for e in eo_h), flush=True)
    print("[parity] long T=131072 per head err(S): " + " ".join(f"{e:.2e}" for e in es_h), flush=True)
    report(f"long T=131072 H=32 all heads (worst o: head {worst_o}, worst S: head {worst_s})",
           o=max(eo_h), S=max(es_h))
    assert max(eo_h) <= 2e-2 and max(es_h) <= 2e-2


def test_mfma_packed_equals_separate_and_is_deterministic():
    lens = [200, 64, 1, 129]
    x = synth.make_packed(20, lens, 2, 128, 128, "bf16", chunk=64)
    q, k, v, b, la, init, cu = dev_tensors(x)
    o, S = kda.prefill(q, k, v, b, la, initial_state=init, cu_seqlens=cu)
    o2, S2 = kda.prefill(q, k, v, b, la, initial_state=init, cu_seqlens=cu)
    assert torch.equal(o, o2) and torch.equal(S, S2), "run-to-run results differ"
    c = x.cu_seqlens
    for n in range(len(lens)):
        sl = slice(int(c[n]), int(c[n + 1]))
        on, Sn = kda.prefill(q[:, sl].contiguous(), k[:, sl].contiguous(), v[:, sl].contiguous(),
                             b[:, sl].contiguous(), la[:, sl].contiguous(), initial_state=init[n:n + 1].contiguous())
        assert torch.equal(on, o[:, sl]), f"document {n}: packed output differs from separate"
        assert torch.equal(Sn, S[n:n + 1]), f"document {n}: packed state differs from separate"


@pytest.mark.parametrize("seed,ndocs,H,odt", [(22, 16, 4, torch.float32), (23, 32, 4, torch.float32),
                                               (24, 40, 4, torch.bfloat16), (25, 17, 5, torch.float32),
                                               (26, 41, 7, torch.float32)])
def test_mfma_wide_scan_tiles_equal_one_tile(seed, ndocs, H, odt):
    """With many (sequence, head) pairs the scan gives each workgroup 2
    (64 to 127 pairs) or 4 (128 or more) column tiles of a head, loading the
    block's shared operands once for them; each tile's arithmetic is that of
    a one-tile workgroup, which one call per document uses (a single
    sequence with a few heads).  Outputs, final states and every chunk-entry
    state must be bitwise equal.  85 and 287 pairs (H = 5, 7) leave the
    last group of 8 pairs partly empty."""
    g = np.random.default_rng(seed)
    lens = [int(n) for n in g.integers(1, 300, ndocs)]
    lens[0], lens[1] = 0, 64
    x = synth.make_packed(seed, lens, H, 128, 128, "bf16", chunk=64)
    q, k, v, b, la, init, cu = dev_tensors(x)
    o, S, cs = kda.prefill(q, k, v, b, la, initial_state=init, cu_seqlens=cu, chunk_states=True, out_dtype=odt)
    c = x.cu_seqlens
    ch = 0
    for n in range(ndocs):
        sl = slice(int(c[n]), int(c[n + 1]))
        if lens[n] == 0:
            assert torch.equal(S[n:n + 1], init[n:n + 1])
            continue
        on, Sn, csn = kda.prefill(q[:, sl].contiguous(), k[:, sl].contiguous(), v[:, sl].contiguous(),
                                  b[:, sl].contiguous(), la[:, sl].contiguous(), initial_state=init[n:n + 1].contiguous(),
                                  chunk_states=True, out_dtype=odt)
        nc = csn.shape[0]
        assert torch.equal(on, o[:, sl]), f"document {n}: output differs"
        assert torch.equal(Sn, S[n:n + 1]), f"document {n}: final state differs"
        assert torch.equal(csn, cs[ch:ch + nc]), f"document {n}: chunk-entry states differ"
        ch += nc
    assert ch == cs.shape[0]
    print(f"[wide scan] {ndocs} documents x {H} heads: bitwise equal to one call per document", flush=True)


def test_mfma_power_of_two_homogeneity():
    x = synth.make_uniform(21, 1, 150, 2, 128, 128, "bf16", chunk=64, state_std=0.2)
    q, k, v, b, la, init, _ = dev_tensors(x)
    o, S = kda.prefill(q, k, v, b, la, initial_state=init)
    o2, S2 = kda.prefill(q, k, 2 * v, b, la, initial_state=2 * init)
    assert torch.equal(o2, 2 * o) and torch.equal(S2, 2 * S)
