"""Recurrent and chunked execution of the same sequences agree on outputs and
final state (Module 04 — KDA II: Chunked Parallelism & the Full Sublayer,
§4: the chunked form must reproduce the recurrent one, with the state
readable at chunk boundaries).  The recurrent side is the GPU decode kernel
run over all T tokens of each sequence in one launch (T single steps); the
chunked side is the GPU prefill.  Both are also held to the fp64 oracle,
and their mutual difference to the same contract (err = max|x - y| /
RMS(y) <= 1e-5 for fp32 inputs, 2e-2 for bf16)."""
import numpy as np
import pytest
import torch

import gated_delta_rule_49_amd as kda
import synth
from oracle import native
from kda_testutil import TOL, dev_tensors, err, report

pytestmark = pytest.mark.gpu


def both(x, chunk):
    q, k, v, b, la, S0, _ = dev_tensors(x)
    o_c, S_c = kda.prefill(q, k, v, b, la, initial_state=S0, chunk_size=chunk)
    S_r = S0.clone()
    o_r, _, _ = kda.decode(q, k, v, b, la, S_r)          # [B, m=T, H, d], state in place
    o_ref, S_ref, _ = native.prefill(x.q, x.k, x.v, x.beta, x.log_alpha, initial_state=x.initial_state)
    return o_c, S_c, o_r, S_r, o_ref, S_ref


@pytest.mark.parametrize("dtype,chunk,T,gate_mean", [
    ("bf16", 64, 200, 0.0),     # matrix-core prefill, ragged last chunk
    ("bf16", 32, 130, -5.0),    # slow decay: the carried state dominates
    ("bf16", 16, 77, 0.0),
    ("f32", 16, 100, 0.0),      # fp32 prefill path
    ("f32", 64, 150, -5.0),
])
def test_recurrent_and_chunked_agree(dtype, chunk, T, gate_mean):
    x = synth.make_uniform(300 + T, 3, T, 4, 128, 128, dtype, chunk=chunk, state_std=0.02, gate_mean=gate_mean)
    o_c, S_c, o_r, S_r, o_ref, S_ref = both(x, chunk)
    e = dict(chunked_o=err(o_c, o_ref), chunked_S=err(S_c, S_ref), recurrent_o=err(o_r, o_ref),
             recurrent_S=err(S_r, S_ref),
             mutual_o=err(o_c, o_r.double().cpu().numpy()), mutual_S=err(S_c, S_r.double().cpu().numpy()))
    report(f"recurrent vs chunked {dtype} C={chunk} T={T} gate_mean={gate_mean}", **e)
    assert max(e.values()) <= TOL[dtype]


def test_chunk_boundary_states_match_recurrent_states():
    """The chunked prefill's state entering every chunk equals the recurrent
    decode's state after the token before it (per-token states)."""
    x = synth.make_uniform(311, 2, 96, 2, 128, 128, "bf16", chunk=32, state_std=0.02, gate_mean=-5.0)
    q, k, v, b, la, S0, _ = dev_tensors(x)
    _, _, cs = kda.prefill(q, k, v, b, la, initial_state=S0, chunk_size=32, chunk_states=True)
    _, _, ts = kda.decode(q, k, v, b, la, S0.clone(), token_states=True)   # [B, T, H, dk, dv]
    # chunks are numbered sequence by sequence: 3 per sequence
    worst = 0.0
    for n in range(2):
        for c in range(3):
            ref = S0[n] if c == 0 else ts[n, 32 * c - 1]
            worst = max(worst, err(cs[3 * n + c], ref.double().cpu().numpy()))
    report("chunk-entry states vs recurrent token states", worst=worst)
    assert worst <= TOL["bf16"]
