"""The overlapped matrix-core prefill against the two-kernel one.

For one sequence with few heads (the scan's column tiles fill at most half
of each XCD) the library runs the per-chunk stage and the scan in one launch:
on each XCD, workgroups computing the chunk blocks of that XCD's heads hand
each block to the scan workgroups of the same XCD through a flag, so the
scan walks the sequence while the blocks are still being produced.  The
arithmetic is the two-kernel path's, instruction for instruction, so its
outputs, final states and chunk-entry states must be bitwise equal to the
two-kernel launch's (forced with KDA_PREFILL_OVERLAP=0), and the device
status must stay 0.  The oracle comparisons of the single-sequence bf16
tests in test_prefill_gpu.py (the T=4096, H=16 workload among them) run on
this launch as well.  With fp32 inputs and d_k = 128 the fp32 path
overlaps its chunk prep and scan the same way (the last cases)."""
import os

import pytest
import torch

import gated_delta_rule_49_amd as kda
import synth
from kda_testutil import dev_tensors

pytestmark = pytest.mark.gpu


def _run(overlap, x, prologue=0, out_dtype=torch.float32, chunk=64):
    q, k, v, b, la, init, _ = dev_tensors(x)
    saved = os.environ.get("KDA_PREFILL_OVERLAP")
    os.environ["KDA_PREFILL_OVERLAP"] = "1" if overlap else "0"
    try:
        status = torch.full((1,), -1, dtype=torch.int32, device=q.device)
        o, S, cs = kda.prefill(q, k, v, b, la, initial_state=init, chunk_states=True, out_dtype=out_dtype,
                               prologue=prologue, device_status=status, chunk_size=chunk)
        torch.cuda.synchronize()
    finally:
        if saved is None:
            del os.environ["KDA_PREFILL_OVERLAP"]
        else:
            os.environ["KDA_PREFILL_OVERLAP"] = saved
    return o, S, cs, int(status.item())


# (seed, T, H, D, out dtype, prologue): XCDs with two heads, one head and
# none (H = 3, 11); one chunk, ragged tails; d = 64 (4 column tiles per head)
CASES = [
    (801, 4096, 16, 128, torch.float32, 0),
    (802, 1000, 3, 128, torch.bfloat16, 0),
    (803, 64, 16, 128, torch.float32, 0),
    (804, 130, 11, 128, torch.float32, 0),
    (805, 777, 8, 64, torch.float32, 0),
    (806, 2048, 32, 64, torch.bfloat16, 0),
    (807, 1500, 16, 128, torch.float32, 7),
]


@pytest.mark.parametrize("seed,T,H,D,odt,pro", CASES)
def test_overlapped_launch_equals_two_kernel_launch(seed, T, H, D, odt, pro):
    if pro:
        x = synth.make_preact(seed, 1, T, H, D, D, "bf16", chunk=64, state_std=0.1, prologue=pro)
    else:
        x = synth.make_uniform(seed, 1, T, H, D, D, "bf16", chunk=64, state_std=0.1)
    a = _run(True, x, pro, odt)
    b = _run(False, x, pro, odt)
    assert a[3] == 0 and b[3] == 0, (a[3], b[3])
    for name, u, w in zip(("o", "final state", "chunk states"), a[:3], b[:3]):
        assert torch.equal(u, w), name
    print(f"[overlap] T={T} H={H} D={D}: bitwise equal to the two-kernel launch", flush=True)


def test_overlapped_long_sequence_repeats_exactly():
    """T=32768, H=16 (512 chunks per head, 8192 hand-offs): three calls on
    one workspace (its flags cleared by each call's table kernel) give the
    same bits as the two-kernel launch."""
    x = synth.make_long(808, 32768, 16, 128, 128, "bf16", chunk=64)
    ref = _run(False, x)
    for _ in range(3):
        got = _run(True, x)
        assert got[3] == 0
        assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1]) and torch.equal(got[2], ref[2])


def test_overlapped_launch_under_every_xcd_rotation():
    """The XCD the hardware deals a launch's first workgroup to depends on
    earlier launches (the round-robin deal continues across them).  Roles
    follow the XCD a workgroup actually runs on, so any rotation gives the
    same bits: before each call 0..7 one-workgroup kernels rotate the deal."""
    x = synth.make_uniform(809, 1, 2048, 16, 128, 128, "bf16", chunk=64, state_std=0.1)
    ref = _run(False, x)
    tiny = torch.zeros(4, device="cuda")
    for shift in range(8):
        for _ in range(shift):
            tiny.add_(1.0)   # one workgroup
        got = _run(True, x)
        assert got[3] == 0, (shift, got[3])
        for u, w in zip(got[:3], ref[:3]):
            assert torch.equal(u, w), shift


def test_expired_wait_reports_and_the_next_call_recovers():
    """The failure path of the hand-off, forced from the host: with a wait
    bound of 0 ticks the scan workgroups give up at their first unpublished
    block (every block takes microseconds to produce), so the call records
    KDA_ERR_DEVICE_WAIT (8) and still completes; the next call, with the
    normal bound, clears the status and gives the two-kernel launch's
    bits."""
    x = synth.make_uniform(810, 1, 1024, 16, 128, 128, "bf16", chunk=64, state_std=0.1)
    ref = _run(False, x)
    os.environ["KDA_PREFILL_WAIT_TICKS"] = "0"
    try:
        bad = _run(True, x)
    finally:
        del os.environ["KDA_PREFILL_WAIT_TICKS"]
    assert bad[3] == 8, bad[3]
    good = _run(True, x)
    assert good[3] == 0
    for u, w in zip(good[:3], ref[:3]):
        assert torch.equal(u, w)


# fp32 inputs (the 1e-5 contract, fp32 matrix cores): with d_k = 128 the
# chunk prep and the fp32 scan overlap the same way, at every chunk size
F32_CASES = [(811, 4096, 16, 64, torch.float32, 0), (812, 1000, 3, 64, torch.bfloat16, 0),
             (813, 130, 11, 64, torch.float32, 0), (814, 1500, 16, 64, torch.float32, 7),
             (815, 999, 5, 32, torch.float32, 0), (816, 777, 16, 16, torch.float32, 0)]


@pytest.mark.parametrize("seed,T,H,C,odt,pro", F32_CASES)
def test_overlapped_fp32_launch_equals_two_kernel_launch(seed, T, H, C, odt, pro):
    if pro:
        x = synth.make_preact(seed, 1, T, H, 128, 128, "f32", chunk=C, state_std=0.1, prologue=pro)
    else:
        x = synth.make_uniform(seed, 1, T, H, 128, 128, "f32", chunk=C, state_std=0.1)
    a = _run(True, x, pro, odt, C)
    b = _run(False, x, pro, odt, C)
    assert a[3] == 0 and b[3] == 0, (a[3], b[3])
    for name, u, w in zip(("o", "final state", "chunk states"), a[:3], b[:3]):
        assert torch.equal(u, w), name
    print(f"[overlap fp32] T={T} H={H} C={C}: bitwise equal to the two-kernel launch", flush=True)
