"""The bf16 chunked backward is deterministic: five runs of one call give
the same bits for all six gradients.  Every sum in its kernels has a fixed
order (dbeta's per-block partial sums included, which once went through
LDS atomics whose order depended on timing), and the device status word
reads 0."""
import pytest
import torch

import gated_delta_rule_49_amd as kda
import synth
from kda_testutil import dev_tensors

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dbeta", "dlog_alpha", "d_initial_state")


@pytest.mark.parametrize("T,H", [(4096, 16), (1000, 3)])
def test_backward_repeats_bitwise(T, H):
    x = synth.make_uniform(907 + H, 1, T, H, 128, 128, "bf16", chunk=64, state_std=0.1)
    q, k, v, b, la, init, _ = dev_tensors(x)
    g = torch.Generator(device="cuda").manual_seed(T + H)
    d_o = torch.randn((1, T, H, 128), generator=g, device="cuda")
    d_final = torch.randn((1, H, 128, 128), generator=g, device="cuda") * 0.1
    _, _, ck = kda.prefill(q, k, v, b, la, initial_state=init, output_final_state=False, chunk_size=64,
                           chunk_states=True)
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    ref = kda.backward(q, k, v, b, la, d_o, initial_state=init, d_final_state=d_final, checkpoints=ck,
                       chunk_size=64, device_status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for _ in range(4):
        got = kda.backward(q, k, v, b, la, d_o, initial_state=init, d_final_state=d_final, checkpoints=ck,
                           chunk_size=64)
        for name, u, w in zip(NAMES, got, ref):
            assert torch.equal(u, w), name
