"""Helpers shared by the GPU parity tests: move seeded inputs to the device in
the workload's dtype and compare against the oracle with the error metric
max|x - x_ref| / RMS(x_ref)."""
import numpy as np
import torch

from oracle import rel_err

# Tolerances of the numerical contract, fixed before any comparison is run
# (Module 11 — Correctness as Architecture Mastery, §4 "Specify the contract
# before you benchmark"): fp32 inputs 1e-5, bf16 inputs with fp32 state and
# accumulation 2e-2, both relative to the RMS of the oracle's result.
TOL = {"f32": 1e-5, "bf16": 2e-2}


def tdtype(dtype: str):
    return torch.float32 if dtype == "f32" else torch.bfloat16


def dev_tensors(x, device="cuda"):
    """(q, k, v, beta, log_alpha, initial_state, cu_seqlens) on the GPU."""
    dt = tdtype(x.dtype)

    def t(a):
        # values are exact in dt (the generator rounded them already)
        return torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=dt)

    init = None if x.initial_state is None else torch.from_numpy(x.initial_state).to(device)
    cu = None if x.cu_seqlens is None else torch.from_numpy(x.cu_seqlens.astype(np.int32)).to(device)
    return t(x.q), t(x.k), t(x.v), t(x.beta), t(x.log_alpha), init, cu


def err(gpu_tensor, ref):
    return rel_err(gpu_tensor.detach().float().cpu().numpy(), ref)


def report(name, **errs):
    msg = " ".join(f"{k}={v:.3e}" for k, v in errs.items())
    print(f"[parity] {name}: {msg}", flush=True)
