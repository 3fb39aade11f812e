"""ctypes binding and build step for the C oracle (``kda_oracle.c``).

TEST INFRASTRUCTURE ONLY (see ``reference.py``).  The build uses gcc with
OpenMP; it targets a generic x86-64-v3 host so the library built here also
loads on other hosts.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kda_oracle.c")
LIB = os.path.join(HERE, "libkda_oracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile ``libkda_oracle.so`` next to its source."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        cmd = ["gcc", "-O3", "-march=x86-64-v3", "-fopenmp", "-fPIC", "-shared", "-std=c11",
               "-Wall", "-o", tmp, SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build(force=False)
        lib = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.kda_oracle_prefill.argtypes = [I64, P, I64, I64, I64, I64, P, P, P, P, P, P, P, P,
                                           I64, P, ctypes.c_int, ctypes.c_int]
        lib.kda_oracle_prefill.restype = ctypes.c_int
        lib.kda_oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().kda_oracle_max_threads())


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def prefill(q, k, v, beta, log_alpha, cu_seqlens=None, initial_state=None, chunk=0,
            want_chunk_states=False, nthreads=0, prologue_flags=0):
    """Run the C oracle.  Arrays as in ``reference.prefill`` (q [B,T,H,dk] ...).
    Rows of a batch are treated as separate sequences (B > 1 requires
    cu_seqlens is None).  ``prologue_flags`` as in ``reference.prologue``.
    Returns (o [B,T,H,dv], final [N,H,dk,dv], chunk_states or None), all
    fp64."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    f32 = np.float32
    # Rows of a batch become consecutive documents of a packed sequence.
    qq, kk, vv, bb, gg = (np.ascontiguousarray(a, dtype=f32).reshape((B * T,) + a.shape[2:])
                          for a in (q, k, v, beta, log_alpha))
    if cu_seqlens is None:
        cu = np.arange(0, B * T + 1, T, dtype=np.int64) if T > 0 else np.zeros(B + 1, np.int64)
    else:
        if B != 1:
            raise ValueError("cu_seqlens requires B == 1")
        cu = np.asarray(cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    init = None if initial_state is None else np.ascontiguousarray(initial_state, dtype=np.float64)
    if init is not None and init.shape != (N, H, dk, dv):
        raise ValueError(f"initial_state shape {init.shape} != {(N, H, dk, dv)}")
    o = np.zeros((B * T, H, dv), np.float64)
    final = np.zeros((N, H, dk, dv), np.float64)
    cs = None
    if want_chunk_states:
        if chunk <= 0:
            raise ValueError("chunk_states need chunk > 0")
        nch = int(sum((int(cu[n + 1] - cu[n]) + chunk - 1) // chunk for n in range(N)))
        cs = np.zeros((nch, H, dk, dv), np.float64)
    rc = _load().kda_oracle_prefill(N, _ptr(cu), B * T, H, dk, dv, _ptr(qq), _ptr(kk), _ptr(vv),
                                    _ptr(bb), _ptr(gg), _ptr(init), _ptr(final), _ptr(o),
                                    int(chunk), _ptr(cs), int(nthreads), int(prologue_flags))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_prefill failed: {rc}")
    return o.reshape(B, T, H, dv), final, cs


def decode_steps(q, k, v, beta, log_alpha, initial_state, nthreads=0, prologue_flags=0):
    """Token-by-token trajectory of B independent sequences over ``steps``
    single-token steps: q [steps,B,H,dk] ...  Returns (o [steps,B,H,dv],
    states [steps,B,H,dk,dv]) in fp64, the state after every step."""
    steps, B, H, dk = q.shape
    dv = v.shape[-1]
    S = np.ascontiguousarray(initial_state, dtype=np.float64)
    outs = np.zeros((steps, B, H, dv), np.float64)
    states = np.zeros((steps, B, H, dk, dv), np.float64)
    for s in range(steps):
        # B sequences of one token each, one packed call
        o, S, _ = prefill(q[s][None], k[s][None], v[s][None], beta[s][None], log_alpha[s][None],
                          cu_seqlens=np.arange(B + 1, dtype=np.int64), initial_state=S,
                          nthreads=nthreads, prologue_flags=prologue_flags)
        outs[s] = o[0]
        states[s] = S
    return outs, states
