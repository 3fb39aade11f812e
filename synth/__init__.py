"""Seeded synthetic input generators (no recurrence arithmetic lives here)."""
from .kda_inputs import (  # noqa: F401
    KDAInputs, DecodeInputs, workload, decode_workload, make_uniform, make_packed, make_preact,
    make_long, long_tensors, slow_decay, c4_lengths, bf16_bits, bits_to_f32, round_bf16,
)
