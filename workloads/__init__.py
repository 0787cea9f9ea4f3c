"""Seeded synthetic inputs for the attention forward pass.

This module only draws and encodes numbers: it holds none of the attention
arithmetic.  Both the float64 oracle (``oracle/``) and the HIP path receive
their inputs from here, byte for byte, so that a parity test compares the two
on identical data.

Recipe (one workload = one seed):
  * Q, then K, then V are drawn in that order from
    ``numpy.random.default_rng(seed)`` (PCG64) as
    ``standard_normal((B, H, N, d), dtype=float32)``.
  * ``f32`` workloads keep the drawn values.
  * ``bf16`` workloads round each float32 to bfloat16 with round-to-nearest-even.
  * ``fp8`` workloads start from the bf16 tensors of the same shape and seed and
    quantise each tensor with one per-tensor scale s = amax|x| / 448 to OCP
    e4m3fn (round-to-nearest-even, saturating at +-448).  The kernel receives
    the e4m3 bytes plus s as a "descale"; the oracle receives the dequantised
    values x8 * s exactly, in float64.
  * Decode workloads (``N_q`` set) draw Q as [B, H, N_q, d] and K, V as
    [B, H_kv, N, d], in the same order.
  * The backward's upstream gradient dO is drawn the same way from
    ``default_rng(seed + 7919)`` and rounded to bfloat16 (``make_grad_output``).
"""

from .encode import (bf16_bits_from_f32, bf16_bits_to_f64, e4m3fn_bits_from_f32,
                     e4m3fn_bits_to_f64, E4M3FN_MAX)
from .gen import Workload, WORKLOADS, DECODE_WORKLOADS, by_name, make_inputs, make_grad_output, AttnInputs

__all__ = [
    "bf16_bits_from_f32", "bf16_bits_to_f64", "e4m3fn_bits_from_f32", "e4m3fn_bits_to_f64",
    "E4M3FN_MAX", "Workload", "WORKLOADS", "DECODE_WORKLOADS", "by_name", "make_inputs", "make_grad_output", "AttnInputs",
]
