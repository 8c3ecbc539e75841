"""Key / head-gate projection — TEST INFRASTRUCTURE ONLY (oracle of
dsaidx_proj_k_norm_rope_quant_store).

Only tests, the smoke check and the benchmark's CPU-baseline leg use this.

The indexer gets its key and its head gates from one projection of the hidden
states, the fused wk_weights_proj GEMM ([sglang-fuse] = sglang PR "[AMD]
[GLM5] Fuse the DSA indexer Q/K rope + quant + K-cache write", section
Motivation):

  out[t, n] = sum_c hidden[t, c] * weight[n, c]
  n < 128          the key row of token t
  128 <= n < 128+H the head gate of head n - 128

written as bf16 (round to nearest, ties to even), the projection's output
type; the key then goes through the key preparation (oracle.k_side) and the
gates are the weights input of the query side.

Plain definition: numpy's float64 matrix product is the sum (every product of
two bf16 values is exact in float64, and the sums carry 53 bits, so the value
is the exact sum to within d * 2^-53 * sum |products|), and the bf16 rounding is
taken directly from that float64 value -- no intermediate fp32 rounding.
Values in the normal bf16 range only (as everywhere in the method, NaN, Inf
and overflow are outside the contract).
"""
from __future__ import annotations

import numpy as np

ROW = 128


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) to float64, exactly."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """The nearest bf16 (8 significant bits) to each float64 value, ties to
    the even significand, as uint16 bit patterns.  x = m * 2^e with
    0.5 <= |m| < 1; the bf16 neighbours are multiples of 2^(e - 8)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    q = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)      # rint: half to even
    return (q.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def projection_values(hidden_bits: np.ndarray, weight_bits: np.ndarray):
    """(out [T, N] float64 sums, abs_sum [T, N] = sum_c |hidden[t, c] *
    weight[n, c]|) for hidden bf16 [T, d] and weight bf16 [N, d]."""
    x = bf16_bits_to_f64(hidden_bits)
    w = bf16_bits_to_f64(weight_bits)
    return x @ w.T, np.abs(x) @ np.abs(w).T


def projection(hidden_bits: np.ndarray, weight_bits: np.ndarray):
    """The projection as the GEMM writes it: (key bf16 bits [T, 128], gate
    bf16 bits [T, H]) for weight rows 0..127 (key) and 128..127+H (gates)."""
    out, _ = projection_values(hidden_bits, weight_bits)
    bits = round_to_bf16_bits(out)
    return np.ascontiguousarray(bits[:, :ROW]), np.ascontiguousarray(bits[:, ROW:])
