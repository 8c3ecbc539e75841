"""Index logits over the index-K cache -- TEST INFRASTRUCTURE ONLY (oracle of
dsaidx_mqa_logits).

Only tests, the smoke check and the benchmark's CPU-baseline leg use this.

The pages name the consumer of the prepared query (the fp8 paged MQA-logits
launch that follows the indexer prep and precedes the top-k: [vllm-47335] =
vLLM PR 47335 "Enable fused indexer-Q RoPE+quant kernel", section Kernel-level
evidence) but do not write out what it computes.  The reading taken here is
the one under which the prep step's fold is exact: folding the per-head query
scale 2^e into the head gate is only valid if the consumer applies a ReLU
(which commutes with a positive factor) to each head's dot product and then
sums the heads weighted by their gates.  With the K row's scale applied the
same way:

  logit[t, s] = k_scale[slot(s)] * sum_h w[t, h] * max(0, sum_d q[t, h, d] * k[slot(s), d])

where q and k are the decoded fp8 codes (E4M3FN), w the folded gates
(weights_out of the prep call) and slot(s) = key_slots[s] (s itself when no
slot list is given).  Key s of query t is valid when s < lengths[t]; other
entries are not defined (NaN here).

Plain definition: exact decoding through the oracle's fp8 table, dot
products in float64 (exact: each product of two E4M3 values has at most 8
significant bits and exponents within [-18, 17], so 128 of them sum exactly
in 53 bits), then the ReLU, gate and scale in float64.
"""
from __future__ import annotations

import numpy as np

import oracle

ROW = 128
_DECODE = None


def decode_table() -> np.ndarray:
    """float64 value of each of the 256 E4M3FN codes (NaN codes as NaN)."""
    global _DECODE
    if _DECODE is None:
        _DECODE = np.array([oracle.fp8_decode(c) for c in range(256)], dtype=np.float64)
    return _DECODE


def head_dots(q_fp8: np.ndarray, k_rows: np.ndarray) -> np.ndarray:
    """dots[t, h, s] = q[t, h, :] . k[s, :] over the decoded codes (float64)."""
    dec = decode_table()
    q = dec[np.asarray(q_fp8, dtype=np.uint8)]
    k = dec[np.asarray(k_rows, dtype=np.uint8)[:, :ROW]]
    T, H, D = q.shape
    return (q.reshape(T * H, D) @ k.T).reshape(T, H, k.shape[0])


def mqa_logits(q_fp8, weights, k_cache, k_scale, key_slots=None, lengths=None) -> np.ndarray:
    """Index logits [T, N] in float64 (NaN where s >= lengths[t])."""
    q_fp8 = np.asarray(q_fp8, dtype=np.uint8)
    T, H, _ = q_fp8.shape
    k_cache = np.asarray(k_cache, dtype=np.uint8)
    slots = np.arange(k_cache.shape[0]) if key_slots is None else np.asarray(key_slots, np.int64)
    dots = head_dots(q_fp8, k_cache[slots])
    w = np.asarray(weights, dtype=np.float64).reshape(T, H)
    out = np.einsum("th,ths->ts", w, np.maximum(dots, 0.0))
    out *= np.asarray(k_scale, dtype=np.float64)[slots][None, :]
    if lengths is not None:
        n = np.clip(np.asarray(lengths, dtype=np.int64), 0, len(slots))
        out[np.arange(out.shape[1])[None, :] >= n[:, None]] = np.nan
    return out
