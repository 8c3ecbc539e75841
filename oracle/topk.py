"""Top-k per row — TEST INFRASTRUCTURE ONLY (oracle of dsaidx_topk_per_row).

Only tests, the smoke check and the benchmark's CPU-baseline leg use this.

The selection that follows the index logits: each query keeps the index_topk
(2048) highest-scoring keys ([sglang-fuse] = sglang PR "[AMD] [GLM5] Fuse the
DSA indexer Q/K rope + quant + K-cache write", section Benchmark; the
topKPerRowDecode launch after the paged MQA logits in vLLM PR 47335,
section Kernel-level evidence).  Plain definition, written out with a sort:

  row r is valid over columns [0, len_r) with len_r = min(lengths[r], cols)
  (all cols when no lengths are given); if len_r <= k the result is
  0, 1, ..., len_r - 1 followed by -1; otherwise it is the indices of the k
  largest valid logits.  Which of several equal logits at the k-th place are
  taken is not determined; the multiset of selected values is.
"""
from __future__ import annotations

import numpy as np


def row_lengths(rows: int, cols: int, lengths=None) -> np.ndarray:
    if lengths is None:
        return np.full(rows, cols, dtype=np.int64)
    return np.clip(np.asarray(lengths, dtype=np.int64), 0, cols)


def topk_values(logits: np.ndarray, k: int, lengths=None):
    """Per row: the k largest valid logits in descending order (float32), and
    the count taken (min(len_r, k)); rows shorter than k are padded with NaN."""
    logits = np.asarray(logits, dtype=np.float32)
    rows, cols = logits.shape
    lens = row_lengths(rows, cols, lengths)
    vals = np.full((rows, k), np.nan, dtype=np.float32)
    count = np.zeros(rows, dtype=np.int64)
    for r in range(rows):
        n = int(lens[r])
        v = np.sort(logits[r, :n])[::-1]
        take = min(n, k)
        vals[r, :take] = v[:take]
        count[r] = take
    return vals, count


def kth_value(logits: np.ndarray, k: int, lengths=None) -> np.ndarray:
    """The k-th largest valid logit of each row (NaN where the row has <= k)."""
    vals, count = topk_values(logits, k, lengths)
    out = np.full(vals.shape[0], np.nan, dtype=np.float32)
    full = count == k
    rows, cols = np.asarray(logits).shape
    lens = row_lengths(rows, cols, lengths)
    out[full & (lens > k)] = vals[full & (lens > k), k - 1]
    return out
