"""The allocation-free top-k entry point against the ordinary one, through the
C ABI: dsaidx_topk_per_row_noalloc takes its split-row workspace from the
library's own device array instead of a caller workspace.  Two calls in a row
(the second smaller, on the same array), a call that needs no workspace, and a
call too large for the array, which must be refused with nothing launched.
Acceptance as for top-k: where a row has more than k valid logits, the k
indices are distinct, inside the row and select the same multiset of values as
the ordinary entry point (and as the oracle); where it has at most k, the
result is exactly 0..len-1 then -1."""
import numpy as np
import pytest
import torch

import rope_fp8_quant_amd as R
from oracle import topk as TK
from rope_fp8_quant_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def same_selection(a: np.ndarray, b: np.ndarray, logits: np.ndarray, lengths, k: int):
    rows, cols = logits.shape
    lens = TK.row_lengths(rows, cols, lengths)
    want, _ = TK.topk_values(logits, k, lengths)
    for r in range(rows):
        n = int(lens[r])
        if n <= k:
            ident = np.concatenate([np.arange(n), np.full(k - n, -1)])
            assert np.array_equal(a[r], ident) and np.array_equal(b[r], ident), r
            continue
        for sel in (a[r], b[r]):
            assert np.all((sel >= 0) & (sel < n)) and np.unique(sel).size == k, r
        va, vb = np.sort(logits[r, a[r]])[::-1], np.sort(logits[r, b[r]])[::-1]
        assert np.array_equal(va, vb), r
        assert np.array_equal(va, want[r]), r


def run_both(rows, cols, k, seed):
    tw = W.topk_make(rows, cols, k=k, lengths="ragged", seed=seed)
    print("\n[case] noalloc rows=%d cols=%d k=%d seed=%d" % (rows, cols, k, seed), flush=True)
    d = torch.from_numpy(tw.logits).cuda()
    dl = torch.from_numpy(tw.lengths).cuda()
    ref = torch.full((rows, k), -7, dtype=torch.int32, device="cuda")
    got = torch.full((rows, k), -7, dtype=torch.int32, device="cuda")
    R.dsaidx_topk_per_row(d, k, ref, dl)
    R.dsaidx_topk_per_row_noalloc(d, k, got, dl)
    torch.cuda.synchronize()
    same_selection(got.cpu().numpy(), ref.cpu().numpy(), tw.logits, tw.lengths, k)
    return R.dsaidx_topk_workspace_bytes(rows, cols, k)


def test_noalloc_matches_workspace_entry_twice():
    """Two split-path calls in a row on the same library array, the second
    smaller (fewer rows, shorter rows), then a call that needs no workspace."""
    ws1 = run_both(64, 131072, 2048, 71)
    ws2 = run_both(9, 40000, 1000, 72)
    assert 0 < ws2 < ws1 <= R.binding.TOPK_NOALLOC_SCRATCH_BYTES
    assert run_both(33, 5000, 256, 73) == 0


def test_noalloc_refuses_a_workspace_beyond_its_array():
    rows, cols, k = 228, 131072, 2048
    assert R.dsaidx_topk_workspace_bytes(rows, cols, k) > R.binding.TOPK_NOALLOC_SCRATCH_BYTES
    d = torch.zeros((rows, cols), dtype=torch.float32, device="cuda")
    out = torch.full((rows, k), -7, dtype=torch.int32, device="cuda")
    with pytest.raises(R.DsaidxError):
        R.dsaidx_topk_per_row_noalloc(d, k, out)
    torch.cuda.synchronize()
    assert bool((out == -7).all())
    # the largest call the array holds still runs
    rows = R.binding.TOPK_NOALLOC_SCRATCH_BYTES // R.dsaidx_topk_workspace_bytes(1, cols, k)
    assert rows == 227
