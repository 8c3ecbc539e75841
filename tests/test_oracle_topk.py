"""Pins of the top-k oracle (CPU only): hand-worked rows, ties, masking by
length, short rows, closed forms (a ramp), and agreement with torch.topk's
selected values (a library cross-check; the oracle itself only sorts)."""
import numpy as np
import pytest
import torch

from oracle import topk as TK


def test_hand_rows():
    x = np.array([[3.0, 1.0, 2.0, -5.0, 7.0],
                  [0.5, 0.5, 0.5, 0.25, 1.0]], np.float32)
    vals, count = TK.topk_values(x, 2)
    assert vals[0].tolist() == [7.0, 3.0] and vals[1].tolist() == [1.0, 0.5]
    assert count.tolist() == [2, 2]
    assert TK.kth_value(x, 2).tolist() == [3.0, 0.5]


def test_lengths_mask_the_tail():
    x = np.array([[1.0, 9.0, 2.0, 8.0, 100.0, 200.0]], np.float32)
    vals, count = TK.topk_values(x, 2, lengths=[4])
    assert vals[0].tolist() == [9.0, 8.0]
    vals, count = TK.topk_values(x, 3, lengths=[2])      # short row: everything valid
    assert count.tolist() == [2] and vals[0, :2].tolist() == [9.0, 1.0] and np.isnan(vals[0, 2])
    assert TK.row_lengths(3, 10, [-4, 3, 99]).tolist() == [0, 3, 10]


def test_ramp_closed_form():
    cols, k = 5000, 2048
    x = np.tile(np.arange(cols, dtype=np.float32), (3, 1))
    x[1] = x[1][::-1]
    lens = [cols, cols, 3000]
    vals, count = TK.topk_values(x, k, lens)
    assert np.array_equal(vals[0], np.arange(cols - 1, cols - 1 - k, -1, dtype=np.float32))
    assert np.array_equal(vals[1], np.arange(cols - 1, cols - 1 - k, -1, dtype=np.float32))
    assert np.array_equal(vals[2], np.arange(2999, 2999 - k, -1, dtype=np.float32))


def test_special_values():
    x = np.array([[-np.inf, 0.0, -0.0, np.inf, -1.0, 1e-40]], np.float32)
    vals, _ = TK.topk_values(x, 4)
    assert vals[0, 0] == np.inf and vals[0, 1] == np.float32(1e-40)
    assert vals[0, 2] == 0.0 and vals[0, 3] == 0.0     # +0 and -0 are equal values


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_values_match_torch_topk(seed):
    rng = np.random.default_rng(seed)
    rows, cols, k = 16, 3000, 257
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x[::3] = np.round(x[::3] * 4) / 4                    # many ties
    lens = rng.integers(0, cols + 1, rows)
    lens[0] = cols
    vals, count = TK.topk_values(x, k, lens)
    for r in range(rows):
        n = int(lens[r])
        if n <= k:
            assert count[r] == n
            continue
        ref = torch.topk(torch.from_numpy(x[r, :n]), k).values.numpy()
        assert np.array_equal(vals[r], ref)
