"""GPU parity of dsaidx_topk_per_row against the top-k oracle.

Acceptance: where a row has more than k valid logits, the k returned indices
are distinct, valid (inside the row's length) and select exactly the oracle's
multiset of the k largest values (ties at the k-th place may be broken either
way); where it has at most k, the result is 0..len-1 followed by -1.
"""
import json

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


def run_topk(logits: np.ndarray, k: int, lengths=None, pad_cols: int = 0, pad_value=np.inf):
    rows, cols = logits.shape
    stride = cols + pad_cols
    stride += (-stride) % 4
    buf = np.full((rows, stride), pad_value, np.float32)
    buf[:, :cols] = logits
    d = torch.from_numpy(buf).cuda()[:, :cols]
    dl = None if lengths is None else torch.from_numpy(np.asarray(lengths, np.int32)).cuda()
    out = torch.full((rows, k), -7, dtype=torch.int32, device="cuda")
    R.dsaidx_topk_per_row(d, k, out, dl)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check(idx: np.ndarray, logits: np.ndarray, k: int, lengths=None):
    rows, cols = logits.shape
    lens = TK.row_lengths(rows, cols, lengths)
    want_vals, count = TK.topk_values(logits, k, lengths)
    ties_broken = 0
    for r in range(rows):
        n = int(lens[r])
        if n <= k:
            assert np.array_equal(idx[r], np.concatenate([np.arange(n), np.full(k - n, -1)])), r
            continue
        sel = idx[r]
        assert np.all((sel >= 0) & (sel < n)), r
        assert np.unique(sel).size == k, r
        got = np.sort(logits[r, sel])[::-1]
        assert np.array_equal(got, want_vals[r]), r       # -0 == +0 compares equal
        kth = want_vals[r, k - 1]
        ties_broken += int(np.count_nonzero(logits[r, :n] == kth) > np.count_nonzero(got == kth))
    return ties_broken


@pytest.mark.parametrize("idx", [0, 1, 2])
def test_named_workloads(idx):
    wl = W.topk_named(idx)
    out = run_topk(wl.logits, wl.k, wl.lengths)
    tb = check(out, wl.logits, wl.k, wl.lengths)
    print("\n[parity] topk %s %s" % (wl.name, json.dumps(dict(rows=int(wl.logits.shape[0]),
                                                               rows_with_tied_kth=tb))), flush=True)


@pytest.mark.parametrize("k", [1, 2, 7, 255, 2048, 4095])
def test_k_values(k):
    wl = W.topk_make(19, 4099, k=k, lengths="ragged", seed=k)
    out = run_topk(wl.logits, k, wl.lengths, pad_cols=5)
    check(out, wl.logits, k, wl.lengths)


def test_all_equal_rows_and_special_values():
    rows, cols, k = 6, 1000, 100
    x = np.zeros((rows, cols), np.float32)
    x[1] = 3.5                                   # every value ties
    x[2, ::2] = -0.0                             # +0 and -0 (equal values)
    x[3] = -np.inf
    x[3, 17] = 1.0
    x[4] = np.linspace(-1, 1, cols, dtype=np.float32)
    x[4, 900:] = np.inf
    x[5] = np.float32(1e-42)                     # fp32 subnormals
    x[5, 5] = np.float32(2e-42)
    out = run_topk(x, k)
    check(out, x, k)
    assert 17 in out[3]
    assert set(range(900, 1000)) == set(out[4].tolist())


def test_lengths_edge_cases():
    rng = np.random.default_rng(3)
    rows, cols, k = 8, 3000, 256
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    lens = np.array([0, 1, 255, 256, 257, 3000, 5000, -3], np.int32)
    out = run_topk(x, k, lens, pad_cols=11, pad_value=np.inf)
    check(out, x, k, lens)
    out = run_topk(x, k, None, pad_cols=11, pad_value=np.inf)
    check(out, x, k, None)


def test_many_rows_prefill_shape():
    wl = W.topk_make(3000, 4096, k=512, lengths="causal", seed=8)
    out = run_topk(wl.logits, 512, wl.lengths)
    check(out, wl.logits, 512, wl.lengths)


@pytest.mark.parametrize("cols", [3000, 8192, 12000, 30000])
def test_list_paths_across_row_counts(cols):
    """From 1024 rows on, a call resolves each long B1 list with one
    wavefront; smaller calls use the whole workgroup.  The same rows go
    through both: plain rows (lists of a few hundred), rows of heavy ties (a
    B1 of one repeated value) and narrow-range rows (B1 beyond the list)."""
    k = 2048
    rng = np.random.default_rng(cols)
    x = rng.standard_normal((1024, cols)).astype(np.float32)
    x[1::3] = np.round(x[1::3] * 8) / 8
    x[2::7] = (100.0 + 1e-3 * x[2::7]).astype(np.float32)
    lengths = rng.integers(k - 10, cols + 1, 1024).astype(np.int32)
    for rows in (1024, 1023):
        out = run_topk(x[:rows], k, lengths[:rows])
        check(out, x[:rows], k, lengths[:rows])


def test_empty_and_invalid_calls():
    x = torch.zeros((0, 64), dtype=torch.float32, device="cuda")
    out = torch.zeros((0, 8), dtype=torch.int32, device="cuda")
    R.dsaidx_topk_per_row(x, 8, out)
    x = torch.zeros((4, 64), dtype=torch.float32, device="cuda")
    out = torch.zeros((4, 8), dtype=torch.int32, device="cuda")
    with pytest.raises(R.DsaidxError):
        R.dsaidx_topk_per_row(x[:, 1:], 8, out)   # data pointer not 16-byte aligned


def test_degenerate_value_ranges():
    """Spans that defeat the linear coarse binning (huge, subnormal, a single
    finite value among infinities) fall back to the exact selection."""
    rows, cols, k = 5, 6000, 300
    rng = np.random.default_rng(9)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x[0, :3] = [-3e38, 3e38, 1e38]                         # span overflows fp32
    x[1] = np.float32(1e-44) * rng.integers(0, 5, cols).astype(np.float32)   # subnormal span
    x[2] = -np.inf
    x[2, 100:500] = 2.0                                    # one finite value
    x[3] = np.round(x[3])                                  # few distinct values: heavy ties
    x[4, :] = 7.0
    x[4, 4000:4300] = np.inf
    out = run_topk(x, k)
    check(out, x, k)


# Every launch variant: register-resident rows of up to 4096 / 8192 / 16384 /
# 32768 logits, the two-dispatch chunk + merge path (merge of up to 16384 and
# up to 32768 candidates), and the generic kernel for k too large for those.
@pytest.mark.parametrize("rows,cols,k,lengths,ws", [
    (5, 4096, 2048, "full", 0),
    (5, 8000, 2048, "ragged", 0),
    (5, 16384, 2048, "full", 0),
    (6, 30001, 2048, "ragged", 0),
    (6, 32768, 10000, "full", 0),
    (9, 131072, 2048, "ragged", 1),
    (4, 200000, 2048, "ragged", 1),
    (4, 65536, 1003, "full", 1),
    (3, 40000, 7, "ragged", 1),
    (3, 50000, 12000, "full", 0),
    (2, 40000, 20000, "ragged", 0),
])
def test_launch_variants(rows, cols, k, lengths, ws):
    wl = W.topk_make(rows, cols, k=k, lengths=lengths, seed=cols + k)
    assert (R.dsaidx_topk_workspace_bytes(rows, cols, k) > 0) == (cols > 32768)
    out = run_topk(wl.logits, k, wl.lengths)
    check(out, wl.logits, k, wl.lengths)


def test_two_phase_row_lengths():
    """Rows of the chunk + merge path that end inside the first chunk, exactly at
    a chunk edge, a few logits into a chunk, and rows of at most k logits."""
    rows, cols, k = 10, 70000, 2048
    rng = np.random.default_rng(21)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    lens = np.array([0, 5, 2048, 2049, 16383, 16384, 16385, 32768 + 3, 69999, 70000], np.int32)
    out = run_topk(x, k, lens)
    check(out, x, k, lens)


def test_workspace_reuse_and_too_small():
    rows, cols, k = 4, 100000, 2048
    wl = W.topk_make(rows, cols, k=k, lengths="ragged", seed=5)
    need = R.dsaidx_topk_workspace_bytes(rows, cols, k)
    assert need > 0
    d = torch.from_numpy(wl.logits).cuda()
    dl = torch.from_numpy(wl.lengths).cuda()
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")
    out = torch.empty((rows, k), dtype=torch.int32, device="cuda")
    for _ in range(2):
        R.dsaidx_topk_per_row(d, k, out, dl, workspace=ws)
        torch.cuda.synchronize()
        check(out.cpu().numpy(), wl.logits, k, wl.lengths)
    with pytest.raises(R.DsaidxError):
        R.dsaidx_topk_per_row(d, k, out, dl, workspace=ws[: need - 16])


def test_long_rows_chunk_edges_and_extreme_k():
    """Rows longer than 32768 logits: lengths on and around 4096-logit chunk
    edges, k = 1 and k = len - 1."""
    rows, cols = 8, 40960
    rng = np.random.default_rng(31)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    lens = np.array([4095, 4096, 4097, 8192, 32768, 32769, 40959, 40960], np.int32)
    for k in (1, 2048, 4094):
        out = run_topk(x, k, lens)
        check(out, x, k, lens)
    k = 40959
    out = run_topk(x[:1], k, None)
    check(out, x[:1], k, None)


def test_long_rows_degenerate_values():
    """Long rows whose k-th value sits in one crowded bin: every logit equal,
    a few distinct values, -inf masses and values in a narrow range."""
    rows, cols, k = 5, 50000, 2048
    rng = np.random.default_rng(41)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x[0] = 1.5
    x[1] = np.round(x[1])
    x[2] = -np.inf
    x[2, 7000:9500] = rng.standard_normal(2500).astype(np.float32)
    x[3] = (1.0 + 0.1 * rng.random(cols)).astype(np.float32)
    x[4, ::3] = -0.0
    x[4, 1::3] = 0.0
    out = run_topk(x, k)
    check(out, x, k)


def test_split_path_under_graph_replay():
    """The four dispatches of a long-row call captured in one HIP graph and
    replayed, with new logits copied in and eager calls between replays;
    every replay is checked."""
    rows, cols, k = 6, 50000, 2048
    d = torch.empty((rows, cols), dtype=torch.float32, device="cuda")
    dl = torch.empty(rows, dtype=torch.int32, device="cuda")
    out = torch.empty((rows, k), dtype=torch.int32, device="cuda")
    ws = torch.empty(R.dsaidx_topk_workspace_bytes(rows, cols, k), dtype=torch.uint8, device="cuda")
    wl0 = W.topk_make(rows, cols, k=k, lengths="ragged", seed=50)
    d.copy_(torch.from_numpy(wl0.logits))
    dl.copy_(torch.from_numpy(wl0.lengths))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        R.dsaidx_topk_per_row(d, k, out, dl, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        R.dsaidx_topk_per_row(d, k, out, dl, workspace=ws)
    other = torch.empty((rows, k), dtype=torch.int32, device="cuda")
    for rep in range(4):
        wl = W.topk_make(rows, cols, k=k, lengths="ragged", seed=51 + rep)
        d.copy_(torch.from_numpy(wl.logits))
        dl.copy_(torch.from_numpy(wl.lengths))
        g.replay()
        torch.cuda.synchronize()
        check(out.cpu().numpy(), wl.logits, k, wl.lengths)
        R.dsaidx_topk_per_row(d[:3], k, other[:3], dl[:3], workspace=ws)   # eager, same workspace
        torch.cuda.synchronize()
        check(other[:3].cpu().numpy(), wl.logits[:3], k, wl.lengths[:3])


@pytest.mark.parametrize("shift", [5.0, -5.0])
def test_rows_that_mislead_a_strided_sample(shift):
    """Logits at every fourth column drawn far below (or above) the rest: an
    estimate of the k-th largest taken from those columns misses, and the
    exact selection must still come out."""
    rows, k = 6, 2048
    for cols in (4096, 8192, 16384, 32768):
        rng = np.random.default_rng(cols)
        x = rng.standard_normal((rows, cols)).astype(np.float32)
        x[:, 0::4] -= shift
        x[:, 1::4] += shift
        lens = np.array([cols, cols - 1, cols // 2 + 3, k + 1, k + 5, 3 * cols // 4], np.int32)
        out = run_topk(x, k, lens)
        check(out, x, k, lens)


def test_long_rows_threshold_bin_over_list_capacity():
    """Rows longer than 32768 whose threshold bin (same top 11 key bits) holds
    more logits than the per-row candidate list takes (max(4096, cols / 16)):
    the selection finishes by re-reading the row."""
    rows, cols, k = 4, 65536, 2048
    rng = np.random.default_rng(61)
    x = (-5.0 + 0.1 * rng.standard_normal((rows, cols))).astype(np.float32)
    for r in range(rows):
        idx = rng.permutation(cols)
        x[r, idx[:5000]] = (1.0 + 0.2 * rng.random(5000)).astype(np.float32)   # one top-11-bit bin
        x[r, idx[5000:5100]] = (3.0 + rng.random(100)).astype(np.float32)
    lens = np.array([cols, cols - 7, 60001, 40000], np.int32)
    out = run_topk(x, k, lens)
    check(out, x, k, lens)


@pytest.mark.parametrize("seed", range(12))
def test_random_shapes(seed):
    """Seeded random draws over rows, columns, k, lengths, row padding and
    value mixes, across the row kernel's shapes and the split-row path."""
    rng = np.random.default_rng(7000 + seed)
    cols = int(rng.choice([1, 100, 2049, 4096, 5000, 8192, 12345, 16384, 20000, 32768, 33000,
                           70000]))
    rows = int(rng.integers(1, max(2, min(40, 2_000_000 // max(cols, 1)))))
    k = int(rng.choice([1, 7, 64, 2048, max(1, cols // 2), cols + 3]))
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    mix = int(rng.integers(4))
    if mix == 1:
        x = np.round(x * 4) / 4                                  # heavy ties
    elif mix == 2:
        x[rng.random((rows, cols)) < 0.05] = -np.inf             # masked keys
        x[rng.random((rows, cols)) < 0.001] = np.inf
    elif mix == 3:
        x = (100.0 + 1e-3 * x).astype(np.float32)                # narrow range
    lengths = None
    if rng.integers(2):
        lengths = rng.integers(-2, cols + 3, rows).astype(np.int32)
    out = run_topk(x, k, lengths, pad_cols=int(rng.choice([0, 1, 7])))
    check(out, x, k, lengths)
