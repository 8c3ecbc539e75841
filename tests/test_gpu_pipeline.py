"""The indexer end to end on the GPU: the fused prep call writes the query
codes, folded gates and index-K cache; the index logits read them back over
the cache slots the call wrote, with causal lengths; the top-k per row
selects from those logits.  Each stage is checked against its oracle on the
device's own inputs to that stage (prep: the acceptance rules; logits: the
matrix unit's bound; top-k: the exact selected values), and the selection is
then checked against the all-oracle chain: every key the device picked must
score, under the oracle's logits, no lower than the oracle's k-th largest
less the logits tolerance, and every key it left out no higher than that
value plus the tolerance."""
import numpy as np
import pytest
import torch

import oracle
import rope_fp8_quant_amd as R
from gpu_util import DeviceCase, check_k, check_q, logits_bound, split_paged
from oracle import logits as LG
from oracle import topk as TK
from rope_fp8_quant_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


@pytest.mark.parametrize("page_size", [0, 16])
def test_prep_logits_topk_chain(page_size):
    T, H, S, k = 300, 64, 1024, 64
    print("\n[case] pipeline T=%d H=%d S=%d k=%d page_size=%d" % (T, H, S, k, page_size), flush=True)
    wl = W.make(T, H, table_rows=4096, pos_mode="contiguous", pos_lo=100, num_slots=S,
                slot_mode="perm_prefix", seed=91 + page_size)
    flags = R.DSAIDX_K_PAGED_CACHE if page_size else 0
    c = DeviceCase(wl, k_flags=flags, page_size=page_size)
    c.run("fused")
    out = c.host()
    report = {}
    check_q(out, wl, report)
    check_k(out, wl, report, k_flags=flags, page_size=page_size)

    # index logits: key s is token s's cache row; token t sees keys 0..t
    slots = wl.out_cache_loc.astype(np.int64)
    lengths = np.arange(1, T + 1, dtype=np.int32)
    lo = torch.full((T, T), float("nan"), dtype=torch.float32, device="cuda")
    args = R.logits_args(c.q_fp8, c.w_out, c.k_cache, lo, k_scale=c.k_scale,
                         key_slots=torch.from_numpy(slots.astype(np.int32)).cuda(),
                         lengths=torch.from_numpy(lengths).cuda(), flags=flags,
                         page_size=page_size, num_slots=S if page_size else None)
    R.dsaidx_mqa_logits(args)
    torch.cuda.synchronize()
    got = lo.cpu().numpy()
    q8, w = out["q_fp8"], out["w_out"]
    if page_size:
        codes, scale = split_paged(out["k_cache"], page_size, S)
    else:
        codes, scale = out["k_cache"], out["k_scale"]
    want = LG.mqa_logits(q8, w, codes, scale, key_slots=slots, lengths=lengths)
    tol = logits_bound(q8, w, codes, scale, slots)
    valid = ~np.isnan(want)
    assert np.all(np.abs(got[valid] - want[valid]) <= tol[valid])
    assert np.all(np.isnan(got[~valid])), "entries past a row's length were written"

    # top-k over the device's logits: the exact selected values
    idx = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    R.dsaidx_topk_per_row(lo, k, idx, torch.from_numpy(lengths).cuda())
    torch.cuda.synchronize()
    sel = idx.cpu().numpy()
    top, count = TK.topk_values(got, k, lengths)
    for t in range(T):
        n = int(lengths[t])
        if n <= k:
            assert np.array_equal(sel[t], np.r_[np.arange(n), -np.ones(k - n, int)]), t
            continue
        assert np.unique(sel[t]).size == k and sel[t].min() >= 0 and sel[t].max() < n, t
        assert np.array_equal(np.sort(got[t, sel[t]])[::-1], top[t]), t

    # the selection against the all-oracle chain
    oq8, ow, _ = oracle.q_side(wl.q, wl.weights, wl.positions, wl.cos, wl.sin)
    okc = np.zeros((S, 128), np.uint8)
    oks = np.zeros(S, np.float32)
    oracle.k_side(wl.k, wl.gamma, wl.beta, wl.eps, wl.positions, wl.out_cache_loc, wl.cos, wl.sin,
                  okc, oks)
    ref = LG.mqa_logits(oq8, ow, okc, oks, key_slots=slots, lengths=lengths)
    # the oracle chain and the device chain differ by the logits arithmetic
    # (within tol) and by the effect of the rare one-code fp8 splits in the
    # prep outputs, which the oracle gives exactly as ref - want
    gap = np.where(valid, np.abs(ref - want) + tol, 0.0)
    assert np.all(np.abs(ref[valid] - got[valid]) <= gap[valid])
    kth = TK.kth_value(np.where(valid, ref, -np.inf).astype(np.float32), k, lengths)
    checked = 0
    for t in range(T):
        n = int(lengths[t])
        if n <= k:
            continue
        band = 2.0 * gap[t, :n].max()
        s = sel[t]
        assert np.all(ref[t, s] >= kth[t] - band), t
        rest = np.setdiff1d(np.arange(n), s)
        assert np.all(ref[t, rest] <= kth[t] + band), t
        checked += 1
    print("[parity] pipeline: %d query codes and %d key codes differ from the oracle chain; %d rows of "
          "top-%d checked against it" % (int(np.count_nonzero(oq8 != q8)),
                                         int(np.count_nonzero(okc[slots] != codes[slots, :128])),
                                         checked, k), flush=True)
