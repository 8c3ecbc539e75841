"""Pins of the oracle's page-interleaved index-K cache writer (CPU only).

The sglang PR "[AMD] [GLM5] Fuse the DSA indexer Q/K rope + quant + K-cache
write" (section Checklist) tests the K-cache writers in two paged layouts
without defining them.  The second layout used here: pages of page_size
slots, each page holding its page_size 128-byte code rows and then its
page_size fp32 scales.  The planar writer's result, moved by that address map
(restated below in numpy), must equal the paged writer's bytes, sentinel bytes
of untouched slots included.
"""
import numpy as np
import pytest

from rope_fp8_quant_amd import workloads as W

ROW = 128
SENT = 0xA5


def planar_then_rearranged(oracle_lib, wl, page, bf16_mode):
    S = wl.num_slots
    kc = np.full((S, ROW), SENT, np.uint8)
    ks = np.frombuffer(bytes([SENT]) * (4 * S), dtype=np.float32).copy()
    oracle_lib.k_side(wl.k, wl.gamma, wl.beta, wl.eps, wl.positions, wl.out_cache_loc,
                      wl.cos, wl.sin, kc, ks, wl.rope_dim, wl.style, bf16_mode)
    pages = []
    for p in range(S // page):
        pages.append(kc[p * page:(p + 1) * page].reshape(-1))
        pages.append(ks[p * page:(p + 1) * page].view(np.uint8))
    return np.concatenate(pages)


@pytest.mark.parametrize("bf16_mode", [0, 1, 2])
@pytest.mark.parametrize("page", [2, 16, 64])
def test_paged_equals_planar_under_the_address_map(oracle_lib, page, bf16_mode):
    wl = W.named(0)
    wl.out_cache_loc = wl.out_cache_loc.copy()
    wl.out_cache_loc[[3, 17]] = [-1, wl.num_slots]          # skipped entries
    want = planar_then_rearranged(oracle_lib, wl, page, bf16_mode)
    got = np.full(wl.num_slots * (ROW + 4), SENT, np.uint8)
    oracle_lib.k_side_paged(wl.k, wl.gamma, wl.beta, wl.eps, wl.positions, wl.out_cache_loc,
                            wl.cos, wl.sin, got, page, wl.num_slots, wl.rope_dim, wl.style,
                            bf16_mode)
    assert np.array_equal(got, want)
    # exactly the valid slots changed: 39 rows of 128 bytes plus their scales
    assert np.count_nonzero(got != SENT) <= 39 * (ROW + 4)
    assert np.count_nonzero(got != SENT) >= 39 * 4


def test_paged_rejects_a_page_size_that_does_not_divide(oracle_lib):
    wl = W.named(0)
    buf = np.zeros(wl.num_slots * (ROW + 4), np.uint8)
    with pytest.raises(ValueError):
        oracle_lib.k_side_paged(wl.k, wl.gamma, wl.beta, wl.eps, wl.positions,
                                wl.out_cache_loc, wl.cos, wl.sin, buf, 3, wl.num_slots)
