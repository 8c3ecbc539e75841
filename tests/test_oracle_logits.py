"""Pins of the index-logits oracle (oracle/logits.py).

Each check ties the oracle to a property of its definition rather than to a
retyped copy of it: the fold identity (the reason the reading holds), the
ReLU identity relu(x) - relu(-x) = x against a plain matrix product, key
permutation, linearity in the key scale, the length mask and a hand-computed
example."""
import numpy as np
import pytest

import oracle
from oracle import logits as LG
from rope_fp8_quant_amd import workloads as W


def _prep(T=6, H=8, S=40, seed=3):
    """A small prep workload through the oracle: folded gates, codes, and the
    unfolded pieces (raw gates, per-head exponents) for the fold identity."""
    wl = W.make(T, H, table_rows=512, num_slots=S, seed=seed)
    q8, w_out, q_scale = oracle.q_side(wl.q, wl.weights, wl.positions, wl.cos, wl.sin)
    k_cache = np.zeros((S, 128), np.uint8)
    k_scale = np.zeros(S, np.float32)
    oracle.k_side(wl.k, wl.gamma, wl.beta, wl.eps, wl.positions, np.arange(T), wl.cos, wl.sin,
                  k_cache, k_scale)
    rng = np.random.default_rng(seed)
    # fill the slots no token wrote with random codes and scales (no NaN codes)
    rest = np.arange(T, S)
    codes = rng.integers(0, 256, size=(len(rest), 128)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x00
    k_cache[rest] = codes
    k_scale[rest] = np.exp2(rng.integers(-12, -4, size=len(rest))).astype(np.float32)
    return wl, q8, w_out, q_scale, k_cache, k_scale


def test_fold_identity():
    """Scaling each head's dot by 2^e inside the ReLU and gating with the raw
    weight equals the folded form the oracle takes: the gate carries 2^e."""
    wl, q8, w_out, q_scale, k_cache, k_scale = _prep()
    got = LG.mqa_logits(q8, w_out, k_cache, k_scale)
    dots = LG.head_dots(q8, k_cache)                                   # [T, H, S]
    gates = (wl.weights.astype(np.uint32) << 16).view(np.float32)       # bf16 gates as fp32
    raw = (gates * np.float32(wl.weight_scale)).astype(np.float64)
    inside = np.maximum(dots * q_scale.astype(np.float64)[:, :, None], 0.0)
    want = np.einsum("th,ths->ts", raw, inside) * k_scale.astype(np.float64)[None, :]
    assert np.allclose(got, want, rtol=1e-12, atol=0.0)
    # w_out is exactly raw * 2^e in fp32, so the two agree to float64 rounding
    assert np.array_equal(w_out, (raw * q_scale).astype(np.float32))


def test_relu_identity_against_matrix_product():
    """relu(x) - relu(-x) = x: logits with every key negated (sign bit of each
    code flipped) subtracted from the plain ones leave a linear form that a
    plain matrix product gives."""
    wl, q8, w_out, q_scale, k_cache, k_scale = _prep(T=5, H=16, S=33, seed=7)
    neg = k_cache ^ np.uint8(0x80)
    diff = LG.mqa_logits(q8, w_out, k_cache, k_scale) - LG.mqa_logits(q8, w_out, neg, k_scale)
    dec = np.array([oracle.fp8_decode(c) for c in range(256)], np.float64)
    qw = np.einsum("th,thd->td", w_out.astype(np.float64), dec[q8])    # gate-weighted query sum
    want = (qw @ dec[k_cache].T) * k_scale.astype(np.float64)[None, :]
    assert np.allclose(diff, want, rtol=1e-12, atol=1e-300)


def test_key_slots_permute_columns_and_scale_is_linear():
    wl, q8, w_out, q_scale, k_cache, k_scale = _prep(T=4, H=8, S=50, seed=11)
    base = LG.mqa_logits(q8, w_out, k_cache, k_scale)
    perm = np.random.default_rng(0).permutation(50)[:37]
    assert np.array_equal(LG.mqa_logits(q8, w_out, k_cache, k_scale, key_slots=perm), base[:, perm])
    assert np.array_equal(LG.mqa_logits(q8, w_out, k_cache, 2.0 * k_scale), 2.0 * base)


def test_lengths_mask():
    wl, q8, w_out, q_scale, k_cache, k_scale = _prep(T=4, H=8, S=30, seed=13)
    base = LG.mqa_logits(q8, w_out, k_cache, k_scale)
    lens = np.array([0, 7, 30, 45])
    got = LG.mqa_logits(q8, w_out, k_cache, k_scale, lengths=lens)
    for t, n in enumerate(np.minimum(lens, 30)):
        assert np.array_equal(got[t, :n], base[t, :n])
        assert np.all(np.isnan(got[t, n:]))


def test_hand_example():
    """Two heads, one nonzero dimension: q = (+1, -1), k = 2, gates (0.5, 3),
    key scale 0.25.  Dots 2 and -2; ReLU 2 and 0; 0.5 * 2 = 1; times 0.25."""
    q8 = np.zeros((1, 2, 128), np.uint8)
    q8[0, 0, 5] = 0x38      # +1.0
    q8[0, 1, 5] = 0xB8      # -1.0
    k = np.zeros((1, 128), np.uint8)
    k[0, 5] = 0x40          # +2.0
    got = LG.mqa_logits(q8, np.array([[0.5, 3.0]], np.float32), k, np.array([0.25], np.float32))
    assert got.shape == (1, 1) and got[0, 0] == 0.25


@pytest.mark.parametrize("H", [1, 3, 16])
def test_all_negative_dots_give_zero(H):
    rng = np.random.default_rng(H)
    q8 = (rng.integers(0x08, 0x70, size=(2, H, 128))).astype(np.uint8)        # positive codes
    k = (rng.integers(0x08, 0x70, size=(9, 128)) | 0x80).astype(np.uint8)     # negative codes
    w = rng.standard_normal((2, H)).astype(np.float32)
    got = LG.mqa_logits(q8, w, k, np.ones(9, np.float32))
    assert np.all(got == 0.0)
