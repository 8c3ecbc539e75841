"""Pins of the oracle's scale rule, RoPE, LayerNorm, quantisation, head-gate
fold and index-K cache write (CPU only).

Each test ties the oracle to something other than itself: a hand-worked
fixture, a closed form, a library routine, an invariant, or brute force.
Operation sources: sglang PR "[AMD] [GLM5] Fuse the DSA indexer Q/K rope +
quant + K-cache write" (sections Motivation, Modifications, Accuracy) and vLLM
PR 47335 "Enable fused indexer-Q RoPE+quant kernel" (sections Summary and
Kernel-level evidence).
"""
import math
import os

import numpy as np
import pytest
import torch

from golden_util import load_hand_examples
from rope_fp8_quant_amd import workloads as W

ROW = 128


def bits(x):
    return np.asarray(x, dtype=np.float32).view(np.uint32)


def bf16(vals):
    return W.f32_to_bf16_bits(np.asarray(vals, dtype=np.float32))


def half_ulp_e4m3(m):
    """Half the E4M3 spacing at magnitude m (m in [0, 448])."""
    m = np.asarray(m, dtype=np.float64)
    k = np.floor(np.log2(np.maximum(m, 2.0 ** -6)))
    return 0.5 * np.where(m < 2.0 ** -6, 2.0 ** -9, np.exp2(k - 3))


# ----------------------------------------------------------- scale rule ----

BOUNDARY_TABLE = [  # (amax, e): hand-worked from "smallest e with amax <= 448*2^e"
    (448.0, 0), (float(np.nextafter(np.float32(448), np.float32(1e9))), 1),
    (224.0, -1), (225.0, 0), (1.75, -8), (3.5, -7), (0.4375, -10),
    (1.9220755, -7), (0.89766765, -8), (896.0, 1), (897.0, 2),
    (0.0, -22), (1e-4, -22), (1e-7, -22), (2.0 ** 100, 92),
]


@pytest.mark.parametrize("amax,e", BOUNDARY_TABLE)
def test_scale_boundary_table(oracle_lib, amax, e):
    assert oracle_lib.ue8m0_exponent(amax) == e


def test_scale_closed_form_mantissa_rule(oracle_lib):
    """For a normal floor-guarded amax = 1.f x 2^E the rule is
    e = E - 8 + [f > 0.75], since 448 = 1.75 x 2^8 (0x600000 = 0.75 x 2^23)."""
    rng = np.random.default_rng(11)
    a = np.exp2(rng.uniform(-14, 60, 20000)).astype(np.float32)
    a = np.concatenate([a, np.float32(1.75) * np.exp2(np.arange(-13, 40)).astype(np.float32)])
    a = np.concatenate([a, np.nextafter(a[-53:], np.float32(np.inf)),
                        np.nextafter(a[-53:], np.float32(0))])
    for v in a:
        g = max(float(v), float(np.float32(1e-4)))
        b = int(bits(g))
        E = (b >> 23) - 127
        want = E - 8 + (1 if (b & 0x7FFFFF) > 0x600000 else 0)
        assert oracle_lib.ue8m0_exponent(float(v)) == want, v
        # and the defining inequality, exactly in binary64
        assert g <= math.ldexp(448.0, want) and g > math.ldexp(448.0, want - 1)


# ---------------------------------------------------------- hand fixture ----

@pytest.mark.parametrize("ex", load_hand_examples(), ids=lambda r: r[0])
def test_hand_examples(oracle_lib, ex):
    name, style, pos, w, xs, e, codes, folded = ex
    cos, sin = W.rope_table(8, 64)
    x = np.zeros((1, 1, ROW), dtype=np.float32)
    for i, v in xs.items():
        x[0, 0, i] = v
    q = bf16(x)
    wts = bf16(np.array([[w]], dtype=np.float32))
    q8, wo, qs = oracle_lib.q_side(q, wts, np.array([pos]), cos, sin, 64, style)
    want = np.zeros(ROW, dtype=np.uint8)
    for i, c in codes.items():
        want[i] = c
    assert np.array_equal(q8[0, 0], want)
    assert qs[0, 0] == 2.0 ** e
    assert wo[0, 0] == np.float32(folded)


# ----------------------------------------------------------------- RoPE ----

def _rand_q(T, H, seed):
    rng = np.random.default_rng(seed)
    return bf16(rng.standard_normal((T, H, ROW)).astype(np.float32) * 3)


@pytest.mark.parametrize("style", [W.NEOX, W.INTERLEAVED])
@pytest.mark.parametrize("rope_dim", [64, 32, 128])
def test_rope_closed_form_complex_rotation(oracle_lib, style, rope_dim):
    """Each rotated pair equals (a + ib) * (c + is), computed in float64 from
    the same fp32 inputs, to within the three fp32 roundings."""
    T, H = 16, 4
    cos, sin = W.rope_table(512, rope_dim)
    q = _rand_q(T, H, 5)
    pos = np.random.default_rng(6).integers(0, 512, T)
    y, _ = oracle_lib.q_values(q, pos, cos, sin, rope_dim, style)
    x = W.bf16_bits_to_f32(q).astype(np.float64)
    half = rope_dim // 2
    i = np.arange(half)
    ia = i if style == W.NEOX else 2 * i
    ib = i + half if style == W.NEOX else 2 * i + 1
    c = cos[pos][:, None, :].astype(np.float64)
    s = sin[pos][:, None, :].astype(np.float64)
    z = (x[..., ia] + 1j * x[..., ib]) * (c + 1j * s)
    bound = 2.0 ** -23 * 1.5 * (np.abs(x[..., ia] * c) + np.abs(x[..., ib] * s)
                                + np.abs(x[..., ib] * c) + np.abs(x[..., ia] * s))
    assert np.all(np.abs(y[..., ia] - z.real) <= bound + 1e-30)
    assert np.all(np.abs(y[..., ib] - z.imag) <= bound + 1e-30)
    rest = np.setdiff1d(np.arange(ROW), np.concatenate([ia, ib]))
    assert np.array_equal(y[..., rest], x[..., rest].astype(np.float32))


def test_rope_position_zero_is_identity(oracle_lib):
    cos, sin = W.rope_table(4, 64)
    assert np.all(cos[0] == 1) and np.all(sin[0] == 0)
    q = _rand_q(3, 5, 9)
    y, _ = oracle_lib.q_values(q, np.zeros(3, np.int64), cos, sin)
    assert np.array_equal(bits(y), bits(W.bf16_bits_to_f32(q)))


def test_interleaved_is_permuted_neox_bitwise(oracle_lib):
    cos, sin = W.rope_table(300, 64)
    q = _rand_q(8, 3, 13)
    pos = np.arange(8) * 37
    perm = np.arange(ROW)
    perm[0:64:2] = np.arange(32)          # interleaved slot 2i  <- NeoX element i
    perm[1:64:2] = np.arange(32) + 32     # interleaved slot 2i+1 <- NeoX element i+32
    y_n, e_n = oracle_lib.q_values(q, pos, cos, sin, 64, W.NEOX)
    y_i, e_i = oracle_lib.q_values(np.ascontiguousarray(q[..., perm]), pos, cos, sin, 64,
                                   W.INTERLEAVED)
    assert np.array_equal(bits(y_i), bits(y_n[..., perm]))
    assert np.array_equal(e_i, e_n)


def test_rope_preserves_pair_norm(oracle_lib):
    cos, sin = W.rope_table(4096, 64)
    q = _rand_q(32, 8, 21)
    pos = np.random.default_rng(22).integers(0, 4096, 32)
    y, _ = oracle_lib.q_values(q, pos, cos, sin)
    x = W.bf16_bits_to_f32(q).astype(np.float64)
    r_in = x[..., :32] ** 2 + x[..., 32:64] ** 2
    r_out = y[..., :32].astype(np.float64) ** 2 + y[..., 32:64].astype(np.float64) ** 2
    cs = (cos[pos].astype(np.float64) ** 2 + sin[pos].astype(np.float64) ** 2)[:, None, :]
    assert np.allclose(r_out, r_in * cs, rtol=1e-6, atol=1e-12)


# ------------------------------------------------------------ LayerNorm ----

def test_layernorm_matches_torch_float64(oracle_lib):
    """Position 0 (identity rotation) isolates LayerNorm; torch's layer_norm in
    float64 is the library reference."""
    rng = np.random.default_rng(3)
    T = 64
    kf = rng.standard_normal((T, ROW)).astype(np.float32) * rng.uniform(0.01, 30, (T, 1)).astype(np.float32)
    kf += rng.uniform(-5, 5, (T, 1)).astype(np.float32)
    k = bf16(kf)
    g = (1 + 0.1 * rng.standard_normal(ROW)).astype(np.float32)
    b = (0.1 * rng.standard_normal(ROW)).astype(np.float32)
    cos, sin = W.rope_table(2, 64)
    y, _ = oracle_lib.k_values(k, g, b, 1e-6, np.zeros(T, np.int64), cos, sin)
    ref = torch.nn.functional.layer_norm(
        torch.from_numpy(W.bf16_bits_to_f32(k).astype(np.float64)), (ROW,),
        torch.from_numpy(g.astype(np.float64)), torch.from_numpy(b.astype(np.float64)),
        eps=1e-6).numpy()
    scale = np.abs(ref).max(axis=1, keepdims=True)
    assert np.all(np.abs(y - ref) <= 2e-6 * scale)


def test_bf16_writer_rounds_like_torch_bf16(oracle_lib):
    """The bf16-intermediate writer at position 0 (identity rotation) returns
    bf16(LayerNorm output); torch's float -> bfloat16 conversion (nearest,
    ties to even) is the library reference."""
    wl = W.named(1)
    z = np.zeros(wl.T, np.int64)
    n32, _ = oracle_lib.k_values(wl.k, wl.gamma, wl.beta, wl.eps, z, wl.cos, wl.sin)
    n16, _ = oracle_lib.k_values(wl.k, wl.gamma, wl.beta, wl.eps, z, wl.cos, wl.sin, bf16_mode=1)
    ref = torch.from_numpy(n32).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(bits(n16), bits(ref))


def test_bf16_round_once_is_bf16_of_the_fp32_value(oracle_lib):
    """The single-rounding reading of the unfused writer (bf16_mode 2) returns
    bf16(fp32 LayerNorm + RoPE value) at real positions: one rounding, after
    the rotation.  torch's float -> bfloat16 conversion is the library
    reference; a rounding before the rotation, or none, fails here."""
    for idx in (0, 2):
        wl = W.named(idx)
        args = (wl.k, wl.gamma, wl.beta, wl.eps, wl.positions, wl.cos, wl.sin, wl.rope_dim, wl.style)
        y32, _ = oracle_lib.k_values(*args)
        y16, _ = oracle_lib.k_values(*args, bf16_mode=2)
        ref = torch.from_numpy(y32).to(torch.bfloat16).to(torch.float32).numpy()
        assert np.array_equal(bits(y16), bits(ref)), wl.name


def test_bf16_writer_ties_go_to_even(oracle_lib):
    """A constant key row normalises to beta exactly, so beta set to exact bf16
    midpoints makes the writer's first rounding a tie (position 0: identity
    rotation, so the second rounding sees bf16 values and changes nothing).
    Ties go to the even bf16 value, as torch rounds."""
    k = W.f32_to_bf16_bits(np.full((1, ROW), 3.0, np.float32))
    mids = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(2 + 2 ** -7), -(2 + 3 * 2 ** -7)], np.float32)
    beta = np.resize(mids, ROW).astype(np.float32)
    cos, sin = W.rope_table(2, 64)
    y, _ = oracle_lib.k_values(k, np.ones(ROW, np.float32), beta, 1e-6, np.zeros(1, np.int64),
                               cos, sin, bf16_mode=1)
    want = np.resize(np.array([1.0, 1 + 2 ** -6, -2.0, -(2 + 2 ** -5)], np.float32), ROW)
    assert np.array_equal(y[0], want)
    assert np.array_equal(torch.from_numpy(beta).to(torch.bfloat16).to(torch.float32).numpy(), want)


def test_layernorm_constant_row_gives_beta(oracle_lib):
    k = bf16(np.full((3, ROW), 2.5, np.float32))
    g = np.linspace(0.5, 1.5, ROW).astype(np.float32)
    b = np.linspace(-0.3, 0.3, ROW).astype(np.float32)
    cos, sin = W.rope_table(2, 64)
    y, _ = oracle_lib.k_values(k, g, b, 1e-6, np.zeros(3, np.int64), cos, sin)
    assert np.array_equal(bits(y), bits(np.broadcast_to(b, (3, ROW))))


def test_layernorm_unit_affine_moments(oracle_lib):
    rng = np.random.default_rng(4)
    k = bf16(rng.standard_normal((16, ROW)).astype(np.float32) * 7 + 3)
    cos, sin = W.rope_table(2, 64)
    one, zero = np.ones(ROW, np.float32), np.zeros(ROW, np.float32)
    y, _ = oracle_lib.k_values(k, one, zero, 1e-6, np.zeros(16, np.int64), cos, sin)
    y = y.astype(np.float64)
    x = W.bf16_bits_to_f32(k).astype(np.float64)
    var = x.var(axis=1)
    assert np.all(np.abs(y.mean(axis=1)) < 1e-6)
    assert np.allclose(y.var(axis=1), var / (var + 1e-6), rtol=1e-5)


# --------------------------------------------------------- quantisation ----

def test_dequantised_values_within_half_ulp(oracle_lib):
    wl = W.named(0)
    y, e = oracle_lib.q_values(wl.q, wl.positions, wl.cos, wl.sin)
    q8, wo, qs = oracle_lib.q_side(wl.q, wl.weights, wl.positions, wl.cos, wl.sin)
    dec = np.array([oracle_lib.fp8_decode(c) for c in range(256)], dtype=np.float64)
    scale = np.exp2(e.astype(np.float64))[..., None]
    v = y.astype(np.float64) / scale
    err = np.abs(dec[q8] - v)
    assert np.all(err <= half_ulp_e4m3(np.abs(v)))
    m = np.abs(dec[q8]).max(axis=-1)
    assert np.all((m >= 224) & (m <= 448))
    assert np.array_equal(qs, np.exp2(e).astype(np.float32))


def test_zero_row_guard(oracle_lib):
    cos, sin = W.rope_table(16, 64)
    q = np.zeros((2, 3, ROW), np.uint16)
    w = bf16(np.array([[1.0, -3.0, 0.5], [2.0, 0.0, 8.0]], np.float32))
    q8, wo, qs = oracle_lib.q_side(q, w, np.array([5, 0]), cos, sin)
    assert np.all((q8 & 0x7F) == 0)      # zero magnitude; rotated zeros may carry a sign
    assert np.all(q8[1] == 0)            # position 0: identity rotation keeps +0
    assert np.all(qs == np.float32(2.0 ** -22))
    assert np.array_equal(wo, W.bf16_bits_to_f32(w) * np.float32(2.0 ** -22))


@pytest.mark.parametrize("ws", [1.0, 0.5, 0.125])
def test_fold_is_exact_power_of_two_scaling(oracle_lib, ws):
    wl = W.named(1)
    q8, wo, qs = oracle_lib.q_side(wl.q, wl.weights, wl.positions, wl.cos, wl.sin,
                                   weight_scale=ws)
    w = W.bf16_bits_to_f32(wl.weights)
    # exact: ws is a power of two and so is the scale
    assert np.array_equal(wo, (w * np.float32(ws)) * qs)
    assert np.all(np.log2(qs) == np.round(np.log2(qs)))


def test_weight_scale_general_value_order(oracle_lib):
    """weights_out = (w * weight_scale) * 2^e with fp32 rounding after the first product."""
    wl = W.named(0)
    ws = 0.0883883461356163  # 1/sqrt(128): not a power of two
    _, wo, qs = oracle_lib.q_side(wl.q, wl.weights, wl.positions, wl.cos, wl.sin,
                                  weight_scale=ws)
    w = W.bf16_bits_to_f32(wl.weights)
    assert np.array_equal(wo, (w * np.float32(ws)) * qs)


# ---------------------------------------------------------- cache write ----

def _k_call(oracle_lib, wl, k_cache, k_scale, bf16_mode=0):
    oracle_lib.k_side(wl.k, wl.gamma, wl.beta, wl.eps, wl.positions, wl.out_cache_loc,
                      wl.cos, wl.sin, k_cache, k_scale, wl.rope_dim, wl.style, bf16_mode)


def test_cache_touched_only_at_out_cache_loc(oracle_lib):
    wl = W.named(0)
    S = wl.num_slots
    kc = np.full((S, 136), 0xA5, np.uint8)          # padded row stride
    ks = np.full(S, np.nan, np.float32)
    _k_call(oracle_lib, wl, kc[:, :ROW], ks)
    touched = np.zeros(S, bool)
    touched[wl.out_cache_loc] = True
    assert np.all(kc[~touched] == 0xA5) and np.all(np.isnan(ks[~touched]))
    assert np.all(kc[:, ROW:] == 0xA5)              # row padding untouched
    y, e = oracle_lib.k_values(wl.k, wl.gamma, wl.beta, wl.eps, wl.positions, wl.cos, wl.sin)
    assert np.array_equal(ks[wl.out_cache_loc], np.exp2(e).astype(np.float32))
    codes = oracle_lib.fp8_encode_array(y * np.exp2(-e).astype(np.float32)[:, None])
    assert np.array_equal(kc[wl.out_cache_loc, :ROW], codes)


def test_cache_skips_out_of_range_slots(oracle_lib):
    wl = W.named(0, T=6)
    wl.out_cache_loc = np.array([-1, 5, wl.num_slots, 7, -100, 2 ** 40], np.int64)
    S = wl.num_slots
    kc = np.full((S, ROW), 0xA5, np.uint8)
    ks = np.full(S, -1.0, np.float32)
    _k_call(oracle_lib, wl, kc, ks)
    changed = np.flatnonzero(np.any(kc != 0xA5, axis=1) | (ks != -1.0))
    assert changed.tolist() == [5, 7]


def round_once_writer_vs_fp32(oracle_lib, wl):
    """Both K-cache writers on one workload, the unfused one read as a single
    bf16 rounding before the quantisation (bf16_mode 2).  Returns the fp32
    writer's values, exponents and codes, the bf16 writer's exponents and
    codes, and the rows whose exponent a bf16 rounding of the row max can
    lower: the fp32 max lies above 448 * 2^(e-1) and rounds onto it (448 * 2^k
    is a bf16 value and rounding is monotone, so no other row can move)."""
    args = (wl.k, wl.gamma, wl.beta, wl.eps, wl.positions, wl.cos, wl.sin, wl.rope_dim, wl.style)
    y32, e32 = oracle_lib.k_values(*args)
    y16, e16 = oracle_lib.k_values(*args, bf16_mode=2)
    c32 = oracle_lib.fp8_encode_array(y32 * np.exp2(-e32).astype(np.float32)[:, None])
    c16 = oracle_lib.fp8_encode_array(y16 * np.exp2(-e16).astype(np.float32)[:, None])
    amax = np.abs(y32).max(axis=1).astype(np.float32)
    amax16 = torch.from_numpy(amax).to(torch.bfloat16).to(torch.float32).numpy()
    edge = (448.0 * np.exp2(e32 - 1.0)).astype(np.float32)
    movable = (amax > edge) & (amax16 == edge)
    return y32, e32, c32, e16, c16, movable


@pytest.mark.parametrize("idx", [0, 1, 2, 3])
def test_two_k_cache_writers_round_once(oracle_lib, idx, capsys):
    """The two-writer comparison of the sglang PR (section Accuracy) with the
    unfused writer read as one bf16 rounding of the finished fp32 value.

    Pinned, on every row whose ue8m0 scale the two writers share: each code
    differs by at most one step (a bf16 rounding moves a value by at most 2^-9
    of itself, less than half an fp8 step), and the single-step writer is never
    farther from the fp32 value.  The scales are identical except on exactly
    the rows whose fp32 max rounds down onto a scale boundary, where the bf16
    writer's exponent is one lower.  On the 41-token workload (the page's
    41 x 128 element count) no row is such a row, and the page's observation --
    identical scales, codes one step apart, the fused writer closer -- holds.
    The number of differing codes is data dependent and only printed."""
    wl = W.named(idx)
    y32, e32, c32, e16, c16, movable = round_once_writer_vs_fp32(oracle_lib, wl)
    assert np.array_equal(e16 != e32, movable)
    assert np.all(e16[movable] == e32[movable] - 1)
    if idx == 0:
        assert not movable.any()
    same = ~movable
    ordv = lambda x: np.where(x & 0x80, -(x & 0x7F).astype(int), (x & 0x7F).astype(int))
    diff = np.abs(ordv(c32[same]) - ordv(c16[same]))
    assert diff.max(initial=0) <= 1
    dec = np.array([oracle_lib.fp8_decode(c) for c in range(256)], dtype=np.float64)
    ref = y32[same].astype(np.float64) * np.exp2(-e32[same].astype(np.float64))[:, None]
    assert np.all(np.abs(dec[c32[same]] - ref) <= np.abs(dec[c16[same]] - ref))
    with capsys.disabled():
        print("\n[two K-cache writers, round once] %s: %d of %d codes differ, each by one code; "
              "%d of %d rows change scale (fp32 max rounds onto a boundary)"
              % (wl.name, np.count_nonzero(diff), diff.size, int(movable.sum()), wl.T))


def test_two_k_cache_writers(oracle_lib, capsys):
    """The two-writer comparison of the sglang PR (section Accuracy) on the
    41 x 128 K values of the 41-token workload: the unfused writer read as
    rounding at both kernel boundaries (bf16_mode 1) vs the single-step fp32
    writer.

    Pinned: the ue8m0 scales are identical; the single-step writer is never
    farther from the fp32 value; the bf16 writer's deviation stays within the
    error of its two bf16 roundings (inputs of the rotation, then its output).
    Not pinned (data dependent): the number of differing codes, and the page's
    "each by exactly one code" -- on this data a few elements sit where the
    rotation cancels (a*c ~ b*s), so the input rounding moves them by more
    than one fp8 step.  Counts are printed, not asserted."""
    wl = W.named(0)
    args = (wl.k, wl.gamma, wl.beta, wl.eps)
    y32, e32 = oracle_lib.k_values(*args, wl.positions, wl.cos, wl.sin)
    y16, e16 = oracle_lib.k_values(*args, wl.positions, wl.cos, wl.sin, bf16_mode=1)
    n32, _ = oracle_lib.k_values(*args, np.zeros(wl.T, np.int64), wl.cos, wl.sin)  # LayerNorm only
    assert np.array_equal(e32, e16)
    inv = np.exp2(-e32).astype(np.float32)[:, None]
    c32 = oracle_lib.fp8_encode_array(y32 * inv)
    c16 = oracle_lib.fp8_encode_array(y16 * inv)
    dec = np.array([oracle_lib.fp8_decode(c) for c in range(256)], dtype=np.float64)
    ref = y32.astype(np.float64) * inv
    assert np.all(np.abs(dec[c32] - ref) <= np.abs(dec[c16] - ref))

    # error model of the bf16 writer (NeoX, rope_dim 64)
    c = wl.cos[wl.positions].astype(np.float64)
    sn = wl.sin[wl.positions].astype(np.float64)
    a, b = n32[:, :32].astype(np.float64), n32[:, 32:64].astype(np.float64)
    u = 2.0 ** -8                                  # bf16 unit roundoff
    rot = np.concatenate([np.abs(a * c) + np.abs(b * sn), np.abs(b * c) + np.abs(a * sn)], axis=1)
    bound = np.concatenate([u * rot + u * np.abs(y32[:, :64]),
                            u * np.abs(y32[:, 64:]) + 1e-30], axis=1) * (1 + 2.0 ** -6)
    bound[:, :64] += 4 * 2.0 ** -24 * rot            # fp32 roundings inside the rotation
    assert np.all(np.abs(y16.astype(np.float64) - y32) <= bound)

    ordv = lambda x: np.where(x & 0x80, -(x & 0x7F).astype(int), (x & 0x7F).astype(int))
    diff = np.abs(ordv(c32) - ordv(c16))
    with capsys.disabled():
        print("\n[two K-cache writers] %d of %d codes differ (%d by one code, %d by more); "
              "max %d codes" % (np.count_nonzero(diff), diff.size,
                                np.count_nonzero(diff == 1), np.count_nonzero(diff > 1),
                                diff.max()))
