"""Pins of the projection oracle (oracle/proj.py), CPU only.

The oracle is numpy's float64 matrix product of bf16 inputs followed by a
rounding to bf16.  Pinned against what does not depend on it:
  - one-hot rows pick one weight column exactly (catches a transposed weight,
    a swapped key / gate split, a wrong column);
  - exact rational sums and an independent rational round-to-nearest-even on a
    small case (catches a dropped term, a different rounding rule);
  - bf16 midpoints built on purpose go to the even neighbour;
  - scaling the hidden states by a power of two scales every output.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import proj as P
from rope_fp8_quant_amd import workloads as W

ROW = 128


def bf16(a):
    return W.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def f64(bits):
    return P.bf16_bits_to_f64(bits)


def exact_bf16_bits(v: Fraction) -> int:
    """Round a rational to the nearest bf16 with ties to the even significand,
    by exact arithmetic: find e with 2^7 <= |v| / 2^e < 2^8, round |v| / 2^e to
    an integer (half to even), rescale, then take the float32 bits."""
    if v == 0:
        return 0
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length() - 8
    while a / Fraction(2) ** e >= 256:
        e += 1
    while a / Fraction(2) ** e < 128:
        e -= 1
    s = a / Fraction(2) ** e
    n = s.numerator // s.denominator
    rem = s - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = np.float32(float(Fraction(n) * Fraction(2) ** e))
    return sign | int(val.view(np.uint32) >> 16)


def test_one_hot_rows_pick_a_weight_column():
    rng = np.random.default_rng(1)
    T, d, H = 6, 96, 10
    wb = bf16(rng.standard_normal((ROW + H, d)))
    cols = np.array([0, 5, 17, 63, 64, 95])
    scale = np.array([1.0, 2.0, 0.5, -1.0, 4.0, 0.25])
    x = np.zeros((T, d), np.float32)
    x[np.arange(T), cols] = scale
    k_bits, g_bits = P.projection(bf16(x), wb)
    w = f64(wb)
    want = w[:, cols].T * scale[:, None]
    assert np.array_equal(f64(k_bits), want[:, :ROW])
    assert np.array_equal(f64(g_bits), want[:, ROW:])
    assert k_bits.shape == (T, ROW) and g_bits.shape == (T, H)


def test_exact_rational_sums_and_rounding():
    rng = np.random.default_rng(2)
    T, d, H = 3, 64, 8
    xb = bf16(rng.standard_normal((T, d)))
    wb = bf16(rng.standard_normal((ROW + H, d)) * 0.125)
    k_bits, g_bits = P.projection(xb, wb)
    got = np.concatenate([k_bits, g_bits], axis=1)
    xf = [[Fraction(float(v)) for v in row] for row in f64(xb)]
    wf = [[Fraction(float(v)) for v in row] for row in f64(wb)]
    for t in range(T):
        for n in range(ROW + H):
            exact = sum(a * b for a, b in zip(xf[t], wf[n]))
            assert int(got[t, n]) == exact_bf16_bits(exact), (t, n)


def test_midpoints_go_to_even():
    d, H = 64, 4
    x = np.zeros((4, d), np.float32)
    x[:, 0] = 1.0
    x[:, 1] = 2.0 ** -8
    w = np.zeros((ROW + H, d), np.float32)
    # output column n: 1 * w[n, 0] + 2^-8 * w[n, 1]
    w[0, 0], w[0, 1] = 1.0, 1.0                    # 1 + 2^-8: midpoint of 1 and 1 + 2^-7 -> 1
    w[1, 0], w[1, 1] = 1.0 + 2.0 ** -7, 1.0        # 1 + 3 * 2^-8 -> 1 + 2^-6 (even)
    w[2, 0], w[2, 1] = -1.0, -1.0                  # -(1 + 2^-8) -> -1
    w[3, 0], w[3, 1] = 1.0, 3.0                    # 1 + 3 * 2^-8 again, other split
    w[ROW, 0], w[ROW, 1] = 2.0, 2.0                # 2 + 2^-7: midpoint of 2 and 2 + 2^-6 -> 2
    # just above a midpoint, by less than fp32 resolves: 1 + 2^-8 + 2^-30 -> 1 + 2^-7 (an
    # intermediate fp32 rounding would land on the midpoint and then go to 1)
    x[:, 2] = 2.0 ** -30
    w[4, 0], w[4, 1], w[4, 2] = 1.0, 1.0, 1.0
    k_bits, g_bits = P.projection(bf16(x), bf16(w))
    assert f64(k_bits)[0, :5].tolist() == [1.0, 1.0 + 2.0 ** -6, -1.0, 1.0 + 2.0 ** -6, 1.0 + 2.0 ** -7]
    assert f64(g_bits)[0, 0] == 2.0


def test_power_of_two_scaling_and_sign():
    rng = np.random.default_rng(3)
    xb = bf16(rng.standard_normal((5, 128)))
    wb = bf16(rng.standard_normal((ROW + 16, 128)) / 8)
    k1, g1 = P.projection(xb, wb)
    k2, g2 = P.projection(bf16(f64(xb) * 4.0), wb)
    k3, g3 = P.projection(bf16(-f64(xb)), wb)
    assert np.array_equal(f64(k2), 4.0 * f64(k1)) and np.array_equal(f64(g2), 4.0 * f64(g1))
    assert np.array_equal(f64(k3), -f64(k1)) and np.array_equal(f64(g3), -f64(g1))


@pytest.mark.parametrize("v", [1.0, 3.0, -1.5, 1.0 + 2.0 ** -7, 255.0, 2.0 ** -40, 0.0])
def test_representable_values_round_to_themselves(v):
    assert f64(P.round_to_bf16_bits(np.array([v])))[0] == v
