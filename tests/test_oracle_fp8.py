"""Pins of the oracle's OCP FP8 E4M3FN encoder (CPU only).

The encoder is written from the format definition; these tests tie it to
things outside itself: the 256-code table it must invert, the midpoint rule,
a brute-force nearest-code search, and torch's own float8_e4m3fn conversion
over every fp32 bit pattern.  Parity with a single fp32 -> fp8 rounding step is
what the sglang PR "Fuse the DSA indexer Q/K rope + quant + K-cache write"
(section Accuracy) relies on.
"""
import math

import numpy as np
import pytest
import torch

NAN_CODES = (0x7F, 0xFF)


def _table(oracle_lib):
    return np.array([oracle_lib.fp8_decode(c) for c in range(256)], dtype=np.float64)


def test_decode_table_known_values(oracle_lib):
    t = _table(oracle_lib)
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x08] == 2.0 ** -6          # smallest normal
    assert t[0x01] == 2.0 ** -9          # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9      # largest subnormal
    assert t[0x38] == 1.0                # exponent field 7 = bias
    assert t[0x77] == 240.0 and t[0x71] == 144.0
    assert t[0x00] == 0.0 and math.copysign(1.0, t[0x80]) == -1.0
    assert math.isnan(t[0x7F]) and math.isnan(t[0xFF])
    finite = [c for c in range(256) if c not in NAN_CODES]
    pos = sorted(t[c] for c in finite if c < 0x80)
    assert len(set(pos)) == 127 and pos == sorted(set(pos))


def test_roundtrip_every_code(oracle_lib):
    for c in range(256):
        if c in NAN_CODES:
            continue
        v = oracle_lib.fp8_decode(c)
        assert oracle_lib.fp8_encode(v) == c, hex(c)


def test_midpoints_go_to_even_code(oracle_lib):
    t = _table(oracle_lib)
    for c in range(0x00, 0x7E):
        lo, hi = t[c], t[c + 1]
        mid = np.float32((lo + hi) / 2)        # exact: needs 5 significant bits
        assert float(mid) == (lo + hi) / 2
        even = c if (c & 1) == 0 else c + 1
        assert oracle_lib.fp8_encode(float(mid)) == even
        assert oracle_lib.fp8_encode(-float(mid)) == even | 0x80
        below = float(np.nextafter(mid, np.float32(-np.inf)))
        above = float(np.nextafter(mid, np.float32(np.inf)))
        assert oracle_lib.fp8_encode(below) == c
        assert oracle_lib.fp8_encode(above) == c + 1


def test_saturation_and_signed_zero(oracle_lib):
    assert oracle_lib.fp8_encode(448.0) == 0x7E
    assert oracle_lib.fp8_encode(449.0) == 0x7E
    assert oracle_lib.fp8_encode(1e30) == 0x7E
    assert oracle_lib.fp8_encode(float("inf")) == 0x7E
    assert oracle_lib.fp8_encode(-1e30) == 0xFE
    assert oracle_lib.fp8_encode(0.0) == 0x00
    assert oracle_lib.fp8_encode(-0.0) == 0x80
    assert oracle_lib.fp8_encode(-1e-10) == 0x80
    assert oracle_lib.fp8_encode(2.0 ** -10) == 0x00       # tie between 0 and 2^-9 -> even
    assert oracle_lib.fp8_encode(3 * 2.0 ** -10) == 0x02   # tie between 1 and 2 (x 2^-9)


def test_encoder_ties_on_every_binade(oracle_lib):
    """Every exact midpoint between neighbouring codes, positive and negative,
    in one vectorised call: ties go to the even code."""
    t = _table(oracle_lib)
    c = np.arange(0x7E)
    mids = ((t[c] + t[c + 1]) / 2).astype(np.float32)
    even = np.where(c % 2 == 0, c, c + 1).astype(np.uint8)
    assert np.array_equal(oracle_lib.fp8_encode_array(mids), even)
    assert np.array_equal(oracle_lib.fp8_encode_array(-mids), even | 0x80)


def test_brute_force_nearest_code(oracle_lib):
    """Nearest code by scanning the whole table, ties to the even code."""
    t = _table(oracle_lib)
    codes = np.array([c for c in range(0x7F)], dtype=np.int64)   # 0x00..0x7E
    vals = t[codes]
    rng = np.random.default_rng(7)
    mags = np.concatenate([
        rng.uniform(0, 448, 4000),
        np.exp2(rng.uniform(-14, 9, 4000)),
        rng.uniform(0, 2.0 ** -5, 2000),
    ]).astype(np.float32)
    mags = np.minimum(mags, np.float32(448))
    signs = rng.choice([-1.0, 1.0], mags.size).astype(np.float32)
    for m, sg in zip(mags, signs):
        d = np.abs(vals - float(m))
        best = np.flatnonzero(d == d.min())
        if best.size == 2:
            pick = codes[best[0]] if codes[best[0]] % 2 == 0 else codes[best[1]]
        else:
            pick = codes[best[0]]
        v = float(m) * float(sg)
        want = int(pick) | (0x80 if sg < 0 else 0)
        assert oracle_lib.fp8_encode(v) == want, (v, hex(want))


def _compare_with_torch(oracle_lib, f):
    ours = oracle_lib.fp8_encode_array(f, nthreads=max(1, min(8, oracle_lib.max_threads())))
    ref = torch.from_numpy(f).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    nan_in = np.isnan(f)
    assert np.all((ours[nan_in] & 0x7F) == 0x7F)      # NaN in -> a NaN code out on both sides
    return int(np.count_nonzero((ours != ref) & ~nan_in))


@pytest.mark.parametrize("sign", [0, 1])
def test_every_in_range_fp32_pattern_matches_torch(oracle_lib, sign):
    """Every fp32 bit pattern with |v| <= 448 (where rounding happens), one
    sign per case: oracle == torch's float8_e4m3fn conversion."""
    limit = int(np.float32(448.0).view(np.uint32)) + 1
    chunk = 1 << 25
    base = np.arange(chunk, dtype=np.uint32)
    bits = np.empty(chunk, dtype=np.uint32)
    bad = 0
    for s in range(0, limit, chunk):
        n = min(chunk, limit - s)
        np.add(base[:n], np.uint32(s | (sign << 31)), out=bits[:n])
        bad += _compare_with_torch(oracle_lib, bits[:n].view(np.float32))
    assert bad == 0


def test_out_of_range_fp32_patterns_saturate_like_torch(oracle_lib):
    """A strided sweep (step 251, every exponent and sign) of the patterns
    with |v| > 448, NaN and infinity included: both sides saturate."""
    lo = int(np.float32(448.0).view(np.uint32)) + 1
    pos = np.arange(lo, 1 << 31, 251, dtype=np.uint32)
    bits = np.concatenate([pos, pos | np.uint32(1 << 31)])
    assert _compare_with_torch(oracle_lib, bits.view(np.float32)) == 0
