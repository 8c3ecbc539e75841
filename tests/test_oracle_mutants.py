"""Planted mistakes in the oracle must fail its pins (CPU only).

Each case copies the oracle source, plants one plausible mistake (a flipped
sign, a transposed operand, a wrong index, a dropped term, an off-by-one
boundary, a different rounding rule), builds it, and runs the pin tests
against that build in a subprocess (ORACLE_LIB points the oracle loader at
it).  The pins pass on the real oracle, so each mutant must make at least one
of them fail.  The exhaustive fp32 sweeps are left out to keep this quick.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "dsaidx_oracle.c")
PIN_TESTS = ["tests/test_oracle_math.py", "tests/test_oracle_fp8.py", "tests/test_oracle_paged.py"]

MUTANTS = [
    ("rope_sign", "y[ia] = ac - bs;", "y[ia] = ac + bs;"),
    ("rope_transposed_operand", "float bs = b * s[i];", "float bs = b * c[i];"),
    ("rope_angle_index", "float bc = b * c[i];", "float bc = b * c[i / 2];"),
    ("rope_pair_index", "int ib = (style == 0) ? i + half : 2 * i + 1;",
     "int ib = (style == 0) ? i + half : 2 * i + 1 - (i > 0);"),
    ("q_position_ignored", "const float* c = cos_t + p * rs;", "const float* c = cos_t + 0 * rs;"),
    ("ln_mean_divisor", "float mu = (float)(s1 / ROW);", "float mu = (float)(s1 / (ROW - 1));"),
    ("ln_variance_divisor", "float var = (float)(s2 / ROW);", "float var = (float)(s2 / (ROW - 1));"),
    ("ln_eps_outside_sqrt", "(float)(1.0 / sqrt((double)var + (double)eps));",
     "(float)(1.0 / sqrt((double)var) + (double)eps);"),
    ("ln_beta_dropped", "n[i] = dg + b[i];", "n[i] = dg;"),
    ("ln_gamma_dropped", "float dg = dn * g[i];", "float dg = dn;"),
    ("scale_boundary", "while (a <= ldexp(FP8_MAX, e - 1)) e--;", "while (a < ldexp(FP8_MAX, e - 1)) e--;"),
    ("scale_floor_dropped", "float ag = (amax > AMAX_FLOOR) ? amax : AMAX_FLOOR;",
     "float ag = (amax > 0.0f) ? amax : AMAX_FLOOR;"),
    ("encode_round_half_up", "double q = nearbyint(a / quantum);", "double q = floor(a / quantum + 0.5);"),
    ("encode_saturates_to_nan", "if (a >= FP8_MAX) return (uint8_t)(sign | 0x7E);",
     "if (a >= FP8_MAX) return (uint8_t)(sign | 0x7F);"),
    ("encode_subnormal_boundary", "(a == 0.0 || E < -6)", "(a == 0.0 || E < -7)"),
    ("encode_sign_dropped", "uint8_t sign = signbit(v) ? 0x80 : 0x00;", "uint8_t sign = (v < 0) ? 0x80 : 0x00;"),
    ("fold_weight_scale_dropped", "w_out[t * H + h] = ws * sc;", "w_out[t * H + h] = wv * sc;"),
    ("cache_ignores_slot", "encode_row(y + t * ROW, e[t], k_cache + slot * row_stride);",
     "encode_row(y + t * ROW, e[t], k_cache + t * row_stride);"),
    ("bf16_round_half_up", "u += 0x7FFFu + lsb;", "u += 0x8000u + 0 * lsb;"),
    ("bf16_once_also_before_rope", "if (bf16_mode == 1) /* the LayerNorm kernel's bf16 output */",
     "if (bf16_mode >= 1) /* the LayerNorm kernel's bf16 output */"),
    ("bf16_once_skipped", "if (bf16_mode == 1 || bf16_mode == 2)", "if (bf16_mode == 1)"),
    ("paged_scale_offset", "memcpy(page + page_size * ROW + off * (int64_t)sizeof(float), &sc, sizeof sc);",
     "memcpy(page + page_size * ROW + (page_size - 1 - off) * (int64_t)sizeof(float), &sc, sizeof sc);"),
]


def test_every_mutation_applies_once():
    src = open(SRC).read()
    for name, old, new in MUTANTS:
        assert src.count(old) == 1, name


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new):
    src = open(SRC).read().replace(old, new)
    mutant_c = tmp_path / "dsaidx_oracle.c"
    mutant_c.write_text(src)
    lib = oracle.build(sources=[str(mutant_c)], out_path=str(tmp_path / "libmutant.so"))
    env = dict(os.environ, ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", "-k", "not every_in_range and not out_of_range_fp32"]
                       + PIN_TESTS, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, "planted mistake %r passed every pin:\n%s" % (name, r.stdout[-2000:])
    assert "failed" in r.stdout or "error" in r.stdout.lower(), r.stdout[-2000:]
