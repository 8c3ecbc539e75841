"""Planted mistakes in the Python oracles (index logits, top-k per row, the
key / head-gate projection) must
fail their pins (CPU only).

Each case copies the oracle module's source, plants one plausible mistake (a
ReLU in the wrong place, a dropped factor, a transposed or reordered operand,
an off-by-one mask, a reversed sort, an ignored length), and runs that
module's pin tests in a subprocess with the mutant swapped in for the real
module (a small pytest plugin loads it under the real module's name before
the tests import it).  The pins pass on the real oracle, so each mutant must
make at least one of them fail.
"""
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

LOGITS = ("oracle/logits.py", "logits", "tests/test_oracle_logits.py")
TOPK = ("oracle/topk.py", "topk", "tests/test_oracle_topk.py")
PROJ = ("oracle/proj.py", "proj", "tests/test_oracle_proj.py")

MUTANTS = [
    ("logits_relu_after_head_sum", LOGITS,
     'out = np.einsum("th,ths->ts", w, np.maximum(dots, 0.0))',
     'out = np.maximum(np.einsum("th,ths->ts", w, dots), 0.0)'),
    ("logits_relu_dropped", LOGITS, "np.maximum(dots, 0.0)", "dots"),
    ("logits_key_scale_dropped", LOGITS,
     "out *= np.asarray(k_scale, dtype=np.float64)[slots][None, :]", "pass"),
    ("logits_key_scale_unpermuted", LOGITS,
     "out *= np.asarray(k_scale, dtype=np.float64)[slots][None, :]",
     "out *= np.asarray(k_scale, dtype=np.float64)[:len(slots)][None, :]"),
    ("logits_keys_reversed", LOGITS, "return (q.reshape(T * H, D) @ k.T)",
     "return (q.reshape(T * H, D) @ k[::-1].T)"),
    ("logits_slots_ignored", LOGITS, "dots = head_dots(q_fp8, k_cache[slots])",
     "dots = head_dots(q_fp8, k_cache[:len(slots)])"),
    ("logits_length_off_by_one", LOGITS, ">= n[:, None]] = np.nan", "> n[:, None]] = np.nan"),
    ("logits_code_sign_dropped", LOGITS,
     "np.array([oracle.fp8_decode(c) for c in range(256)], dtype=np.float64)",
     "np.abs(np.array([oracle.fp8_decode(c) for c in range(256)], dtype=np.float64))"),
    ("topk_ascending", TOPK, "v = np.sort(logits[r, :n])[::-1]", "v = np.sort(logits[r, :n])"),
    ("topk_lengths_ignored", TOPK, "return np.clip(np.asarray(lengths, dtype=np.int64), 0, cols)",
     "return np.full(rows, cols, dtype=np.int64)"),
    ("topk_takes_one_less", TOPK, "take = min(n, k)", "take = min(n, k - 1) if n > k else min(n, k)"),
    ("topk_length_off_by_one", TOPK, "v = np.sort(logits[r, :n])[::-1]",
     "v = np.sort(logits[r, :n + 1])[::-1]"),
    ("proj_key_gate_split_swapped", PROJ,
     "return np.ascontiguousarray(bits[:, :ROW]), np.ascontiguousarray(bits[:, ROW:])",
     "return np.ascontiguousarray(bits[:, -ROW:]), np.ascontiguousarray(bits[:, :-ROW])"),
    ("proj_round_half_up", PROJ, "q = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)",
     "q = np.ldexp(np.floor(np.ldexp(m, 8) + 0.5), e - 8)"),
    ("proj_truncates", PROJ, "q = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)",
     "q = np.ldexp(np.trunc(np.ldexp(m, 8)), e - 8)"),
    ("proj_seven_bits", PROJ, "q = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)",
     "q = np.ldexp(np.rint(np.ldexp(m, 7)), e - 7)"),
    ("proj_rounds_through_fp32", PROJ, "    x = np.asarray(x, dtype=np.float64)\n",
     "    x = np.asarray(x, dtype=np.float32).astype(np.float64)\n"),
    ("proj_weight_transposed", PROJ, "return x @ w.T, np.abs(x) @ np.abs(w).T",
     "return (x.T[:w.shape[0]].T @ w[:, :x.shape[0]].T[:x.shape[1]] if x.shape[0] == w.shape[1] "
     "else x[:, ::-1] @ w.T), np.abs(x) @ np.abs(w).T"),
]

PLUGIN = textwrap.dedent('''
    import importlib.util, os, sys
    def pytest_configure(config):
        import oracle
        name = os.environ["MUTANT_MODULE"]
        spec = importlib.util.spec_from_file_location("oracle." + name, os.environ["MUTANT_PATH"])
        mod = importlib.util.module_from_spec(spec)
        sys.modules["oracle." + name] = mod
        spec.loader.exec_module(mod)
        setattr(oracle, name, mod)
''')


def test_every_mutation_applies_once():
    for name, (path, _, _), old, new in MUTANTS:
        assert open(os.path.join(ROOT, path)).read().count(old) == 1, name


@pytest.mark.parametrize("name,target,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, target, old, new):
    path, module, pins = target
    src = open(os.path.join(ROOT, path)).read().replace(old, new)
    mutant = tmp_path / ("mutant_%s.py" % module)
    mutant.write_text(src)
    (tmp_path / "mutant_plugin.py").write_text(PLUGIN)
    env = dict(os.environ, MUTANT_MODULE=module, MUTANT_PATH=str(mutant),
               PYTHONPATH=os.pathsep.join([str(tmp_path), ROOT, os.environ.get("PYTHONPATH", "")]))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-p", "mutant_plugin", "-m", "not gpu", pins],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, "planted mistake %r passed every pin:\n%s" % (name, r.stdout[-2000:])
    assert "failed" in r.stdout or "error" in r.stdout.lower(), r.stdout[-2000:]
