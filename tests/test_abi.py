"""C-ABI boundary checks that need no GPU.

The library must load, export every function include/dsaidx.h declares, agree
with the binding on struct layout, and reject bad arguments on the host before
any HIP call (so these run on a machine without a GPU).  Device pointers here
are fake, aligned addresses: the library never dereferences them on the host.
"""
import ctypes
import os
import re

import pytest

from rope_fp8_quant_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER_DIR = os.path.join(ROOT, "include")

FAKE = 0x10000  # aligned, never dereferenced on the host


def declared_functions():
    names = set()
    for fn in os.listdir(HEADER_DIR):
        if fn.endswith(".h"):
            text = open(os.path.join(HEADER_DIR, fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(dsaidx_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.LIB_PATH):
        from rope_fp8_quant_amd import build
        build.build()
    return B.lib()


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(L, n), n
    assert set(B.EXPORTED) == set(names)


def test_abi_version_and_struct_sizes(L):
    assert B.dsaidx_abi_version() == 6
    assert L.dsaidx_struct_size(0) == ctypes.sizeof(B.DsaidxRope) == 40
    assert L.dsaidx_struct_size(1) == ctypes.sizeof(B.DsaidxQArgs) == 88
    assert L.dsaidx_struct_size(2) == ctypes.sizeof(B.DsaidxKArgs) == 104
    assert L.dsaidx_struct_size(3) == ctypes.sizeof(B.DsaidxLogitsArgs) == 112
    assert L.dsaidx_struct_size(4) == ctypes.sizeof(B.DsaidxProjArgs) == 80
    assert L.dsaidx_struct_size(7) == 0


def test_status_strings(L):
    assert B.status_string(0) == "DSAIDX_OK"
    assert B.status_string(1) == "DSAIDX_ERR_INVALID_ARGUMENT"
    assert B.status_string(2) == "DSAIDX_ERR_UNSUPPORTED"
    assert B.status_string(3) == "DSAIDX_ERR_HIP"
    assert B.status_string(99) == "DSAIDX_UNKNOWN_STATUS"


def test_device_supported_without_gpu_does_not_crash(L):
    v = L.dsaidx_device_supported(0)
    assert v in (0, 1)
    assert L.dsaidx_device_supported(-1) == 0
    assert L.dsaidx_device_supported(1 << 20) == 0


def good_rope(**kw):
    r = B.DsaidxRope(FAKE, FAKE + 128, 64, 4096, 64, 0)
    for k, v in kw.items():
        setattr(r, k, v)
    return r


def good_q(T=1, **kw):
    q = B.DsaidxQArgs(FAKE, 64 * 128, 128, FAKE, 64, FAKE, T, 64, 1.0, FAKE, FAKE, None)
    for k, v in kw.items():
        setattr(q, k, v)
    return q


def good_k(T=1, **kw):
    k = B.DsaidxKArgs(FAKE, 128, FAKE, FAKE, 1e-6, 0, FAKE, FAKE, T, FAKE, 128, FAKE, 4096, 0)
    for k_, v in kw.items():
        setattr(k, k_, v)
    return k


def call_q(L, q, r):
    return L.dsaidx_q_rope_quant_fold(ctypes.byref(q), ctypes.byref(r), None)


def call_k(L, k, r, entry="dsaidx_k_norm_rope_quant_store"):
    return getattr(L, entry)(ctypes.byref(k), ctypes.byref(r), None)


def call_fused(L, q, k, r):
    return L.dsaidx_qk_fused(ctypes.byref(q), ctypes.byref(k), ctypes.byref(r), None)


def test_empty_calls_are_ok_without_launch(L):
    r = good_rope()
    assert call_q(L, good_q(T=0), r) == B.DSAIDX_OK
    assert call_k(L, good_k(T=0), r) == B.DSAIDX_OK
    assert call_k(L, good_k(T=0), r, "dsaidx_k_only_prepare_store") == B.DSAIDX_OK
    assert call_fused(L, good_q(T=0), good_k(T=0), r) == B.DSAIDX_OK
    # empty tensors may carry NULL data pointers
    null_q = B.DsaidxQArgs()
    null_k = B.DsaidxKArgs()
    null_r = B.DsaidxRope()
    assert call_q(L, null_q, null_r) == B.DSAIDX_OK
    assert call_k(L, null_k, null_r) == B.DSAIDX_OK
    assert call_fused(L, null_q, null_k, null_r) == B.DSAIDX_OK


def test_null_structs_rejected(L):
    assert L.dsaidx_q_rope_quant_fold(None, ctypes.byref(good_rope()), None) == 1
    assert L.dsaidx_qk_fused(ctypes.byref(good_q()), ctypes.byref(good_k()), None, None) == 1
    assert L.dsaidx_q_rope_quant_fold(ctypes.byref(good_q()), None, None) == 1
    assert L.dsaidx_k_norm_rope_quant_store(None, ctypes.byref(good_rope()), None) == 1
    assert L.dsaidx_k_only_prepare_store(None, ctypes.byref(good_rope()), None) == 1
    assert L.dsaidx_qk_fused(ctypes.byref(good_q()), None, ctypes.byref(good_rope()), None) == 1


BAD_ROPE = [dict(cos=None), dict(sin=None), dict(cos=FAKE + 2), dict(sin=FAKE + 1),
            dict(rope_dim=0), dict(rope_dim=-2), dict(rope_dim=7), dict(rope_dim=63),
            dict(rope_dim=130), dict(rope_dim=144), dict(style=2), dict(style=-1),
            dict(row_stride=16), dict(rope_dim=6, row_stride=2), dict(max_position=0)]
GOOD_ROPE = [dict(rope_dim=2, row_stride=1), dict(rope_dim=6, row_stride=3), dict(rope_dim=126, row_stride=63),
             dict(rope_dim=24), dict(row_stride=34), dict(cos=FAKE + 4, sin=FAKE + 8), dict(style=1, rope_dim=10)]


@pytest.mark.parametrize("kw", BAD_ROPE, ids=lambda d: str(d))
def test_bad_rope_rejected(L, kw):
    r = good_rope(**kw)
    assert call_q(L, good_q(), r) == B.DSAIDX_ERR_INVALID_ARGUMENT
    assert call_k(L, good_k(), r) == B.DSAIDX_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("kw", GOOD_ROPE, ids=lambda d: str(d))
def test_every_even_rope_dim_and_table_stride_accepted(L, kw):
    """Any even rope_dim in [2, 128] and any row stride >= rope_dim / 2 with
    4-byte aligned tables passes the checks (the launch itself then fails on a
    machine without a GPU, with a status other than INVALID_ARGUMENT)."""
    r = good_rope(**kw)
    assert call_q(L, good_q(), r) != B.DSAIDX_ERR_INVALID_ARGUMENT
    assert call_k(L, good_k(), r) != B.DSAIDX_ERR_INVALID_ARGUMENT


BAD_Q = [dict(q=None), dict(weights=None), dict(positions=None), dict(q_fp8=None),
         dict(weights_out=None), dict(q=FAKE + 8), dict(positions=FAKE + 4),
         dict(q_fp8=FAKE + 4), dict(weights_out=FAKE + 2), dict(q_scale_out=FAKE + 2),
         dict(weights=FAKE + 1), dict(num_tokens=-1), dict(num_heads=0), dict(num_heads=5000),
         dict(q_stride_h=120), dict(q_stride_h=132), dict(q_stride_t=63 * 128),
         dict(q_stride_t=64 * 128 + 4), dict(w_stride_t=63), dict(weight_scale=float("inf")),
         dict(weight_scale=float("nan"))]


@pytest.mark.parametrize("kw", BAD_Q, ids=lambda d: str(d))
def test_bad_q_rejected(L, kw):
    q = good_q(**kw)
    assert call_q(L, q, good_rope()) == B.DSAIDX_ERR_INVALID_ARGUMENT
    assert call_fused(L, q, good_k(), good_rope()) == B.DSAIDX_ERR_INVALID_ARGUMENT


BAD_K = [dict(k=None), dict(ln_gamma=None), dict(ln_beta=None), dict(positions=None),
         dict(out_cache_loc=None), dict(k_cache=None), dict(k_scale=None),
         dict(k=FAKE + 8), dict(ln_gamma=FAKE + 4), dict(out_cache_loc=FAKE + 4),
         dict(k_cache=FAKE + 4), dict(k_scale=FAKE + 2), dict(num_tokens=-3),
         dict(k_stride_t=64), dict(k_stride_t=130), dict(ln_eps=0.0), dict(ln_eps=-1e-6),
         dict(ln_eps=float("nan")), dict(ln_eps=float("inf")), dict(flags=8), dict(flags=-1),
         dict(flags=5), dict(flags=7, page_size=64, num_slots=128),
         dict(k_cache_row_stride=120), dict(k_cache_row_stride=132), dict(num_slots=0),
         dict(flags=1, k_scale=None),
         dict(flags=2, page_size=0), dict(flags=2, page_size=1), dict(flags=2, page_size=3),
         dict(flags=2, page_size=-64), dict(flags=2, page_size=1 << 21),
         dict(flags=2, page_size=64, num_slots=100), dict(flags=3, page_size=6, num_slots=64)]


@pytest.mark.parametrize("kw", BAD_K, ids=lambda d: str(d))
def test_bad_k_rejected(L, kw):
    k = good_k(**kw)
    for entry in ("dsaidx_k_norm_rope_quant_store", "dsaidx_k_only_prepare_store"):
        assert call_k(L, k, good_rope(), entry) == B.DSAIDX_ERR_INVALID_ARGUMENT
    assert call_fused(L, good_q(), k, good_rope()) == B.DSAIDX_ERR_INVALID_ARGUMENT


def test_fused_token_count_mismatch_rejected(L):
    assert call_fused(L, good_q(T=3), good_k(T=4), good_rope()) == B.DSAIDX_ERR_INVALID_ARGUMENT
    assert call_fused(L, good_q(T=0), good_k(T=4), good_rope()) == B.DSAIDX_ERR_INVALID_ARGUMENT
    assert call_fused(L, good_q(T=2), good_k(T=0), good_rope()) == B.DSAIDX_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("T", [-1, (1 << 40) + 1])
def test_token_count_range(L, T):
    assert call_q(L, good_q(T=T), good_rope()) == B.DSAIDX_ERR_INVALID_ARGUMENT
    assert call_k(L, good_k(T=T), good_rope()) == B.DSAIDX_ERR_INVALID_ARGUMENT


def test_fp8_selftest_argument_checks(L):
    assert L.dsaidx_fp8_encode_selftest(FAKE, FAKE, 0, 0, None) == B.DSAIDX_OK
    assert L.dsaidx_fp8_encode_selftest(FAKE, FAKE, -1, 0, None) == 1
    assert L.dsaidx_fp8_encode_selftest(None, FAKE, 8, 0, None) == 1
    assert L.dsaidx_fp8_encode_selftest(FAKE, None, 8, 0, None) == 1
    assert L.dsaidx_fp8_encode_selftest(FAKE + 2, FAKE, 8, 0, None) == 1
    assert L.dsaidx_fp8_encode_selftest(FAKE, FAKE + 4, 8, 0, None) == 1
    assert L.dsaidx_fp8_encode_selftest(FAKE, FAKE, 8, -127, None) == 1
    assert L.dsaidx_fp8_encode_selftest(FAKE, FAKE, 8, 128, None) == 1


def test_hbm_stream_argument_checks(L):
    f = L.dsaidx_hbm_stream
    assert f(0, FAKE, FAKE, 0, 0, None) == B.DSAIDX_OK            # nothing to do
    assert f(2, None, None, 0, 0, None) == B.DSAIDX_OK
    for bad in [(3, FAKE, FAKE, 64), (-1, FAKE, FAKE, 64), (0, FAKE, FAKE, -16),
                (0, FAKE, FAKE, 24), (0, FAKE, FAKE, (1 << 38) + 16), (0, None, FAKE, 64),
                (0, FAKE, None, 64), (1, None, FAKE, 64), (1, FAKE, None, 64), (2, FAKE, None, 64),
                (0, FAKE + 8, FAKE, 64), (0, FAKE, FAKE + 4, 64), (2, None, FAKE + 8, 64)]:
        mode, src, dst, n = bad
        assert f(mode, src, dst, n, 0, None) == B.DSAIDX_ERR_INVALID_ARGUMENT, bad


def test_topk_argument_checks(L):
    P = ctypes.c_void_p
    ok = dict(logits=FAKE, row_stride=2048, lengths=None, rows=4, cols=2048, k=64, out=FAKE)

    def call(**kw):
        a = dict(ok, **kw)
        return L.dsaidx_topk_per_row(P(a["logits"]), a["row_stride"], P(a["lengths"]), a["rows"],
                                     a["cols"], a["k"], P(a["out"]), P(a.get("ws")),
                                     a.get("ws_bytes", 0), None)
    assert call(rows=0) == B.DSAIDX_OK
    assert call(rows=0, logits=None, out=None) == B.DSAIDX_OK
    for bad in (dict(rows=-1), dict(rows=1 << 31), dict(cols=-1), dict(cols=1 << 31), dict(k=0),
                dict(k=(1 << 20) + 1), dict(logits=None), dict(out=None), dict(logits=FAKE + 4),
                dict(out=FAKE + 2), dict(lengths=FAKE + 2), dict(row_stride=2047),
                dict(row_stride=2050), dict(row_stride=1024)):
        assert call(**bad) == B.DSAIDX_ERR_INVALID_ARGUMENT, bad


def test_topk_workspace_size_and_checks(L):
    P = ctypes.c_void_p
    ws = L.dsaidx_topk_workspace_bytes
    assert ws(64, 16384, 2048) == 0
    assert ws(64, 32768, 2048) == 0
    # rows longer than 32768: per row a 2048-bin histogram and counters
    # (8224 bytes) and a list of max(4096, cols / 16) (key, index) pairs
    assert ws(64, 131072, 2048) == 64 * (8224 + 8 * 8192)
    assert ws(3, 32769, 7) == 3 * (8224 + 8 * 4096)
    assert ws(64, 50000, 40000) == 64 * (8224 + 8 * 4096)
    assert ws(2, 1000003, 2048) == 2 * (8224 + 8 * 62500)
    assert ws(0, 131072, 2048) == 0
    assert ws(-1, 10, 1) == -1 and ws(1, 10, 0) == -1 and ws(1, -1, 1) == -1
    assert ws(1 << 20, 1 << 30, 8) == -1      # grid of rows * ceil(cols / 4096) workgroups too large
    assert ws((1 << 31) - 1, 32768, 8) == 0
    need = ws(2, 131072, 2048)

    def call(w, nbytes, rows=2, cols=131072):
        return L.dsaidx_topk_per_row(P(FAKE), cols, None, rows, cols, 2048, P(FAKE), P(w), nbytes,
                                     None)
    assert call(None, 0) == B.DSAIDX_ERR_INVALID_ARGUMENT
    assert call(FAKE, need - 1) == B.DSAIDX_ERR_INVALID_ARGUMENT
    assert call(FAKE + 4, need) == B.DSAIDX_ERR_INVALID_ARGUMENT
    assert call(None, 0, rows=0) == B.DSAIDX_OK
    assert call(FAKE, 1 << 62, rows=1 << 20, cols=1 << 30) == B.DSAIDX_ERR_INVALID_ARGUMENT


C_PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "dsaidx.h"

int main(void) {
    dsaidx_rope rope;
    dsaidx_q_args q;
    dsaidx_k_args k;
    memset(&rope, 0, sizeof rope);
    memset(&q, 0, sizeof q);
    memset(&k, 0, sizeof k);
    if (dsaidx_abi_version() != DSAIDX_ABI_VERSION) return 1;
    if (dsaidx_struct_size(0) != sizeof(dsaidx_rope)) return 2;
    if (dsaidx_struct_size(1) != sizeof(dsaidx_q_args)) return 3;
    if (dsaidx_struct_size(2) != sizeof(dsaidx_k_args)) return 4;
    if (dsaidx_struct_size(3) != sizeof(dsaidx_logits_args)) return 5;
    /* empty calls: OK without touching a device */
    if (dsaidx_qk_fused(&q, &k, &rope, NULL) != DSAIDX_OK) return 5;
    if (dsaidx_topk_per_row(NULL, 0, NULL, 0, 0, 1, NULL, NULL, 0, NULL) != DSAIDX_OK) return 6;
    /* rejected on the host */
    q.num_tokens = 1;
    if (dsaidx_q_rope_quant_fold(&q, &rope, NULL) != DSAIDX_ERR_INVALID_ARGUMENT) return 7;
    if (dsaidx_topk_workspace_bytes(1, 1 << 20, 2048) <= 0) return 8;
    printf("%s %d\n", dsaidx_status_string(DSAIDX_ERR_UNSUPPORTED), dsaidx_device_supported(-1));
    return 0;
}
"""


def test_header_compiles_and_links_as_c99(L, tmp_path):
    """include/dsaidx.h is plain C: a C99 program built with -Wall -Werror
    against it links to libdsaidx.so and runs the host-side paths."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    src = tmp_path / "abi.c"
    exe = tmp_path / "abi"
    src.write_text(C_PROGRAM)
    libdir = os.path.dirname(B.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", HEADER_DIR,
                    str(src), "-o", str(exe), "-L", libdir, "-ldsaidx", "-Wl,-rpath," + libdir],
                   check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert r.stdout.strip() == "DSAIDX_ERR_UNSUPPORTED 0"


def test_binding_refuses_host_tensors(L):
    """The binding hands plain device pointers to the library, which never
    reads them on the host: every tensor builder and wrapper refuses a host
    tensor with ValueError before anything is launched."""
    import torch
    T, H, S = 2, 4, 8
    bf = lambda *s: torch.zeros(s, dtype=torch.bfloat16)
    f32 = lambda *s: torch.zeros(s, dtype=torch.float32)
    i64 = lambda *s: torch.zeros(s, dtype=torch.int64)
    u8 = lambda *s: torch.zeros(s, dtype=torch.uint8)
    cases = [
        lambda: B.rope_args(f32(16, 32), f32(16, 32)),
        lambda: B.q_args(bf(T, H, 128), bf(T, H), i64(T), u8(T, H, 128), f32(T, H)),
        lambda: B.k_args(bf(T, 128), f32(128), f32(128), 1e-6, i64(T), i64(T), u8(S, 128), f32(S)),
        lambda: B.logits_args(u8(T, H, 128), f32(T, H), u8(S, 128), f32(T, S), k_scale=f32(S)),
        lambda: B.dsaidx_topk_per_row(f32(T, 64), 4, torch.zeros((T, 4), dtype=torch.int32)),
        lambda: B.dsaidx_fp8_encode_selftest(f32(64), u8(64)),
    ]
    for make in cases:
        with pytest.raises(ValueError, match="GPU tensor"):
            make()


def good_proj(**kw):
    p = B.DsaidxProjArgs(FAKE, 7168, FAKE, 7168, 7168, 64, 0, FAKE, 64, None, 128)
    for k_, v in kw.items():
        setattr(p, k_, v)
    return p


def call_proj(L, p, k, r):
    return L.dsaidx_proj_k_norm_rope_quant_store(ctypes.byref(p), ctypes.byref(k), ctypes.byref(r), None)


BAD_PROJ = [dict(hidden=None), dict(weight=None), dict(gates_out=None), dict(hidden=FAKE + 8),
            dict(weight=FAKE + 8), dict(gates_out=FAKE + 1), dict(k_out=FAKE + 8),
            dict(hidden_dim=0), dict(hidden_dim=32), dict(hidden_dim=96), dict(hidden_dim=7168 + 32), dict(hidden_dim=1 << 21),
            dict(hidden_stride_t=7160), dict(hidden_stride_t=7172), dict(weight_stride_n=7160),
            dict(hidden_stride_t=(1 << 22) + 8), dict(weight_stride_n=(1 << 22) + 8),
            dict(weight_stride_n=7172), dict(num_heads=0), dict(num_heads=65), dict(reserved=1),
            dict(gates_stride_t=63), dict(k_out=FAKE, k_out_stride_t=120),
            dict(k_out=FAKE, k_out_stride_t=132)]


@pytest.mark.parametrize("kw", BAD_PROJ, ids=lambda d: str(d))
def test_bad_projection_rejected(L, kw):
    assert call_proj(L, good_proj(**kw), good_k(k=None, k_stride_t=0), good_rope()) == \
        B.DSAIDX_ERR_INVALID_ARGUMENT


def test_projection_checks_key_side_but_not_its_row(L):
    """The projection computes the key: k and k_stride_t are not looked at,
    the rest of the key side is checked as for the key entry."""
    ok = call_proj(L, good_proj(), good_k(k=None, k_stride_t=0), good_rope())
    assert ok != B.DSAIDX_ERR_INVALID_ARGUMENT          # no GPU here: the launch itself fails
    assert call_proj(L, good_proj(), good_k(k=None, ln_eps=0.0), good_rope()) == \
        B.DSAIDX_ERR_INVALID_ARGUMENT
    assert call_proj(L, good_proj(), good_k(k=None, out_cache_loc=None), good_rope()) == \
        B.DSAIDX_ERR_INVALID_ARGUMENT
    assert call_proj(L, good_proj(hidden=None), good_k(T=0), good_rope()) == B.DSAIDX_OK
