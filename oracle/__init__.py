"""ctypes loader for the C oracle — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product package
(``rope_fp8_quant_amd``) never imports it, and the two share no code.

The arithmetic lives in ``dsaidx_oracle.c``; this module only builds the
shared library when it is missing and marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SOURCES = [os.path.join(_HERE, "dsaidx_oracle.c")]

ROW = 128
NEOX = 0
INTERLEAVED = 1


def build(force: bool = True, sources=None, out_path: str = LIB_PATH) -> str:
    """Compile the oracle with gcc (fp32, no contraction, OpenMP)."""
    if not force and os.path.exists(out_path):
        return out_path
    tmp = out_path + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math",
           "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra", "-I" + _HERE,
           "-o", tmp] + list(sources or SOURCES) + ["-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out_path)
    return out_path


_lib = None


def lib() -> ctypes.CDLL:
    """The oracle library.  ORACLE_LIB overrides the path (the mutation tests
    point it at builds of the oracle with a planted mistake)."""
    global _lib
    if _lib is None:
        path = os.environ.get("ORACLE_LIB", LIB_PATH)
        if path == LIB_PATH and not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        i32 = ctypes.c_int
        f32 = ctypes.c_float
        L.oracle_fp8_encode.argtypes = [f32]
        L.oracle_fp8_encode.restype = ctypes.c_uint8
        L.oracle_fp8_decode.argtypes = [ctypes.c_uint8]
        L.oracle_fp8_decode.restype = f32
        L.oracle_fp8_encode_array.argtypes = [P, P, i64, i32]
        L.oracle_fp8_encode_array.restype = None
        L.oracle_ue8m0_exponent.argtypes = [f32]
        L.oracle_ue8m0_exponent.restype = i32
        L.oracle_q.argtypes = [P, i64, i64, P, i64, P, i64, i32, f32,
                               P, P, i64, i64, i32, i32, P, P, P, i32]
        L.oracle_q.restype = i32
        L.oracle_q_values.argtypes = [P, i64, i64, P, i64, i32, P, P, i64, i64, i32, i32,
                                      P, P, i32]
        L.oracle_q_values.restype = i32
        L.oracle_k_values.argtypes = [P, i64, P, P, f32, P, i64,
                                      P, P, i64, i64, i32, i32, i32, P, P, i32]
        L.oracle_k_values.restype = i32
        L.oracle_k.argtypes = [P, i64, P, P, f32, P, P, i64,
                               P, P, i64, i64, i32, i32, i32, P, i64, P, i64, i32]
        L.oracle_k.restype = i32
        L.oracle_k_paged.argtypes = [P, i64, P, P, f32, P, P, i64,
                                     P, P, i64, i64, i32, i32, i32, P, i64, i64, i32]
        L.oracle_k_paged.restype = i32
        L.oracle_max_threads.argtypes = []
        L.oracle_max_threads.restype = i32
        _lib = L
    return _lib


def _p(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _elem_strides(a: np.ndarray):
    return tuple(s // a.itemsize for s in a.strides)


# ----------------------------------------------------------------- scalars --

def fp8_encode(v: float) -> int:
    return int(lib().oracle_fp8_encode(float(v)))


def fp8_decode(code: int) -> float:
    return float(lib().oracle_fp8_decode(int(code)))


def fp8_encode_array(v: np.ndarray, nthreads: int = 0) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    lib().oracle_fp8_encode_array(_p(v), _p(out), v.size, nthreads)
    return out


def ue8m0_exponent(amax: float) -> int:
    return int(lib().oracle_ue8m0_exponent(float(amax)))


def max_threads() -> int:
    return int(lib().oracle_max_threads())


# ---------------------------------------------------------------- Q and K --

def rope_tables(cos: np.ndarray, sin: np.ndarray):
    """Check two [P, >=R/2] fp32 views that share a row stride."""
    assert cos.dtype == np.float32 and sin.dtype == np.float32
    assert cos.shape[0] == sin.shape[0]
    rs = _elem_strides(cos)[0]
    assert _elem_strides(sin)[0] == rs and _elem_strides(cos)[1] == 1
    return rs, cos.shape[0]


def q_side(q, weights, positions, cos, sin, rope_dim=64, style=NEOX,
           weight_scale=1.0, nthreads=0):
    """q: uint16 (bf16 bits) [T, H, 128] view with unit inner stride;
    weights: uint16 [T, H] view with unit inner stride.
    Returns (q_fp8 [T,H,128] uint8, weights_out [T,H] f32, q_scale [T,H] f32)."""
    T, H, D = q.shape
    assert D == ROW and q.dtype == np.uint16 and weights.dtype == np.uint16
    q_st, q_sh, q_si = _elem_strides(q)
    w_st, w_sh = _elem_strides(weights)
    assert q_si == 1 and w_sh == 1
    positions = np.ascontiguousarray(positions, dtype=np.int64)
    rs, P = rope_tables(cos, sin)
    q_fp8 = np.empty((T, H, ROW), dtype=np.uint8)
    w_out = np.empty((T, H), dtype=np.float32)
    q_scale = np.empty((T, H), dtype=np.float32)
    rc = lib().oracle_q(_p(q), q_st, q_sh, _p(weights), w_st, _p(positions), T, H,
                        float(weight_scale), _p(cos), _p(sin), rs, P, rope_dim, style,
                        _p(q_fp8), _p(w_out), _p(q_scale), nthreads)
    if rc != 0:
        raise ValueError("oracle_q: position out of range")
    return q_fp8, w_out, q_scale


def q_values(q, positions, cos, sin, rope_dim=64, style=NEOX, nthreads=0):
    """Returns (y [T,H,128] f32 after RoPE, e [T,H] int32)."""
    T, H, D = q.shape
    assert D == ROW and q.dtype == np.uint16
    q_st, q_sh, q_si = _elem_strides(q)
    assert q_si == 1
    positions = np.ascontiguousarray(positions, dtype=np.int64)
    rs, P = rope_tables(cos, sin)
    y = np.empty((T, H, ROW), dtype=np.float32)
    e = np.empty((T, H), dtype=np.int32)
    rc = lib().oracle_q_values(_p(q), q_st, q_sh, _p(positions), T, H, _p(cos), _p(sin),
                               rs, P, rope_dim, style, _p(y), _p(e), nthreads)
    if rc != 0:
        raise ValueError("oracle_q_values: position out of range")
    return y, e


def k_values(k, gamma, beta, eps, positions, cos, sin, rope_dim=64, style=NEOX,
             bf16_mode=0, nthreads=0):
    """Returns (y [T,128] f32 after LayerNorm + RoPE, e [T] int32)."""
    T, D = k.shape
    assert D == ROW and k.dtype == np.uint16
    k_st, k_si = _elem_strides(k)
    assert k_si == 1
    gamma = np.ascontiguousarray(gamma, dtype=np.float32)
    beta = np.ascontiguousarray(beta, dtype=np.float32)
    positions = np.ascontiguousarray(positions, dtype=np.int64)
    rs, P = rope_tables(cos, sin)
    y = np.empty((T, ROW), dtype=np.float32)
    e = np.empty((T,), dtype=np.int32)
    rc = lib().oracle_k_values(_p(k), k_st, _p(gamma), _p(beta), float(eps), _p(positions), T,
                               _p(cos), _p(sin), rs, P, rope_dim, style, bf16_mode,
                               _p(y), _p(e), nthreads)
    if rc != 0:
        raise ValueError("oracle_k_values: position out of range")
    return y, e


def k_side(k, gamma, beta, eps, positions, out_cache_loc, cos, sin, k_cache, k_scale,
           rope_dim=64, style=NEOX, bf16_mode=0, nthreads=0):
    """Writes into k_cache (uint8 [S, >=128] view, unit inner stride) and
    k_scale (f32 [S]) in place, at the slots in out_cache_loc."""
    T, D = k.shape
    assert D == ROW and k.dtype == np.uint16
    k_st, k_si = _elem_strides(k)
    assert k_si == 1
    assert k_cache.dtype == np.uint8 and k_scale.dtype == np.float32
    row_stride, ci = _elem_strides(k_cache)
    assert ci == 1 and k_scale.flags.c_contiguous
    S = k_cache.shape[0]
    assert k_scale.shape[0] == S
    gamma = np.ascontiguousarray(gamma, dtype=np.float32)
    beta = np.ascontiguousarray(beta, dtype=np.float32)
    positions = np.ascontiguousarray(positions, dtype=np.int64)
    loc = np.ascontiguousarray(out_cache_loc, dtype=np.int64)
    rs, P = rope_tables(cos, sin)
    rc = lib().oracle_k(_p(k), k_st, _p(gamma), _p(beta), float(eps), _p(positions), _p(loc), T,
                        _p(cos), _p(sin), rs, P, rope_dim, style, bf16_mode,
                        _p(k_cache), row_stride, _p(k_scale), S, nthreads)
    if rc != 0:
        raise ValueError("oracle_k: position out of range (rc=%d)" % rc)


def k_side_paged(k, gamma, beta, eps, positions, out_cache_loc, cos, sin, cache, page_size,
                 num_slots, rope_dim=64, style=NEOX, bf16_mode=0, nthreads=0):
    """Writes into cache (uint8, num_slots * 132 bytes, page-interleaved) in place."""
    T, D = k.shape
    assert D == ROW and k.dtype == np.uint16
    k_st, k_si = _elem_strides(k)
    assert k_si == 1
    assert cache.dtype == np.uint8 and cache.flags.c_contiguous
    assert cache.size == num_slots * (ROW + 4)
    gamma = np.ascontiguousarray(gamma, dtype=np.float32)
    beta = np.ascontiguousarray(beta, dtype=np.float32)
    positions = np.ascontiguousarray(positions, dtype=np.int64)
    loc = np.ascontiguousarray(out_cache_loc, dtype=np.int64)
    rs, P = rope_tables(cos, sin)
    rc = lib().oracle_k_paged(_p(k), k_st, _p(gamma), _p(beta), float(eps), _p(positions), _p(loc),
                              T, _p(cos), _p(sin), rs, P, rope_dim, style, bf16_mode,
                              _p(cache), page_size, num_slots, nthreads)
    if rc != 0:
        raise ValueError("oracle_k_paged failed (rc=%d)" % rc)
