"""Thin ctypes binding of libdsaidx (argument marshalling only).

Every step of the computation runs in the library's HIP kernels; this module
fills the C argument structs from torch tensors (device pointers and strides)
and calls the entry points of the same names.  torch is used for device memory
and streams only.  There is no fallback: if libdsaidx.so is missing or the
device is not supported, the calls raise.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libdsaidx.so")
ROW = 128

DSAIDX_OK = 0
DSAIDX_ERR_INVALID_ARGUMENT = 1
DSAIDX_ERR_UNSUPPORTED = 2
DSAIDX_ERR_HIP = 3
DSAIDX_ROPE_NEOX = 0
DSAIDX_ROPE_INTERLEAVED = 1
DSAIDX_K_BF16_INTERMEDIATE = 0x1
DSAIDX_K_PAGED_CACHE = 0x2
DSAIDX_K_BF16_ROUND_ONCE = 0x4
PAGED_SLOT_BYTES = ROW + 4   # one code row and one fp32 scale per slot
EXPORTED = ("dsaidx_q_rope_quant_fold", "dsaidx_k_norm_rope_quant_store", "dsaidx_qk_fused",
            "dsaidx_k_only_prepare_store", "dsaidx_device_supported", "dsaidx_status_string",
            "dsaidx_abi_version", "dsaidx_struct_size", "dsaidx_fp8_encode_selftest",
            "dsaidx_topk_per_row", "dsaidx_topk_workspace_bytes", "dsaidx_mqa_logits",
            "dsaidx_hbm_stream", "dsaidx_topk_per_row_noalloc",
            "dsaidx_proj_k_norm_rope_quant_store")
TOPK_NOALLOC_SCRATCH_BYTES = 16 << 20


class DsaidxError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s failed: %s" % (where, status_string(status)))


class DsaidxRope(ctypes.Structure):
    _fields_ = [("cos", ctypes.c_void_p), ("sin", ctypes.c_void_p),
                ("row_stride", ctypes.c_int64), ("max_position", ctypes.c_int64),
                ("rope_dim", ctypes.c_int32), ("style", ctypes.c_int32)]


class DsaidxQArgs(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("q_stride_t", ctypes.c_int64),
                ("q_stride_h", ctypes.c_int64), ("weights", ctypes.c_void_p),
                ("w_stride_t", ctypes.c_int64), ("positions", ctypes.c_void_p),
                ("num_tokens", ctypes.c_int64), ("num_heads", ctypes.c_int32),
                ("weight_scale", ctypes.c_float), ("q_fp8", ctypes.c_void_p),
                ("weights_out", ctypes.c_void_p), ("q_scale_out", ctypes.c_void_p)]


class DsaidxKArgs(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("k_stride_t", ctypes.c_int64),
                ("ln_gamma", ctypes.c_void_p), ("ln_beta", ctypes.c_void_p),
                ("ln_eps", ctypes.c_float), ("flags", ctypes.c_int32),
                ("positions", ctypes.c_void_p), ("out_cache_loc", ctypes.c_void_p),
                ("num_tokens", ctypes.c_int64), ("k_cache", ctypes.c_void_p),
                ("k_cache_row_stride", ctypes.c_int64), ("k_scale", ctypes.c_void_p),
                ("num_slots", ctypes.c_int64), ("page_size", ctypes.c_int64)]


class DsaidxLogitsArgs(ctypes.Structure):
    _fields_ = [("q_fp8", ctypes.c_void_p), ("weights", ctypes.c_void_p),
                ("num_tokens", ctypes.c_int64), ("num_heads", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("k_cache", ctypes.c_void_p),
                ("k_cache_row_stride", ctypes.c_int64), ("k_scale", ctypes.c_void_p),
                ("num_slots", ctypes.c_int64), ("page_size", ctypes.c_int64),
                ("key_slots", ctypes.c_void_p), ("num_keys", ctypes.c_int64),
                ("lengths", ctypes.c_void_p), ("logits", ctypes.c_void_p),
                ("logits_stride", ctypes.c_int64)]


class DsaidxProjArgs(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_void_p), ("hidden_stride_t", ctypes.c_int64),
                ("weight", ctypes.c_void_p), ("weight_stride_n", ctypes.c_int64),
                ("hidden_dim", ctypes.c_int64), ("num_heads", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("gates_out", ctypes.c_void_p),
                ("gates_stride_t", ctypes.c_int64), ("k_out", ctypes.c_void_p),
                ("k_out_stride_t", ctypes.c_int64)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libdsaidx.so (built in-tree by rope_fp8_quant_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libdsaidx.so is not built (%s); run "
                               "`python -m rope_fp8_quant_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        for name, args in (("dsaidx_q_rope_quant_fold", [ctypes.POINTER(DsaidxQArgs),
                                                         ctypes.POINTER(DsaidxRope), P]),
                           ("dsaidx_k_norm_rope_quant_store", [ctypes.POINTER(DsaidxKArgs),
                                                               ctypes.POINTER(DsaidxRope), P]),
                           ("dsaidx_k_only_prepare_store", [ctypes.POINTER(DsaidxKArgs),
                                                            ctypes.POINTER(DsaidxRope), P]),
                           ("dsaidx_qk_fused", [ctypes.POINTER(DsaidxQArgs),
                                                ctypes.POINTER(DsaidxKArgs),
                                                ctypes.POINTER(DsaidxRope), P]),
                           ("dsaidx_mqa_logits", [ctypes.POINTER(DsaidxLogitsArgs), P]),
                           ("dsaidx_proj_k_norm_rope_quant_store",
                            [ctypes.POINTER(DsaidxProjArgs), ctypes.POINTER(DsaidxKArgs),
                             ctypes.POINTER(DsaidxRope), P])):
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        L.dsaidx_topk_per_row.argtypes = [P, ctypes.c_int64, P, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_int32, P, P, ctypes.c_int64, P]
        L.dsaidx_topk_per_row.restype = ctypes.c_int
        L.dsaidx_topk_per_row_noalloc.argtypes = [P, ctypes.c_int64, P, ctypes.c_int64,
                                                  ctypes.c_int64, ctypes.c_int32, P, P]
        L.dsaidx_topk_per_row_noalloc.restype = ctypes.c_int
        L.dsaidx_topk_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32]
        L.dsaidx_topk_workspace_bytes.restype = ctypes.c_int64
        L.dsaidx_fp8_encode_selftest.argtypes = [P, P, ctypes.c_int64, ctypes.c_int32, P]
        L.dsaidx_fp8_encode_selftest.restype = ctypes.c_int
        L.dsaidx_hbm_stream.argtypes = [ctypes.c_int32, P, P, ctypes.c_int64, ctypes.c_uint32, P]
        L.dsaidx_hbm_stream.restype = ctypes.c_int
        L.dsaidx_device_supported.argtypes = [ctypes.c_int]
        L.dsaidx_device_supported.restype = ctypes.c_int
        L.dsaidx_status_string.argtypes = [ctypes.c_int]
        L.dsaidx_status_string.restype = ctypes.c_char_p
        L.dsaidx_abi_version.argtypes = []
        L.dsaidx_abi_version.restype = ctypes.c_int
        L.dsaidx_struct_size.argtypes = [ctypes.c_int]
        L.dsaidx_struct_size.restype = ctypes.c_size_t
        for which, cls in enumerate((DsaidxRope, DsaidxQArgs, DsaidxKArgs, DsaidxLogitsArgs,
                                     DsaidxProjArgs)):
            if L.dsaidx_struct_size(which) != ctypes.sizeof(cls):
                raise RuntimeError("libdsaidx ABI mismatch for %s" % cls.__name__)
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().dsaidx_status_string(int(status)).decode()


def dsaidx_status_string(status: int) -> str:
    return status_string(status)


def dsaidx_device_supported(device: int = 0) -> bool:
    return bool(lib().dsaidx_device_supported(int(device)))


def dsaidx_abi_version() -> int:
    return int(lib().dsaidx_abi_version())


# ------------------------------------------------------ stream handling ----

def _stream_handle(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status: int, where: str):
    if status != DSAIDX_OK:
        raise DsaidxError(status, where)


# -------------------------------------------------------- entry points ----

def dsaidx_q_rope_quant_fold(q: DsaidxQArgs, rope: DsaidxRope, stream=None) -> None:
    _check(lib().dsaidx_q_rope_quant_fold(ctypes.byref(q), ctypes.byref(rope),
                                          _stream_handle(stream)), "dsaidx_q_rope_quant_fold")


def dsaidx_k_norm_rope_quant_store(k: DsaidxKArgs, rope: DsaidxRope, stream=None) -> None:
    _check(lib().dsaidx_k_norm_rope_quant_store(ctypes.byref(k), ctypes.byref(rope),
                                                _stream_handle(stream)),
           "dsaidx_k_norm_rope_quant_store")


def dsaidx_qk_fused(q: DsaidxQArgs, k: DsaidxKArgs, rope: DsaidxRope, stream=None) -> None:
    _check(lib().dsaidx_qk_fused(ctypes.byref(q), ctypes.byref(k), ctypes.byref(rope),
                                 _stream_handle(stream)), "dsaidx_qk_fused")


def dsaidx_proj_k_norm_rope_quant_store(proj: "DsaidxProjArgs", k: DsaidxKArgs, rope: DsaidxRope,
                                        stream=None) -> None:
    _check(lib().dsaidx_proj_k_norm_rope_quant_store(ctypes.byref(proj), ctypes.byref(k),
                                                     ctypes.byref(rope), _stream_handle(stream)),
           "dsaidx_proj_k_norm_rope_quant_store")


def dsaidx_k_only_prepare_store(k: DsaidxKArgs, rope: DsaidxRope, stream=None) -> None:
    _check(lib().dsaidx_k_only_prepare_store(ctypes.byref(k), ctypes.byref(rope),
                                             _stream_handle(stream)), "dsaidx_k_only_prepare_store")


def dsaidx_fp8_encode_selftest(inp, out, scale_exp: int = 0, stream=None) -> None:
    """out = E4M3FN(inp / 2^scale_exp) with the kernels' device conversion.
    inp: float32 device tensor (contiguous, inp / 2^scale_exp in [-448, 448]);
    out: 1-byte device tensor with as many elements."""
    _on_device(inp=inp, out=out)
    _need(inp.is_contiguous() and out.is_contiguous() and inp.numel() == out.numel()
          and out.element_size() == 1, "contiguous float32 input and 1-byte output of equal size")
    _check(lib().dsaidx_fp8_encode_selftest(ctypes.c_void_p(_ptr(inp)), ctypes.c_void_p(_ptr(out)),
                                            inp.numel(), int(scale_exp), _stream_handle(stream)),
           "dsaidx_fp8_encode_selftest")


def dsaidx_topk_workspace_bytes(rows: int, cols: int, k: int) -> int:
    """Workspace bytes dsaidx_topk_per_row needs for this shape (0 for most)."""
    n = lib().dsaidx_topk_workspace_bytes(int(rows), int(cols), int(k))
    if n < 0:
        raise DsaidxError(DSAIDX_ERR_INVALID_ARGUMENT, "dsaidx_topk_workspace_bytes")
    return n


def dsaidx_topk_per_row(logits, k: int, out, lengths=None, stream=None, workspace=None) -> None:
    """logits: float32 device tensor [rows, cols] with unit column stride and a
    row stride that is a multiple of 4; lengths: int32 [rows] or None; out:
    contiguous int32 [rows, k]; workspace: a contiguous device tensor of at
    least dsaidx_topk_workspace_bytes(rows, cols, k) bytes, or None to have one
    allocated here when that size is not 0 (keep one to reuse, e.g. under graph
    capture)."""
    import torch
    _on_device(logits=logits, out=out, lengths=lengths, workspace=workspace)
    _need(logits.dtype == torch.float32 and logits.dim() == 2 and logits.stride(1) == 1,
          "logits must be float32 [rows, cols] with unit column stride")
    rows, cols = logits.shape
    _need(out.dtype == torch.int32 and tuple(out.shape) == (rows, k) and out.is_contiguous(),
          "out must be contiguous int32 [rows, k]")
    if lengths is not None:
        _need(lengths.dtype == torch.int32 and lengths.numel() == rows and lengths.is_contiguous(),
              "lengths must be contiguous int32 [rows]")
    ws_bytes = 0
    if workspace is None:
        need = dsaidx_topk_workspace_bytes(rows, cols, k)
        if need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=logits.device)
    if workspace is not None:
        _need(workspace.is_contiguous(), "workspace must be contiguous")
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().dsaidx_topk_per_row(ctypes.c_void_p(_ptr(logits)), logits.stride(0) if rows else cols,
                                     ctypes.c_void_p(_ptr(lengths)), rows, cols, int(k),
                                     ctypes.c_void_p(_ptr(out)), ctypes.c_void_p(_ptr(workspace)),
                                     ws_bytes, _stream_handle(stream)),
           "dsaidx_topk_per_row")


DSAIDX_HBM_COPY = 0
DSAIDX_HBM_READ = 1
DSAIDX_HBM_WRITE = 2


def dsaidx_hbm_stream(mode: int, src, dst, nbytes: int, word: int = 0, stream=None) -> None:
    """Reference HBM stream (a measurement helper): copy, read or write nbytes
    with the preparation kernel's access pattern.  src / dst: contiguous
    device tensors of at least nbytes (dst at least 16 bytes for a read)."""
    _on_device(src=src, dst=dst)
    for t in (src, dst):
        if t is not None:
            _need(t.is_contiguous(), "src / dst must be contiguous")
    if mode != DSAIDX_HBM_WRITE:
        _need(src is not None and src.numel() * src.element_size() >= nbytes, "src too small")
    need_dst = 16 if mode == DSAIDX_HBM_READ else nbytes
    _need(dst is not None and dst.numel() * dst.element_size() >= need_dst, "dst too small")
    _check(lib().dsaidx_hbm_stream(int(mode), ctypes.c_void_p(_ptr(src)), ctypes.c_void_p(_ptr(dst)),
                                   int(nbytes), int(word) & 0xFFFFFFFF, _stream_handle(stream)),
           "dsaidx_hbm_stream")


def dsaidx_topk_per_row_noalloc(logits, k: int, out, lengths=None, stream=None) -> None:
    """dsaidx_topk_per_row without a workspace argument and without any
    allocation, here or in the library: rows longer than 32768 logits use the
    library's own 16 MiB device array (calls on one GPU must be ordered on one
    stream).  Same tensor rules as dsaidx_topk_per_row."""
    import torch
    _on_device(logits=logits, out=out, lengths=lengths)
    _need(logits.dtype == torch.float32 and logits.dim() == 2 and logits.stride(1) == 1,
          "logits must be float32 [rows, cols] with unit column stride")
    rows, cols = logits.shape
    _need(out.dtype == torch.int32 and tuple(out.shape) == (rows, k) and out.is_contiguous(),
          "out must be contiguous int32 [rows, k]")
    if lengths is not None:
        _need(lengths.dtype == torch.int32 and lengths.numel() == rows and lengths.is_contiguous(),
              "lengths must be contiguous int32 [rows]")
    _check(lib().dsaidx_topk_per_row_noalloc(ctypes.c_void_p(_ptr(logits)),
                                             logits.stride(0) if rows else cols,
                                             ctypes.c_void_p(_ptr(lengths)), rows, cols, int(k),
                                             ctypes.c_void_p(_ptr(out)), _stream_handle(stream)),
           "dsaidx_topk_per_row_noalloc")


def dsaidx_mqa_logits(args: DsaidxLogitsArgs, stream=None) -> None:
    _check(lib().dsaidx_mqa_logits(ctypes.byref(args), _stream_handle(stream)), "dsaidx_mqa_logits")


# ------------------------------------------- struct builders from tensors ----

def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _on_device(**tensors):
    """Every given tensor (None skipped) lives on the current GPU.  The library
    takes plain device pointers and never reads them on the host, so a host
    tensor or one on another device must be refused here, before any launch."""
    import torch
    for name, t in tensors.items():
        if t is None:
            continue
        _need(isinstance(t, torch.Tensor) and t.is_cuda, "%s must be a GPU tensor" % name)
        _need(t.device.index == torch.cuda.current_device(),
              "%s is on cuda:%d, not on the current device cuda:%d"
              % (name, t.device.index, torch.cuda.current_device()))


def rope_args(cos, sin, rope_dim: int = 64, style: int = DSAIDX_ROPE_NEOX) -> DsaidxRope:
    """cos, sin: float32 [P, >= rope_dim/2] views with unit column stride and
    a common row stride (e.g. the two halves of one [P, rope_dim] cache)."""
    import torch
    _on_device(cos=cos, sin=sin)
    _need(cos.dtype == torch.float32 and sin.dtype == torch.float32, "cos/sin must be float32")
    _need(cos.dim() == 2 and sin.dim() == 2 and cos.shape[0] == sin.shape[0], "cos/sin [P, n]")
    _need(cos.stride(1) == 1 and sin.stride(1) == 1 and cos.stride(0) == sin.stride(0),
          "cos/sin need unit column stride and one row stride")
    return DsaidxRope(_ptr(cos), _ptr(sin), cos.stride(0), cos.shape[0], rope_dim, style)


def q_args(q, weights, positions, q_fp8, weights_out, q_scale_out=None,
           weight_scale: float = 1.0) -> DsaidxQArgs:
    """q: bf16 [T, H, 128] (unit inner stride); weights: bf16 [T, H] (unit
    inner stride); positions int64 [T]; q_fp8 uint8 or float8_e4m3fn
    [T, H, 128] contiguous; weights_out (and q_scale_out) float32 [T, H]
    contiguous."""
    import torch
    _on_device(q=q, weights=weights, positions=positions, q_fp8=q_fp8, weights_out=weights_out,
               q_scale_out=q_scale_out)
    _need(q.dtype == torch.bfloat16 and q.dim() == 3 and q.shape[2] == ROW and q.stride(2) == 1,
          "q must be bf16 [T, H, 128] with unit inner stride")
    T, H = q.shape[0], q.shape[1]
    _need(weights.dtype == torch.bfloat16 and tuple(weights.shape) == (T, H)
          and weights.stride(1) == 1, "weights must be bf16 [T, H] with unit inner stride")
    _need(positions.dtype == torch.int64 and positions.numel() == T and positions.is_contiguous(),
          "positions must be contiguous int64 [T]")
    _need(q_fp8.element_size() == 1 and tuple(q_fp8.shape) == (T, H, ROW) and q_fp8.is_contiguous(),
          "q_fp8 must be a contiguous 1-byte [T, H, 128] tensor")
    for name, t in (("weights_out", weights_out), ("q_scale_out", q_scale_out)):
        if t is not None:
            _need(t.dtype == torch.float32 and tuple(t.shape) == (T, H) and t.is_contiguous(),
                  "%s must be contiguous float32 [T, H]" % name)
    return DsaidxQArgs(_ptr(q), q.stride(0), q.stride(1), _ptr(weights), weights.stride(0),
                       _ptr(positions), T, H, float(weight_scale), _ptr(q_fp8),
                       _ptr(weights_out), _ptr(q_scale_out))


def k_args(k, ln_gamma, ln_beta, ln_eps: float, positions, out_cache_loc, k_cache,
           k_scale=None, flags: int = 0, page_size: int = 0, num_slots=None) -> DsaidxKArgs:
    """k: bf16 [T, 128] (unit inner stride), or None for the projection entry
    (T is then the length of positions); ln_gamma/ln_beta float32 [128];
    positions/out_cache_loc int64 [T].

    Planar cache (default): k_cache 1-byte [S, >=128] (unit inner stride;
    codes go to the first 128 bytes of each row), k_scale float32 [S].
    Paged cache (flags has DSAIDX_K_PAGED_CACHE): k_cache a contiguous 1-byte
    tensor of num_slots * 132 bytes holding pages of page_size slots (code
    rows, then fp32 scales); k_scale unused.  DSAIDX_K_BF16_ROUND_ONCE or
    DSAIDX_K_BF16_INTERMEDIATE selects one of the two readings of the unfused
    (bf16) K-cache writer."""
    import torch
    _on_device(k=k, ln_gamma=ln_gamma, ln_beta=ln_beta, positions=positions,
               out_cache_loc=out_cache_loc, k_cache=k_cache, k_scale=k_scale)
    if k is None:   # the projection entry computes the key itself
        T = positions.numel()
    else:
        _need(k.dtype == torch.bfloat16 and k.dim() == 2 and k.shape[1] == ROW and k.stride(1) == 1,
              "k must be bf16 [T, 128] with unit inner stride")
        T = k.shape[0]
    for name, t in (("ln_gamma", ln_gamma), ("ln_beta", ln_beta)):
        _need(t.dtype == torch.float32 and t.numel() == ROW and t.is_contiguous(),
              "%s must be contiguous float32 [128]" % name)
    for name, t in (("positions", positions), ("out_cache_loc", out_cache_loc)):
        _need(t.dtype == torch.int64 and t.numel() == T and t.is_contiguous(),
              "%s must be contiguous int64 [T]" % name)
    _need(k_cache.element_size() == 1, "k_cache must be a 1-byte tensor")
    if flags & DSAIDX_K_PAGED_CACHE:
        _need(k_cache.is_contiguous(), "a paged k_cache must be contiguous")
        S = int(num_slots) if num_slots is not None else k_cache.numel() // PAGED_SLOT_BYTES
        _need(k_cache.numel() >= S * PAGED_SLOT_BYTES, "paged k_cache smaller than num_slots * 132")
        row_stride, scale_ptr = 0, _ptr(k_scale)
    else:
        _need(k_cache.dim() == 2 and k_cache.shape[1] >= ROW and k_cache.stride(1) == 1,
              "k_cache must be a 1-byte [S, >=128] tensor")
        S = k_cache.shape[0]
        _need(k_scale is not None and k_scale.dtype == torch.float32 and k_scale.numel() == S
              and k_scale.is_contiguous(), "k_scale must be contiguous float32 [S]")
        row_stride, scale_ptr = k_cache.stride(0), _ptr(k_scale)
    return DsaidxKArgs(_ptr(k), k.stride(0) if k is not None else ROW, _ptr(ln_gamma), _ptr(ln_beta),
                       float(ln_eps),
                       int(flags), _ptr(positions), _ptr(out_cache_loc), T, _ptr(k_cache),
                       row_stride, scale_ptr, S, int(page_size))


def proj_args(hidden, weight, gates_out, k_out=None) -> DsaidxProjArgs:
    """hidden: bf16 [T, d] with unit inner stride; weight: bf16 [128 + H, d]
    with unit inner stride (a Linear layer's [out, in] layout); gates_out:
    bf16 [T, H] with unit inner stride; k_out: bf16 [T, 128] with unit inner
    stride, or None."""
    import torch
    _on_device(hidden=hidden, weight=weight, gates_out=gates_out, k_out=k_out)
    _need(hidden.dtype == torch.bfloat16 and hidden.dim() == 2 and hidden.stride(1) == 1,
          "hidden must be bf16 [T, d] with unit inner stride")
    T, d = hidden.shape
    _need(weight.dtype == torch.bfloat16 and weight.dim() == 2 and weight.shape[1] == d
          and weight.shape[0] > ROW and weight.stride(1) == 1,
          "weight must be bf16 [128 + H, d] with unit inner stride")
    H = weight.shape[0] - ROW
    _need(gates_out.dtype == torch.bfloat16 and tuple(gates_out.shape) == (T, H)
          and gates_out.stride(1) == 1, "gates_out must be bf16 [T, H] with unit inner stride")
    if k_out is not None:
        _need(k_out.dtype == torch.bfloat16 and tuple(k_out.shape) == (T, ROW) and k_out.stride(1) == 1,
              "k_out must be bf16 [T, 128] with unit inner stride")
    return DsaidxProjArgs(_ptr(hidden), hidden.stride(0) if T else d, _ptr(weight), weight.stride(0), d,
                          H, 0, _ptr(gates_out), gates_out.stride(0) if T else H, _ptr(k_out),
                          k_out.stride(0) if (k_out is not None and T) else ROW)


def logits_args(q_fp8, weights, k_cache, logits, k_scale=None, key_slots=None, lengths=None,
                flags: int = 0, page_size: int = 0, num_slots=None) -> DsaidxLogitsArgs:
    """q_fp8: 1-byte [T, H, 128] contiguous (16-byte aligned); weights: float32
    [T, H] contiguous; logits: float32 [T, N] with unit column stride (N keys);
    key_slots: int32 [N] or None (key s is slot s); lengths: int32 [T] or
    None.  The cache arguments are those of k_args (read only)."""
    import torch
    _on_device(q_fp8=q_fp8, weights=weights, k_cache=k_cache, logits=logits, k_scale=k_scale,
               key_slots=key_slots, lengths=lengths)
    _need(q_fp8.element_size() == 1 and q_fp8.dim() == 3 and q_fp8.shape[2] == ROW
          and q_fp8.is_contiguous(), "q_fp8 must be a contiguous 1-byte [T, H, 128] tensor")
    T, H = q_fp8.shape[0], q_fp8.shape[1]
    _need(weights.dtype == torch.float32 and tuple(weights.shape) == (T, H) and weights.is_contiguous(),
          "weights must be contiguous float32 [T, H]")
    _need(logits.dtype == torch.float32 and logits.dim() == 2 and logits.shape[0] == T
          and logits.stride(1) == 1, "logits must be float32 [T, N] with unit column stride")
    N = logits.shape[1]
    if key_slots is not None:
        _need(key_slots.dtype == torch.int32 and key_slots.numel() == N and key_slots.is_contiguous(),
              "key_slots must be contiguous int32 [N]")
    if lengths is not None:
        _need(lengths.dtype == torch.int32 and lengths.numel() == T and lengths.is_contiguous(),
              "lengths must be contiguous int32 [T]")
    _need(k_cache.element_size() == 1, "k_cache must be a 1-byte tensor")
    if flags & DSAIDX_K_PAGED_CACHE:
        _need(k_cache.is_contiguous(), "a paged k_cache must be contiguous")
        S = int(num_slots) if num_slots is not None else k_cache.numel() // PAGED_SLOT_BYTES
        _need(k_cache.numel() >= S * PAGED_SLOT_BYTES, "paged k_cache smaller than num_slots * 132")
        row_stride = 0
    else:
        _need(k_cache.dim() == 2 and k_cache.shape[1] >= ROW and k_cache.stride(1) == 1,
              "k_cache must be a 1-byte [S, >=128] tensor")
        S = k_cache.shape[0]
        _need(k_scale is not None and k_scale.dtype == torch.float32 and k_scale.numel() == S
              and k_scale.is_contiguous(), "k_scale must be contiguous float32 [S]")
        row_stride = k_cache.stride(0)
    return DsaidxLogitsArgs(_ptr(q_fp8), _ptr(weights), T, H, int(flags), _ptr(k_cache), row_stride,
                            _ptr(k_scale), S, int(page_size), _ptr(key_slots), N, _ptr(lengths),
                            _ptr(logits), logits.stride(0) if T else N)
