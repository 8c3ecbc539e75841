"""Shared helpers of the GPU parity tests: put a workload on the device in a
chosen layout, run an entry point through the C ABI, run the oracle on the
same inputs, and compare by the acceptance rules:

  * ue8m0 scales and cache slot placement: exact;
  * fp8 codes: at most one code apart (ordinal distance, +0 == -0) on at most
    0.1% of the elements of each output;
  * folded weights: relative error <= 1e-6 (expected exact: the scale is a
    power of two and the multiplication order is fixed).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import rope_fp8_quant_amd as R
from rope_fp8_quant_amd import workloads as W

ROW = 128
SENTINEL = 0xA5


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


class DeviceCase:
    """A workload on the device.

    q_head_pad     extra bf16 elements after each head vector (padded head stride)
    gemm_layout    k and weights as column slices of one [T, 128 + H] bf16 buffer,
                   the layout of a fused wk/weights projection output
    combined_table cos/sin as the two halves of one [P, rope_dim] buffer
    cache_row_pad  extra bytes after each 128-byte cache row
    k_flags        DSAIDX_K_* bits (bf16-intermediate writer, paged cache)
    page_size      slots per page of the paged cache
    """

    def __init__(self, wl: W.Workload, q_head_pad=0, gemm_layout=False, combined_table=False,
                 cache_row_pad=0, q_scale_out=True, k_flags=0, page_size=0):
        self.wl = wl
        self.k_flags, self.page_size = k_flags, page_size
        T, H = wl.T, wl.H
        if q_head_pad:
            buf = torch.zeros((T, H, ROW + q_head_pad), dtype=torch.bfloat16, device="cuda")
            buf[:, :, :ROW] = dev_bf16(wl.q)
            self.q = buf[:, :, :ROW]
        else:
            self.q = dev_bf16(wl.q)
        if gemm_layout:
            buf = torch.zeros((T, ROW + H), dtype=torch.bfloat16, device="cuda")
            buf[:, :ROW] = dev_bf16(wl.k)
            buf[:, ROW:] = dev_bf16(wl.weights)
            self.k, self.weights = buf[:, :ROW], buf[:, ROW:]
        else:
            self.k, self.weights = dev_bf16(wl.k), dev_bf16(wl.weights)
        half = wl.rope_dim // 2
        if combined_table:
            tab = torch.cat([dev(wl.cos), dev(wl.sin)], dim=1).contiguous()
            self.cos, self.sin = tab[:, :half], tab[:, half:]
        else:
            self.cos, self.sin = dev(wl.cos), dev(wl.sin)
        self.positions = dev(wl.positions.astype(np.int64))
        self.loc = dev(wl.out_cache_loc.astype(np.int64))
        self.gamma, self.beta = dev(wl.gamma), dev(wl.beta)
        self.q_fp8 = torch.full((T, H, ROW), SENTINEL, dtype=torch.uint8, device="cuda")
        self.w_out = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
        self.q_scale = (torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
                        if q_scale_out else None)
        if k_flags & R.DSAIDX_K_PAGED_CACHE:
            self.cache_full = torch.full((wl.num_slots * (ROW + 4),), SENTINEL, dtype=torch.uint8,
                                         device="cuda")
            self.k_cache = self.cache_full
            self.k_scale = None
        else:
            cache = torch.full((wl.num_slots, ROW + cache_row_pad), SENTINEL, dtype=torch.uint8,
                               device="cuda")
            self.cache_full = cache
            self.k_cache = cache[:, :ROW]
            self.k_scale = torch.full((wl.num_slots,), float("nan"), dtype=torch.float32,
                                      device="cuda")

    def rope(self):
        return R.rope_args(self.cos, self.sin, self.wl.rope_dim, self.wl.style)

    def qa(self):
        return R.q_args(self.q, self.weights, self.positions, self.q_fp8, self.w_out,
                        self.q_scale, self.wl.weight_scale)

    def ka(self):
        return R.k_args(self.k, self.gamma, self.beta, self.wl.eps, self.positions, self.loc,
                        self.k_cache, self.k_scale, flags=self.k_flags, page_size=self.page_size,
                        num_slots=self.wl.num_slots)

    def run(self, entry: str):
        if entry == "fused":
            R.dsaidx_qk_fused(self.qa(), self.ka(), self.rope())
        elif entry == "q":
            R.dsaidx_q_rope_quant_fold(self.qa(), self.rope())
        elif entry == "k":
            R.dsaidx_k_norm_rope_quant_store(self.ka(), self.rope())
        elif entry == "k_only":
            R.dsaidx_k_only_prepare_store(self.ka(), self.rope())
        elif entry == "q+k":
            R.dsaidx_q_rope_quant_fold(self.qa(), self.rope())
            R.dsaidx_k_norm_rope_quant_store(self.ka(), self.rope())
        else:
            raise ValueError(entry)
        torch.cuda.synchronize()

    def host(self):
        out = dict(q_fp8=self.q_fp8.cpu().numpy(), w_out=self.w_out.cpu().numpy(),
                   k_cache=self.cache_full.cpu().numpy())
        if self.k_scale is not None:
            out["k_scale"] = self.k_scale.cpu().numpy()
        if self.q_scale is not None:
            out["q_scale"] = self.q_scale.cpu().numpy()
        return out


# -------------------------------------------------------------- oracle ----

def oracle_q(wl: W.Workload, tokens=None):
    q, w, pos = wl.q, wl.weights, wl.positions
    if tokens is not None:
        q, w, pos = q[tokens], w[tokens], pos[tokens]
    return oracle.q_side(q, w, pos, wl.cos, wl.sin, wl.rope_dim, wl.style, wl.weight_scale)


def bf16_mode_of(k_flags: int) -> int:
    """The oracle's bf16_mode for a set of DSAIDX_K_* flags."""
    if k_flags & R.DSAIDX_K_BF16_INTERMEDIATE:
        return 1
    return 2 if k_flags & R.DSAIDX_K_BF16_ROUND_ONCE else 0


def oracle_k(wl: W.Workload, cache_row_pad=0, k_flags=0, page_size=0):
    bf16_mode = bf16_mode_of(k_flags)
    if k_flags & R.DSAIDX_K_PAGED_CACHE:
        buf = np.full(wl.num_slots * (ROW + 4), SENTINEL, np.uint8)
        oracle.k_side_paged(wl.k, wl.gamma, wl.beta, wl.eps, wl.positions, wl.out_cache_loc,
                            wl.cos, wl.sin, buf, page_size, wl.num_slots, wl.rope_dim, wl.style,
                            bf16_mode)
        return split_paged(buf, page_size, wl.num_slots)
    kc = np.full((wl.num_slots, ROW + cache_row_pad), SENTINEL, np.uint8)
    ks = np.full(wl.num_slots, np.nan, np.float32)
    oracle.k_side(wl.k, wl.gamma, wl.beta, wl.eps, wl.positions, wl.out_cache_loc, wl.cos,
                  wl.sin, kc[:, :ROW], ks, wl.rope_dim, wl.style, bf16_mode)
    return kc, ks


def split_paged(buf: np.ndarray, page_size: int, num_slots: int):
    """Code rows [S, 128] and scales [S] of a page-interleaved cache buffer
    (pages of page_size code rows followed by page_size fp32 scales)."""
    pages = buf.reshape(num_slots // page_size, page_size * (ROW + 4))
    codes = pages[:, :page_size * ROW].reshape(num_slots, ROW)
    scales = np.ascontiguousarray(pages[:, page_size * ROW:]).view(np.float32).reshape(num_slots)
    return codes, scales


# ---------------------------------------------------------- comparison ----

def ordinal(c: np.ndarray) -> np.ndarray:
    mag = (c & 0x7F).astype(np.int32)
    return np.where(c & 0x80, -mag, mag)


def compare_codes(got: np.ndarray, want: np.ndarray, what: str, report: dict):
    assert got.shape == want.shape, what
    d = np.abs(ordinal(got) - ordinal(want))
    n_diff = int(np.count_nonzero(d))
    report[what] = dict(elements=int(d.size), differ=n_diff, max_steps=int(d.max(initial=0)),
                        bytes_differ=int(np.count_nonzero(got != want)))
    assert d.max(initial=0) <= 1, (what, report[what])
    assert n_diff <= 0.001 * d.size, (what, report[what])


def compare_exact_f32(got: np.ndarray, want: np.ndarray, what: str):
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), what


def compare_rel(got: np.ndarray, want: np.ndarray, what: str, rel=1e-6):
    err = np.abs(got.astype(np.float64) - want.astype(np.float64))
    assert np.all(err <= rel * np.abs(want.astype(np.float64))), (what, float(err.max()))


def check_q(out: dict, wl: W.Workload, report: dict, tokens=None):
    """Query side.  Beyond the acceptance rules, the query arithmetic is fixed
    op for op (bf16 -> fp32 exact, separately rounded products and sums, a
    power-of-two scale), so the codes and folded weights must match the oracle
    byte for byte."""
    q8, wo, qs = oracle_q(wl, tokens)
    got_q8 = out["q_fp8"] if tokens is None else out["q_fp8"][tokens]
    got_wo = out["w_out"] if tokens is None else out["w_out"][tokens]
    compare_codes(got_q8, q8, "q_fp8", report)
    compare_rel(got_wo, wo, "weights_out")
    report["weights_out_bit_exact"] = bool(np.array_equal(got_wo.view(np.uint32), wo.view(np.uint32)))
    assert report["q_fp8"]["bytes_differ"] == 0, report["q_fp8"]
    assert report["weights_out_bit_exact"]
    if "q_scale" in out:
        got_qs = out["q_scale"] if tokens is None else out["q_scale"][tokens]
        compare_exact_f32(got_qs, qs, "q_scale")


def k_rows_near_scale_boundary(wl: W.Workload, k_flags=0) -> int:
    """Key rows whose amax (after LayerNorm and RoPE, in the oracle) lies within
    4 fp32 ulps of a scale boundary 1.75 * 2^E, where a LayerNorm reduction
    order different from the oracle's could move the ue8m0 exponent.  The
    scales are still compared exactly; this count says how many rows that
    exactness rests on the fp64 sums for."""
    bf16_mode = bf16_mode_of(k_flags)
    y, _ = oracle.k_values(wl.k, wl.gamma, wl.beta, wl.eps, wl.positions, wl.cos, wl.sin,
                           wl.rope_dim, wl.style, bf16_mode)
    ag = np.maximum(np.abs(y).max(axis=1), np.float32(1e-4)).astype(np.float32)
    mant = (ag.view(np.uint32) & 0x7FFFFF).astype(np.int64)
    return int(np.count_nonzero(np.abs(mant - 0x600000) <= 4))


def check_k(out: dict, wl: W.Workload, report: dict, cache_row_pad=0, k_flags=0, page_size=0):
    kc, ks = oracle_k(wl, cache_row_pad, k_flags, page_size)
    report["k_rows_near_scale_boundary"] = k_rows_near_scale_boundary(wl, k_flags)
    if k_flags & R.DSAIDX_K_PAGED_CACHE:
        got_kc, got_ks = split_paged(out["k_cache"], page_size, wl.num_slots)
    else:
        got_kc, got_ks = out["k_cache"], out["k_scale"]
    # slot placement and scales: exact (NaN sentinel compared bitwise)
    compare_exact_f32(got_ks, ks, "k_scale")
    touched = np.zeros(wl.num_slots, bool)
    loc = wl.out_cache_loc
    touched[loc[(loc >= 0) & (loc < wl.num_slots)]] = True
    assert np.all(got_kc[~touched] == SENTINEL), "cache rows outside out_cache_loc changed"
    assert np.all(got_kc[:, ROW:] == SENTINEL), "cache row padding changed"
    compare_codes(got_kc[touched, :ROW], kc[touched, :ROW], "k_cache", report)
    # Beyond the acceptance rule: on these seeded inputs the kernels' fp64
    # LayerNorm sums (a different order from the oracle's) leave the fp32 mean,
    # variance and reciprocal root the same, so the codes match byte for byte.
    # The kernels are deterministic, so this holds run after run.
    assert report["k_cache"]["bytes_differ"] == 0, report["k_cache"]


# ------------------------------------------------------- index logits ----

def logits_bound(q8: np.ndarray, w: np.ndarray, codes: np.ndarray, scale: np.ndarray,
                 slots: np.ndarray) -> np.ndarray:
    """Per-entry tolerance of the index logits [T, len(slots)], from the matrix
    unit's arithmetic: every E4M3 x E4M3 product is exact, but the unit aligns
    the 128 products of a dot to the largest one (errors of at most 2^-10.65 of
    the largest product were seen on MI355X), then the gate multiply and head
    sum round in fp32.  Allowed: k_scale * sum_h |w| * (2^-8 * max|q| * max|k|
    + 2^-16 * sum_d |q k|)."""
    from oracle import logits as LG
    dec = np.abs(LG.decode_table())
    qa, ka = dec[q8], dec[codes[slots, :ROW]]
    absdots = (qa.reshape(-1, ROW) @ ka.T).reshape(q8.shape[0], q8.shape[1], -1)
    per_dot = 2.0 ** -8 * qa.max(axis=2)[:, :, None] * ka.max(axis=1)[None, None, :] + 2.0 ** -16 * absdots
    b = np.einsum("th,ths->ts", np.abs(w.astype(np.float64)), per_dot)
    return b * scale.astype(np.float64)[slots][None, :] + 1e-30
