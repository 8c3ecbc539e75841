#!/usr/bin/env python3
"""Throughput of the fused DSA-indexer Q/K preparation on one MI355X.

One step = one dsaidx_qk_fused call over the whole long-prefill batch
(T = 65536 tokens at positions 196608..262143, H = 64 heads, D = 128,
rope_dim 64 NeoX, cos/sin table of 262144 rows, 262144-slot index-K cache,
contiguous slots): query RoPE + E4M3FN/ue8m0 quantisation + head-gate fold
and key LayerNorm + RoPE + quantisation + cache store, in one dispatch.
Inputs are resident in HBM before timing starts; the 1.68 GB a step moves is
far larger than the 256 MB last-level cache, so every step streams from HBM.

Printed: one JSON line with tokens/s (value), ms per step, the HBM roofline
of the kernel (algorithmic bytes / measured launch time against 8 TB/s), the
oracle's CPU throughput on a bounded sample, and secondary measurements
(decode-batch microseconds per call, the 8192-token prefill chunk with buffer
rotation, the k-only decode path, the top-k per row and index-logits steps
that follow, and reference HBM streams -- copy, read-only, write-only -- that
give the achievable rate for this kernel's mix of reads and writes).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused indexer Q/K prep tokens/s and achieved HBM GB/s (% peak); \u00b5s/call"
PEAK_HBM_GBPS = 8000.0
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense fp8 matrix peak (no sparsity)
WARM_MS = 100.0      # warm-up of the bandwidth-bound secondary measurements (GPU clock ramp)
WARM_MS_MAIN = 200.0   # warm-up of the headline measurement, on top of --warmup steps
WARM_MS_LATENCY = 20.0   # the latency-bound decode ones (insensitive to it; keeps traces small)
KERNEL_SOURCES = [os.path.join(ROOT, "rope_fp8_quant_amd", "csrc", f)
                  for f in ("dsaidx_kernels.hip", "dsaidx_prep_device.h", "dsaidx_internal.h",
                            "dsaidx_api.cpp")]
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "hbm_traffic_indexer_qk_prep_long_prefill_T65536.txt")


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the prep kernel's sources with comments and blank space
    removed, so that a comment edit does not void the recorded counters."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def recorded_traffic(expected_hash: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when there is none or it was taken on other kernel sources."""
    if not os.path.exists(TRAFFIC_SUMMARY):
        return None
    text = open(TRAFFIC_SUMMARY).read()
    m_hash = re.search(r"^kernel_source_sha256_16:\s*([0-9a-f]+)", text, re.M)
    m_bytes = re.search(r"^hbm_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    if not m_hash or not m_bytes or m_hash.group(1) != expected_hash:
        return None
    return float(m_bytes.group(1))


class Case:
    """Device buffers of one workload for the fused call (inputs copied once)."""

    def __init__(self, wl, torch, R, k_flags=0, page_size=0):
        import numpy as np
        self.wl = wl
        T, H = wl.T, wl.H

        def bf16(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)

        self.q, self.k, self.w = bf16(wl.q), bf16(wl.k), bf16(wl.weights)
        self.pos = torch.from_numpy(wl.positions).cuda()
        self.loc = torch.from_numpy(wl.out_cache_loc).cuda()
        self.cos = torch.from_numpy(wl.cos).cuda()
        self.sin = torch.from_numpy(wl.sin).cuda()
        self.gamma = torch.from_numpy(wl.gamma).cuda()
        self.beta = torch.from_numpy(wl.beta).cuda()
        self.q_fp8 = torch.empty((T, H, 128), dtype=torch.uint8, device="cuda")
        self.w_out = torch.empty((T, H), dtype=torch.float32, device="cuda")
        if k_flags & R.DSAIDX_K_PAGED_CACHE:
            self.k_cache = torch.zeros((wl.num_slots * (128 + 4),), dtype=torch.uint8, device="cuda")
            self.k_scale = None
        else:
            self.k_cache = torch.zeros((wl.num_slots, 128), dtype=torch.uint8, device="cuda")
            self.k_scale = torch.zeros((wl.num_slots,), dtype=torch.float32, device="cuda")
        self.qa = R.q_args(self.q, self.w, self.pos, self.q_fp8, self.w_out)
        self.ka = R.k_args(self.k, self.gamma, self.beta, wl.eps, self.pos, self.loc,
                           self.k_cache, self.k_scale, flags=k_flags, page_size=page_size,
                           num_slots=wl.num_slots)
        self.rope = R.rope_args(self.cos, self.sin, wl.rope_dim, wl.style)


def warm_up(torch, fn, warm_ms):
    """Call fn until at least warm_ms of wall time has passed: the GPU ramps
    its clocks up over tens of milliseconds of load (an 8192-token call timed
    after 20 warmup calls from idle runs about 9 % slower than warm)."""
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < warm_ms:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()


def time_calls(torch, fn, steps, warmup, warm_ms=0.0):
    """Mean milliseconds per call over `steps` back-to-back calls, bracketed by
    HIP events on the stream the calls are enqueued on, after `warmup` calls
    (and at least warm_ms of them, when given)."""
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    if warm_ms > 0:
        warm_up(torch, fn, warm_ms)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def time_graph(torch, fn, calls, replays, warm_ms=WARM_MS_LATENCY):
    """Mean milliseconds per call when `calls` calls are captured in one HIP
    graph and the graph is replayed `replays` times (after warm_ms of replays)."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for _ in range(calls):
            fn()
    g.replay()
    torch.cuda.synchronize()
    warm_up(torch, g.replay, warm_ms)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    start.record(stream)
    for _ in range(replays):
        g.replay()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / (calls * replays)


def cpu_baseline(wl, runs=3, decode_runs=100):
    """The oracle (as it stands) on the host: the whole workload (Q and K
    sides) on every core in this process's affinity set, median of `runs`
    runs; the same on one thread over a leading slice; and the 64-token decode
    batch, median of `decode_runs` calls on one thread and on all cores."""
    import numpy as np

    import oracle
    cores = len(os.sched_getaffinity(0))
    kc = np.zeros((wl.num_slots, 128), np.uint8)
    ks = np.zeros(wl.num_slots, np.float32)

    def run(n, nt):
        t0 = time.perf_counter()
        oracle.q_side(wl.q[:n], wl.weights[:n], wl.positions[:n], wl.cos, wl.sin, wl.rope_dim,
                      wl.style, wl.weight_scale, nthreads=nt)
        oracle.k_side(wl.k[:n], wl.gamma, wl.beta, wl.eps, wl.positions[:n],
                      wl.out_cache_loc[:n], wl.cos, wl.sin, kc, ks, wl.rope_dim, wl.style,
                      nthreads=nt)
        return time.perf_counter() - t0

    ts = sorted(run(wl.T, cores) for _ in range(runs))
    med = ts[len(ts) // 2]
    out = dict(value=wl.T / med, unit="tokens/s", cores=cores, kind="oracle",
               sample="all %d tokens of %s (Q and K sides), median of %d runs (%.2f s each) on %d "
                      "threads (every core in the affinity set)" % (wl.T, wl.name, runs, med, cores))
    n1 = min(wl.T, 2048)
    t1 = sorted(run(n1, 1) for _ in range(runs))
    out["single_thread"] = {"value": n1 / t1[len(t1) // 2], "unit": "tokens/s",
                            "sample": "first %d tokens, 1 thread, median of %d runs" % (n1, runs)}
    # the 64-token decode batch: median microseconds per call
    from rope_fp8_quant_amd import workloads as W
    d = W.named(1)
    dkc = np.zeros((d.num_slots, 128), np.uint8)
    dks = np.zeros(d.num_slots, np.float32)
    for label, nt in (("us_per_call_1_thread", 1), ("us_per_call_all_threads", cores)):
        tt = []
        for _ in range(decode_runs):
            t0 = time.perf_counter()
            oracle.q_side(d.q, d.weights, d.positions, d.cos, d.sin, d.rope_dim, d.style,
                          d.weight_scale, nthreads=nt)
            oracle.k_side(d.k, d.gamma, d.beta, d.eps, d.positions, d.out_cache_loc, d.cos, d.sin,
                          dkc, dks, d.rope_dim, d.style, nthreads=nt)
            tt.append(time.perf_counter() - t0)
        out.setdefault("decode_batch_T64", {"runs": decode_runs})[label] = sorted(tt)[decode_runs // 2] * 1e6
    return out


def hbm_reference(torch, R, read_bytes, write_bytes, steps=20):
    """The library's reference HBM streams (the prep kernel's access pattern:
    16-byte nontemporal accesses, one-shot grid) over the prep call's own read
    and write byte counts: a copy, a read-only and a write-only stream.  The
    ideal time of a read_bytes + write_bytes mix is read_bytes / read rate +
    write_bytes / write rate."""
    big = max(read_bytes, write_bytes)
    big += (-big) % 16
    src = torch.zeros(big, dtype=torch.uint8, device="cuda")
    dst = torch.empty(big, dtype=torch.uint8, device="cuda")
    rb, wb = read_bytes - read_bytes % 16, write_bytes - write_bytes % 16
    cb = (read_bytes + write_bytes) // 2
    cb -= cb % 16
    ms_copy = time_calls(torch, lambda: R.dsaidx_hbm_stream(R.binding.DSAIDX_HBM_COPY, src, dst, cb),
                         steps, 3, WARM_MS)
    ms_read = time_calls(torch, lambda: R.dsaidx_hbm_stream(R.binding.DSAIDX_HBM_READ, src, dst, rb,
                                                            0xFFFFFFFF), steps, 3, WARM_MS)
    ms_write = time_calls(torch, lambda: R.dsaidx_hbm_stream(R.binding.DSAIDX_HBM_WRITE, None, dst, wb,
                                                             0x5A5A5A5A), steps, 3, WARM_MS)
    del src, dst
    torch.cuda.empty_cache()
    read_gbps = rb / (ms_read * 1e-3) / 1e9
    write_gbps = wb / (ms_write * 1e-3) / 1e9
    return {"copy_GBps": 2 * cb / (ms_copy * 1e-3) / 1e9, "copy_bytes_moved": 2 * cb,
            "read_only_GBps": read_gbps, "read_bytes": rb,
            "write_only_GBps": write_gbps, "write_bytes": wb,
            "mix_ideal_us": (read_bytes / read_gbps + write_bytes / write_gbps) / 1e3}


def topk_measurements(torch, R, W, steps=50):
    """Top-k per row over index logits (index_topk = 2048) on the named
    synthetic workloads: microseconds per call and algorithmic GB/s."""
    out = {}
    for ti in range(len(W.TOPK_NAMED)):
        tw = W.topk_named(ti)
        lg = torch.from_numpy(tw.logits).cuda()
        ln = torch.from_numpy(tw.lengths).cuda()
        rows, cols = tw.logits.shape
        ot = torch.empty((rows, tw.k), dtype=torch.int32, device="cuda")
        nws = R.dsaidx_topk_workspace_bytes(rows, cols, tw.k)
        ws = torch.empty(max(nws, 16), dtype=torch.uint8, device="cuda")
        call = lambda: R.dsaidx_topk_per_row(lg, tw.k, ot, ln, workspace=ws)
        mst = time_calls(torch, call, steps, 5, WARM_MS)
        # the same calls replayed from a HIP graph: device time without the
        # Python and ctypes enqueue cost, which matters for the short calls
        msg = time_graph(torch, call, 20, 10, WARM_MS)
        bt = W.topk_bytes_per_call(rows, tw.lengths, tw.k)
        out[tw.name] = {"us_per_call": mst * 1e3, "us_per_call_graph": msg * 1e3,
                        "algorithmic_bytes": bt, "achieved_GBps": bt / (mst * 1e-3) / 1e9,
                        "dispatches": 4 if nws else 1, "workspace_bytes": nws}
        del lg, ln, ot, ws
    torch.cuda.empty_cache()
    return out


def logits_measurements(torch, R, W, steps=20):
    """Index logits (fp8 dots on the matrix cores, ReLU, gate-weighted head
    sum, key scale) on the named synthetic workloads: microseconds per call and
    achieved operations against the MI355X dense fp8 peak."""
    out = {}
    for li in range(len(W.LOGITS_NAMED)):
        lw = W.logits_named(li)
        T, H = lw.q_fp8.shape[:2]
        N = len(lw.key_slots)
        dq = torch.from_numpy(lw.q_fp8).cuda()
        dw = torch.from_numpy(lw.weights).cuda()
        dk = torch.from_numpy(lw.k_cache).cuda()
        dks = torch.from_numpy(lw.k_scale).cuda()
        dsl = torch.from_numpy(lw.key_slots).cuda()
        dln = torch.from_numpy(lw.lengths).cuda()
        lo = torch.empty((T, N), dtype=torch.float32, device="cuda")
        args = R.logits_args(dq, dw, dk, lo, k_scale=dks, key_slots=dsl, lengths=dln)
        call = lambda: R.dsaidx_mqa_logits(args)
        mst = time_calls(torch, call, steps, 3, WARM_MS)
        msg = time_graph(torch, call, 10, 5, WARM_MS)
        fl = W.logits_flops_per_call(H, lw.lengths)
        bt = W.logits_bytes_per_call(T, H, N, lw.lengths)
        out[lw.name] = {"us_per_call": mst * 1e3, "us_per_call_graph": msg * 1e3,
                        "T": T, "H": H, "keys": N,
                        "algorithmic_ops": fl, "achieved_TOPs": fl / (mst * 1e-3) / 1e12,
                        "frac_of_fp8_peak": fl / (mst * 1e-3) / 1e12 / PEAK_FP8_TFLOPS,
                        "algorithmic_bytes": bt, "achieved_GBps": bt / (mst * 1e-3) / 1e9}
        del dq, dw, dk, dks, dsl, dln, lo
    torch.cuda.empty_cache()
    return out


PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak (no sparsity)


def proj_measurement(torch, R, W, steps=20):
    """The key / head-gate projection with the key preparation in its
    epilogue, at the long-prefill size: hidden [65536, 7168] bf16 times the
    [192, 7168] weight on the matrix cores, the 128 key columns prepared into
    the 262144-slot cache, the 64 gate columns written as bf16."""
    T, d, H = 65536, 7168, 64
    pw = W.proj_make(T, d, H, seed=4004, name="proj_long_prefill_T65536", table_rows=262144,
                     pos_mode="contiguous", pos_lo=196608, num_slots=262144, slot_mode="contiguous")
    kw = pw.key

    def bf16(a):
        import numpy as np
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)

    hid, wt = bf16(pw.hidden), bf16(pw.weight)
    gates = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    pos = torch.from_numpy(kw.positions).cuda()
    loc = torch.from_numpy(kw.out_cache_loc).cuda()
    gam, bet = torch.from_numpy(kw.gamma).cuda(), torch.from_numpy(kw.beta).cuda()
    cos, sin = torch.from_numpy(kw.cos).cuda(), torch.from_numpy(kw.sin).cuda()
    kc = torch.zeros((kw.num_slots, 128), dtype=torch.uint8, device="cuda")
    ks = torch.zeros((kw.num_slots,), dtype=torch.float32, device="cuda")
    pa = R.proj_args(hid, wt, gates)
    ka = R.k_args(None, gam, bet, kw.eps, pos, loc, kc, ks)
    ra = R.rope_args(cos, sin, kw.rope_dim, kw.style)
    call = lambda: R.dsaidx_proj_k_norm_rope_quant_store(pa, ka, ra)
    ms = time_calls(torch, call, steps, 3, WARM_MS)
    bt = W.proj_bytes_per_call(T, d, H, kw.rope_dim)
    fl = W.proj_flops_per_call(T, d, H)
    del hid, wt, gates, kc, ks
    torch.cuda.empty_cache()
    return {"us_per_call": ms * 1e3, "T": T, "d": d, "H": H, "algorithmic_bytes": bt,
            "achieved_GBps": bt / (ms * 1e-3) / 1e9, "frac_of_hbm_peak": bt / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
            "algorithmic_flops": fl, "achieved_TFLOPs": fl / (ms * 1e-3) / 1e12,
            "frac_of_bf16_peak": fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}


def decode_step_measurement(torch, R, W):
    """One indexer decode step for a 64-request batch at a 16384-key context,
    replayed from a HIP graph: the fused prep call (64 tokens into a
    262144-slot index-K cache), the index logits over 16384 cache slots with
    ragged lengths, and the top-k (k = 2048) per row."""
    import numpy as np
    lw = W.logits_named(0)
    wl = W.make(64, 64, values="sparse_outliers", table_rows=8192, num_slots=lw.k_cache.shape[0],
                slot_mode="random_distinct", seed=1001, name="decode_step_T64")
    c = Case(wl, torch, R)
    c.k_cache.copy_(torch.from_numpy(lw.k_cache))
    c.k_scale.copy_(torch.from_numpy(lw.k_scale))
    T, N, k = 64, len(lw.key_slots), 2048
    dsl = torch.from_numpy(lw.key_slots).cuda()
    dln = torch.from_numpy(lw.lengths).cuda()
    lo = torch.empty((T, N), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    la = R.logits_args(c.q_fp8, c.w_out, c.k_cache, lo, k_scale=c.k_scale, key_slots=dsl, lengths=dln)
    ws = torch.empty(max(R.dsaidx_topk_workspace_bytes(T, N, k), 16), dtype=torch.uint8, device="cuda")

    def step():
        R.dsaidx_qk_fused(c.qa, c.ka, c.rope)
        R.dsaidx_mqa_logits(la)
        R.dsaidx_topk_per_row(lo, k, idx, dln, workspace=ws)

    ms = time_graph(torch, step, 20, 20)
    del c, lo, idx, ws
    torch.cuda.empty_cache()
    return {"us_per_step_graph": ms * 1e3, "tokens": T, "keys": N, "k": k, "dispatches": 3}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--warm-ms", type=float, default=WARM_MS_MAIN,
                    help="milliseconds of warm-up calls before the timed steps (GPU clock ramp)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the decode, prefill-chunk and k-only measurements")
    ap.add_argument("--topk-only", action="store_true",
                    help="time only the top-k-per-row workloads (a JSON object of its own)")
    ap.add_argument("--logits-only", action="store_true",
                    help="time only the index-logits workloads (a JSON object of its own)")
    ap.add_argument("--proj-only", action="store_true",
                    help="time only the projection with the key preparation in its epilogue")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this path has no cross-GPU step (every token and "
              "head is independent), and only --gpus 1 is supported", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import rope_fp8_quant_amd as R
    from rope_fp8_quant_amd import workloads as W

    torch.cuda.set_device(0)
    if not R.dsaidx_device_supported(0):
        raise SystemExit("cuda:0 is not a gfx950 device")
    if args.topk_only:
        print(json.dumps({"topk_per_row": topk_measurements(torch, R, W, args.steps)}), flush=True)
        return
    if args.proj_only:
        print(json.dumps({"proj_long_prefill_T65536_d7168": proj_measurement(torch, R, W, args.steps)}),
              flush=True)
        return
    if args.logits_only:
        print(json.dumps({"mqa_logits": logits_measurements(torch, R, W, min(args.steps, 50))}),
              flush=True)
        return

    log("generating long_prefill_T65536 inputs")
    wl = W.named(4)
    c = Case(wl, torch, R)
    bytes_call = W.bytes_per_call(wl.T, wl.H, "fused", wl.rope_dim)

    def fused():
        R.dsaidx_qk_fused(c.qa, c.ka, c.rope)

    log("timing %d fused steps after %d warmup steps and %.0f ms of warm-up calls"
        % (args.steps, args.warmup, args.warm_ms))
    torch.cuda.synchronize()
    ms = time_calls(torch, fused, args.steps, args.warmup, args.warm_ms)
    achieved = bytes_call / (ms * 1e-3) / 1e9
    src_hash = kernel_source_hash()
    traffic = recorded_traffic(src_hash)
    result = {
        "metric": METRIC,
        "value": wl.T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "T": wl.T, "H": wl.H, "D": 128,
                   "rope_dim": wl.rope_dim, "rope_style": "neox", "positions": "196608..262143",
                   "table_rows": wl.table_rows, "cache_slots": wl.num_slots,
                   "entry": "dsaidx_qk_fused", "inputs": "bf16 q/k/weights",
                   "outputs": "e4m3fn codes + fp32 scales/weights",
                   "algorithmic_bytes_per_step": bytes_call},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS,
                     "traffic": traffic, "kernel_source_sha256_16": src_hash},
        "us_per_call": ms * 1e3,
    }
    del c
    torch.cuda.empty_cache()

    if not args.no_extras:
        log("secondary measurements")
        extras = {}
        # decode batch, 64 tokens: back-to-back calls and graph replay
        wl1 = W.named(1)
        c1 = Case(wl1, torch, R)

        def fused1():
            R.dsaidx_qk_fused(c1.qa, c1.ka, c1.rope)

        ms_eager = time_calls(torch, fused1, 2000, 200, WARM_MS_LATENCY)
        ms_graph = time_graph(torch, fused1, 100, 20)
        # the floor for any dispatch under graph replay: a one-element fill
        tiny = torch.zeros(1, dtype=torch.float32, device="cuda")
        ms_floor = time_graph(torch, lambda: tiny.fill_(1.0), 100, 20)
        extras["decode_batch_T64"] = {"us_per_call_eager": ms_eager * 1e3,
                                      "us_per_call_graph": ms_graph * 1e3,
                                      "bytes_per_call": W.bytes_per_call(64),
                                      "us_per_dispatch_floor_graph": ms_floor * 1e3}
        # one token (the pages' single-request decode): graph replay
        c1t = Case(W.named(1, T=1), torch, R)
        ms_t1 = time_graph(torch, lambda: R.dsaidx_qk_fused(c1t.qa, c1t.ka, c1t.rope), 100, 20)
        extras["decode_T1"] = {"us_per_call_graph": ms_t1 * 1e3, "bytes_per_call": W.bytes_per_call(1)}
        del c1t
        # 512-token decode, interleaved RoPE: fused and k-only
        wl2 = W.named(2)
        c2 = Case(wl2, torch, R)
        ms2 = time_graph(torch, lambda: R.dsaidx_qk_fused(c2.qa, c2.ka, c2.rope), 100, 10)
        ms2k = time_graph(torch, lambda: R.dsaidx_k_only_prepare_store(c2.ka, c2.rope), 100, 10)
        extras["decode_large_interleaved_T512"] = {"us_per_call_fused_graph": ms2 * 1e3,
                                                   "us_per_call_k_only_graph": ms2k * 1e3}
        c2b = Case(wl2, torch, R, k_flags=R.DSAIDX_K_BF16_INTERMEDIATE)
        ms2b = time_graph(torch, lambda: R.dsaidx_k_only_prepare_store(c2b.ka, c2b.rope), 100, 10)
        extras["decode_large_interleaved_T512"]["us_per_call_k_only_bf16_writer_graph"] = ms2b * 1e3
        del c1, c2, c2b
        # the same long prefill into the page-interleaved index-K cache (64-slot pages)
        cp = Case(wl, torch, R, k_flags=R.DSAIDX_K_PAGED_CACHE, page_size=64)
        msp = time_calls(torch, lambda: R.dsaidx_qk_fused(cp.qa, cp.ka, cp.rope), 50, 5, WARM_MS)
        extras["long_prefill_T65536_paged_cache"] = {
            "us_per_call": msp * 1e3, "achieved_GBps": bytes_call / (msp * 1e-3) / 1e9,
            "frac_of_peak": bytes_call / (msp * 1e-3) / 1e9 / PEAK_HBM_GBPS}
        del cp
        torch.cuda.empty_cache()
        # a TP8 rank's share of the long prefill: 8 of the 64 heads (the key
        # row has no head axis, so every rank prepares all of it)
        wl8 = W.make(65536, 8, values="zero_rows", table_rows=262144, pos_mode="contiguous",
                     pos_lo=196608, num_slots=262144, slot_mode="contiguous", seed=1004,
                     name="long_prefill_T65536_H8")
        c8 = Case(wl8, torch, R)
        ms8 = time_calls(torch, lambda: R.dsaidx_qk_fused(c8.qa, c8.ka, c8.rope), 100, 10, WARM_MS)
        b8 = W.bytes_per_call(wl8.T, 8)
        extras["long_prefill_T65536_H8_tp8_share"] = {
            "us_per_call": ms8 * 1e3, "bytes_per_call": b8, "achieved_GBps": b8 / (ms8 * 1e-3) / 1e9,
            "frac_of_peak": b8 / (ms8 * 1e-3) / 1e9 / PEAK_HBM_GBPS}
        del c8, wl8
        torch.cuda.empty_cache()
        # 8192-token prefill chunk: 4 rotating buffer sets (> 800 MB) so no
        # step finds its inputs in the last-level cache
        wl3 = W.named(3)
        sets = [Case(wl3, torch, R) for _ in range(4)]
        it = [0]

        def fused3():
            s = sets[it[0] & 3]
            it[0] += 1
            R.dsaidx_qk_fused(s.qa, s.ka, s.rope)

        ms3 = time_calls(torch, fused3, 200, 20, WARM_MS)
        b3 = W.bytes_per_call(wl3.T)
        extras["prefill_chunk_T8192"] = {"us_per_call": ms3 * 1e3, "tokens_per_s": wl3.T / (ms3 * 1e-3),
                                         "achieved_GBps": b3 / (ms3 * 1e-3) / 1e9,
                                         "frac_of_peak": b3 / (ms3 * 1e-3) / 1e9 / PEAK_HBM_GBPS}
        del sets
        torch.cuda.empty_cache()
        extras.update(topk_measurements(torch, R, W))
        extras.update(logits_measurements(torch, R, W))
        extras["decode_step_T64_ctx16384"] = decode_step_measurement(torch, R, W)
        extras["proj_long_prefill_T65536_d7168"] = proj_measurement(torch, R, W)
        result["secondary"] = extras

    # what plain streams reach with this kernel's access pattern and its own
    # read / write byte counts, and torch's device copy of the same byte count
    rd, wr = W.bytes_per_call_split(wl.T, wl.H, "fused", wl.rope_dim)
    ref = hbm_reference(torch, R, rd, wr)
    ref["prep_read_bytes"], ref["prep_write_bytes"] = rd, wr
    ref["prep_frac_of_mix_ideal"] = ref["mix_ideal_us"] / (ms * 1e3)
    n = bytes_call // 2
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    msc = time_calls(torch, lambda: dst.copy_(src), 20, 3, WARM_MS)
    copy_gbps = 2 * n / (msc * 1e-3) / 1e9
    result.setdefault("secondary", {})["plain_copy"] = {"bytes_moved": 2 * n,
                                                         "achieved_GBps": copy_gbps}
    result["secondary"]["hbm_reference_streams"] = ref
    result["roofline"]["frac_of_plain_copy"] = achieved / copy_gbps
    result["roofline"]["frac_of_mix_ideal"] = ref["prep_frac_of_mix_ideal"]
    del src, dst

    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample")
        result["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
