"""Seeded synthetic inputs for the DSA-indexer Q/K preparation.

This module only draws inputs (numpy, host memory).  It holds none of the
method's arithmetic, and it is the one piece of code that both the GPU path's
tests/benchmark and the CPU oracle's tests use.

Every array has its own random stream, spawned from ``SeedSequence(seed)`` in a
fixed order: q, k, weights, positions, gamma, beta, slots, special structure.
bf16 inputs are drawn in float32 and rounded to bf16 (nearest, ties to even)
by bit arithmetic; they are returned as uint16 bit patterns.

The five named workloads mirror the shapes the pages discuss: a 41-token
decode (the size of the pages' K-cache writer comparison, 41 x 128 values),
a 64-request decode batch, a 512-token decode batch with interleaved RoPE, an
8192-token prefill chunk and a 65536-token prefill deep into a 262144-token
context ([sglang-fuse] Accuracy and Benchmark; [vllm-47335] End-to-end).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

ROW = 128          # head vector / K row width
NEOX = 0
INTERLEAVED = 1
ROPE_BASE = 10000.0

_STREAMS = ("q", "k", "weights", "positions", "gamma", "beta", "slots", "special")


@dataclass
class Workload:
    name: str
    T: int
    H: int
    rope_dim: int
    style: int
    q: np.ndarray            # uint16 bf16 bits [T, H, 128]
    k: np.ndarray            # uint16 bf16 bits [T, 128]
    weights: np.ndarray      # uint16 bf16 bits [T, H]
    positions: np.ndarray    # int64 [T]
    cos: np.ndarray          # float32 [P, rope_dim/2]
    sin: np.ndarray          # float32 [P, rope_dim/2]
    gamma: np.ndarray        # float32 [128]
    beta: np.ndarray         # float32 [128]
    eps: float
    num_slots: int
    out_cache_loc: np.ndarray  # int64 [T]
    weight_scale: float = 1.0
    info: dict = field(default_factory=dict)

    @property
    def table_rows(self) -> int:
        return self.cos.shape[0]


def f32_to_bf16_bits(x: np.ndarray, chunk: int = 1 << 24) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); finite inputs only."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint16)
    for s in range(0, flat.size, chunk):
        u = flat[s:s + chunk].view(np.uint32)
        r = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
        out[s:s + chunk] = (r >> np.uint32(16)).astype(np.uint16)
    return out.reshape(x.shape)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def rope_table(rows: int, rope_dim: int = 64, base: float = ROPE_BASE):
    """cos/sin [rows, rope_dim/2]: angle(p, j) = p * base^(-2j/rope_dim) in
    float64, each rounded to float32.  The table is an input of the method."""
    j = np.arange(rope_dim // 2, dtype=np.float64)
    inv_freq = base ** (-2.0 * j / rope_dim)
    ang = np.arange(rows, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def _rngs(seed):
    kids = np.random.SeedSequence(seed).spawn(len(_STREAMS))
    return {name: np.random.default_rng(s) for name, s in zip(_STREAMS, kids)}


def _draw_values(rng, shape, values, chunk_rows=2048):
    """Draw float32 values row-chunk by row-chunk (first axis) and round to bf16."""
    out = np.empty(shape, dtype=np.uint16)
    n0 = shape[0]
    for s in range(0, n0, chunk_rows):
        sub = (min(chunk_rows, n0 - s),) + tuple(shape[1:])
        if values == "student_t3":
            v = rng.standard_t(3, size=sub).astype(np.float32)
        else:
            v = rng.standard_normal(sub, dtype=np.float32)
        out[s:s + sub[0]] = f32_to_bf16_bits(v)
    return out


def make(T: int, H: int = 64, *, rope_dim: int = 64, style: int = NEOX,
         values: str = "normal", table_rows: int = 4096, pos_mode: str = "uniform",
         pos_lo: int = 0, pos_hi: int | None = None, num_slots: int = 4096,
         slot_mode: str = "random_distinct", seed: int = 0, name: str = "custom",
         eps: float = 1e-6) -> Workload:
    """Build a workload.

    values: "normal" N(0,1); "student_t3"; "outlier_channels" (N(0,1), channels
      3 and 77 of every head and of k times 20); "sparse_outliers" (N(0,1) with
      each entry times 50 with probability 0.01); "zero_rows" (N(0,1) with
      round(0.001 * rows) Q rows and K rows set to zero).
    pos_mode: "uniform" ints in [pos_lo, pos_hi); "contiguous" pos_lo + t.
    slot_mode: "perm_prefix" first T of a permutation of the slots;
      "random_distinct"; "contiguous" (block at a random offset).
    """
    if pos_hi is None:
        pos_hi = table_rows
    r = _rngs(seed)
    base_values = "student_t3" if values == "student_t3" else "normal"
    q_bits = _draw_values(r["q"], (T, H, ROW), base_values)
    k_bits = _draw_values(r["k"], (T, ROW), base_values)
    w_bits = f32_to_bf16_bits(r["weights"].standard_normal((T, H), dtype=np.float32))
    if pos_mode == "contiguous":
        positions = pos_lo + np.arange(T, dtype=np.int64)
    else:
        positions = r["positions"].integers(pos_lo, pos_hi, size=T, dtype=np.int64)
    gamma = (1.0 + 0.1 * r["gamma"].standard_normal(ROW)).astype(np.float32)
    beta = (0.1 * r["beta"].standard_normal(ROW)).astype(np.float32)
    rs = r["slots"]
    if slot_mode == "perm_prefix":
        loc = rs.permutation(num_slots)[:T].astype(np.int64)
    elif slot_mode == "contiguous":
        off = int(rs.integers(0, num_slots - T + 1))
        loc = off + np.arange(T, dtype=np.int64)
    else:
        loc = rs.choice(num_slots, size=T, replace=False).astype(np.int64)

    info = {}
    sp = r["special"]
    if values == "outlier_channels":
        for ch in (3, 77):
            qf = bf16_bits_to_f32(q_bits[:, :, ch]) * np.float32(20.0)
            q_bits[:, :, ch] = f32_to_bf16_bits(qf)
            kf = bf16_bits_to_f32(k_bits[:, ch]) * np.float32(20.0)
            k_bits[:, ch] = f32_to_bf16_bits(kf)
    elif values == "sparse_outliers":
        for arr in (q_bits, k_bits):
            flat = arr.reshape(-1)
            mask = sp.random(flat.size) < 0.01
            idx = np.nonzero(mask)[0]
            flat[idx] = f32_to_bf16_bits(bf16_bits_to_f32(flat[idx]) * np.float32(50.0))
        info["outlier_scale"] = 50.0
    elif values == "zero_rows":
        nq = int(round(0.001 * T * H))
        nk = int(round(0.001 * T))
        zq = np.sort(sp.choice(T * H, size=nq, replace=False)) if nq else np.zeros(0, np.int64)
        zk = np.sort(sp.choice(T, size=nk, replace=False)) if nk else np.zeros(0, np.int64)
        q_bits.reshape(T * H, ROW)[zq] = 0
        k_bits[zk] = 0
        info["zero_q_rows"] = zq.astype(np.int64)
        info["zero_k_rows"] = zk.astype(np.int64)

    cos, sin = rope_table(table_rows, rope_dim)
    return Workload(name=name, T=T, H=H, rope_dim=rope_dim, style=style, q=q_bits, k=k_bits,
                    weights=w_bits, positions=positions, cos=cos, sin=sin, gamma=gamma,
                    beta=beta, eps=eps, num_slots=num_slots, out_cache_loc=loc, info=info)


# The five named workloads.  Index -> (name, keyword arguments of make()).
NAMED = [
    ("decode_tiny_T41", dict(T=41, values="outlier_channels", table_rows=4096,
                             num_slots=4096, slot_mode="perm_prefix")),
    ("decode_batch_T64", dict(T=64, values="sparse_outliers", table_rows=8192,
                              num_slots=65536, slot_mode="random_distinct")),
    ("decode_large_interleaved_T512", dict(T=512, style=INTERLEAVED, values="normal",
                                           table_rows=131072, num_slots=262144,
                                           slot_mode="random_distinct")),
    ("prefill_chunk_T8192", dict(T=8192, values="student_t3", table_rows=8192,
                                 pos_mode="contiguous", pos_lo=0, num_slots=262144,
                                 slot_mode="contiguous")),
    ("long_prefill_T65536", dict(T=65536, values="zero_rows", table_rows=262144,
                                 pos_mode="contiguous", pos_lo=196608, num_slots=262144,
                                 slot_mode="contiguous")),
]


def named(idx: int, T: int | None = None) -> Workload:
    """Named workload idx (seed 1000 + idx).  T overrides the token count for
    a smaller instance of the same recipe (positions and slots re-drawn)."""
    name, kw = NAMED[idx]
    kw = dict(kw)
    if T is not None:
        kw["T"] = T
        if kw.get("pos_mode") == "contiguous":
            kw["pos_lo"] = min(kw.get("pos_lo", 0), kw["table_rows"] - T)
    return make(seed=1000 + idx, name=name, **kw)


def bytes_per_token(H: int = 64, entry: str = "fused", rope_dim: int = 64,
                    q_scale_out: bool = False) -> int:
    """Algorithmic HBM bytes per token: each input read once, each output
    written once; the cos/sin row is counted once per token, not per head."""
    cos_sin = 2 * (rope_dim // 2) * 4
    # q bf16 + weights bf16 + position + cos/sin + q_fp8 + weights_out (fp32)
    q_side = H * ROW * 2 + H * 2 + 8 + cos_sin + H * ROW + H * 4
    if q_scale_out:
        q_side += H * 4
    # k bf16 + position + slot + fp8 row + fp32 scale
    k_side = ROW * 2 + 8 + 8 + ROW + 4
    if entry == "q":
        return q_side
    if entry == "k":
        return k_side + cos_sin
    return q_side + k_side - 8   # fused: the position is read once per token


def bytes_per_call_split(T: int, H: int = 64, entry: str = "fused", rope_dim: int = 64):
    """(read, written) algorithmic bytes of one call; they sum to
    bytes_per_call.  Reads: q, weights, position, cos/sin, k, slot, gamma and
    beta; writes: q_fp8, weights_out, the key's code row and scale."""
    writes_q = H * ROW + H * 4
    writes_k = ROW + 4
    writes = (0 if entry == "k" else writes_q) + (0 if entry == "q" else writes_k)
    total = bytes_per_call(T, H, entry, rope_dim)
    return total - T * writes, T * writes


def bytes_per_call(T: int, H: int = 64, entry: str = "fused", rope_dim: int = 64) -> int:
    """bytes_per_token * T, plus the LayerNorm gamma and beta (fp32 [128] each)
    once per call for the entries that run K rows."""
    per_call = 0 if entry == "q" else 2 * ROW * 4
    return T * bytes_per_token(H, entry, rope_dim) + per_call


# ---------------------------------------- key / head-gate projection ----

@dataclass
class ProjWorkload:
    """Inputs of the key / head-gate projection with the key preparation in
    its epilogue: hidden states and the projection weight, plus the key side
    (positions, slots, LayerNorm parameters, rope table) of `key`, a Workload
    whose q / k / weights are not used."""
    name: str
    T: int
    d: int
    H: int
    hidden: np.ndarray      # uint16 (bf16 bits) [T, d]
    weight: np.ndarray      # uint16 (bf16 bits) [128 + H, d]
    key: Workload


def proj_make(T: int, d: int = 7168, H: int = 64, *, seed: int = 0, name: str = "custom",
              **key_kw) -> ProjWorkload:
    """Hidden states N(0,1) and weight N(0, 1/d), both rounded to bf16, so each
    projected value is about N(0,1); the key side from make(T, H, ...) with
    key_kw (positions, slots, table, rope) and the same seed.  The pages give
    no hidden size; d = 7168 is the hidden width of the DeepSeek-V3 family whose
    sparse-attention indexer the pages run."""
    kids = np.random.SeedSequence(seed).spawn(2)
    rh, rw = (np.random.default_rng(s) for s in kids)
    hidden = _draw_values(rh, (T, d), "normal", chunk_rows=max(1, (1 << 24) // d))
    weight = f32_to_bf16_bits(rw.standard_normal((ROW + H, d), dtype=np.float32)
                              * np.float32(1.0 / np.sqrt(d)))
    key = make(min(T, 1) if T == 0 else T, H=1, seed=seed, name=name + "_key", **key_kw)
    return ProjWorkload(name=name, T=T, d=d, H=H, hidden=hidden, weight=weight, key=key)


def proj_bytes_per_call(T: int, d: int = 7168, H: int = 64, rope_dim: int = 64) -> int:
    """Algorithmic HBM bytes of one projection call: hidden [T, d] and weight
    [128 + H, d] bf16 read once, the key side's reads (position, slot, cos/sin
    row per token; gamma and beta once) and writes (code row and scale), and
    the gates written as bf16 [T, H]."""
    key_side = T * (8 + 8 + 2 * (rope_dim // 2) * 4 + ROW + 4) + 2 * ROW * 4
    return T * d * 2 + (ROW + H) * d * 2 + key_side + T * H * 2


def proj_flops_per_call(T: int, d: int = 7168, H: int = 64) -> int:
    """2 * T * d * (128 + H): one multiply and one add per term."""
    return 2 * T * d * (ROW + H)


# ------------------------------------------------ top-k per row inputs ----

@dataclass
class TopkWorkload:
    name: str
    logits: np.ndarray      # float32 [rows, cols]
    lengths: np.ndarray     # int32 [rows]: valid columns of each row
    k: int


def topk_make(rows: int, cols: int, k: int = 2048, *, lengths: str = "full", seed: int = 0,
              name: str = "custom") -> TopkWorkload:
    """Index logits for the top-k selection.  Values N(0,1) float32; every
    fourth row rounded to multiples of 1/8 (many ties); 1% of the entries
    -inf (masked keys).  lengths: "full" (every column), "ragged" (uniform in
    [cols/2, cols]) or "causal" (row r of the last `rows` queries of a
    `cols`-token context sees cols - rows + 1 + r keys)."""
    kids = np.random.SeedSequence(seed).spawn(3)
    rv, rm, rl = (np.random.default_rng(s) for s in kids)
    x = rv.standard_normal((rows, cols), dtype=np.float32)
    x[::4] = np.round(x[::4] * 8) / 8
    mask = rm.random((rows, cols)) < 0.01
    x[mask] = -np.inf
    if lengths == "full":
        lens = np.full(rows, cols, np.int32)
    elif lengths == "ragged":
        lens = rl.integers(cols // 2, cols + 1, rows).astype(np.int32)
    elif lengths == "causal":
        lens = (cols - rows + 1 + np.arange(rows)).astype(np.int32)
    else:
        raise ValueError(lengths)
    return TopkWorkload(name=name, logits=x, lengths=lens, k=k)


TOPK_NAMED = [
    ("topk_decode_batch64_ctx16384", dict(rows=64, cols=16384, lengths="ragged")),
    ("topk_decode_batch64_ctx131072", dict(rows=64, cols=131072, lengths="ragged")),
    ("topk_prefill_causal_T8192", dict(rows=8192, cols=8192, lengths="causal")),
]


def topk_named(idx: int) -> TopkWorkload:
    name, kw = TOPK_NAMED[idx]
    return topk_make(seed=2000 + idx, name=name, **kw)


def topk_bytes_per_call(rows: int, lengths, k: int = 2048) -> int:
    """Algorithmic bytes: every valid logit read once, the length of each row,
    and k indices written per row."""
    return int(np.sum(np.asarray(lengths, dtype=np.int64))) * 4 + rows * 4 + rows * k * 4


# -------------------------------------------------- index-logits inputs ----

@dataclass
class LogitsWorkload:
    name: str
    q_fp8: np.ndarray       # uint8 E4M3FN codes [T, H, 128]
    weights: np.ndarray     # float32 [T, H] (folded head gates)
    k_cache: np.ndarray     # uint8 [S, 128] index-K cache codes
    k_scale: np.ndarray     # float32 [S] (powers of two)
    key_slots: np.ndarray   # int32 [N]: cache slot of key s
    lengths: np.ndarray     # int32 [T]: keys valid for token t


def _random_codes(rng, shape) -> np.ndarray:
    """Uniform E4M3FN bytes with the two NaN codes replaced by zero."""
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0
    return c


def logits_make(T: int, N: int, H: int = 64, *, num_slots: int = 262144, lengths: str = "full",
                slots: str = "contiguous", seed: int = 0, name: str = "custom") -> LogitsWorkload:
    """Prepared queries and an index-K cache for the index logits.  Codes are
    uniform over the non-NaN E4M3FN bytes (every binade), key scales 2^-12..2^-3,
    gates N(0,1) * 2^-10..2^-5 (the range of folded ue8m0 gates).
    slots: "contiguous" (N slots from a random offset) or "random" (N distinct
    slots of the cache).  lengths: "full", "ragged" (uniform in [N/2, N]) or
    "causal" (token t of the last T of an N-key context sees N - T + 1 + t keys)."""
    kids = np.random.SeedSequence(seed).spawn(6)
    rq, rw, rk, rs, rl, rp = (np.random.default_rng(s) for s in kids)
    q8 = _random_codes(rq, (T, H, ROW))
    w = (rw.standard_normal((T, H), dtype=np.float32)
         * np.exp2(rw.integers(-10, -4, size=(T, H))).astype(np.float32))
    kc = _random_codes(rk, (num_slots, ROW))
    ks = np.exp2(rk.integers(-12, -2, size=num_slots)).astype(np.float32)
    if slots == "contiguous":
        off = int(rp.integers(0, num_slots - N + 1))
        ksl = np.arange(off, off + N, dtype=np.int32)
    elif slots == "random":
        ksl = rp.permutation(num_slots)[:N].astype(np.int32)
    else:
        raise ValueError(slots)
    if lengths == "full":
        lens = np.full(T, N, np.int32)
    elif lengths == "ragged":
        lens = rl.integers(N // 2, N + 1, T).astype(np.int32)
    elif lengths == "causal":
        lens = (N - T + 1 + np.arange(T)).astype(np.int32)
    else:
        raise ValueError(lengths)
    return LogitsWorkload(name=name, q_fp8=q8, weights=w, k_cache=kc, k_scale=ks, key_slots=ksl,
                          lengths=lens)


LOGITS_NAMED = [
    ("logits_decode_batch64_ctx16384", dict(T=64, N=16384, lengths="ragged", slots="random")),
    ("logits_prefill_causal_T8192", dict(T=8192, N=8192, lengths="causal")),
    ("logits_prefill_full_T8192", dict(T=8192, N=8192, lengths="full")),
]


def logits_named(idx: int) -> LogitsWorkload:
    name, kw = LOGITS_NAMED[idx]
    return logits_make(seed=3000 + idx, name=name, **kw)


def logits_flops_per_call(H: int, lengths) -> int:
    """Algorithmic operations: one 128-term dot (2 * 128 ops) per head and
    valid (token, key) pair; the gate and head sum are not counted."""
    return 2 * ROW * H * int(np.sum(np.asarray(lengths, dtype=np.int64)))


def logits_bytes_per_call(T: int, H: int, N: int, lengths) -> int:
    """Algorithmic bytes: q codes and gates read once, each key's 128 codes,
    scale and slot index read once, each valid logit written once."""
    return T * H * (ROW + 4) + N * (ROW + 4 + 4) + T * 4 + \
        int(np.sum(np.asarray(lengths, dtype=np.int64))) * 4
