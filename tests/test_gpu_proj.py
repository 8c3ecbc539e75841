"""GPU parity of dsaidx_proj_k_norm_rope_quant_store: the key / head-gate
projection on the matrix cores with the key preparation in its epilogue,
through the C ABI, against the oracles (oracle/proj.py, then the key oracle).

Acceptance.  The projection's fp32 sums differ from the exact sums by at most
the summation bound E = (d - 1) * 2^-24 * sum |products| (any order of fp32
additions), so each bf16 output must lie between bf16(x - E) and bf16(x + E)
for the exact sum x; at most 0.1 % of the outputs may differ from bf16(x).  The key cache
must then hold what the key preparation stores from the oracle's bf16 key:
every row whose projected key equals the oracle's byte for byte exactly (the
preparation arithmetic is bit-reproducible), and the few rows with a flipped
element within one code per element.  The epilogue is also checked against
the key entry point run on the kernel's own projected key: the same bytes.
"""
import json

import numpy as np
import pytest
import torch

import oracle
import rope_fp8_quant_amd as R
from gpu_util import ROW, SENTINEL, bf16_mode_of, dev, dev_bf16, ordinal, split_paged
from oracle import proj as P
from rope_fp8_quant_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def log(what, rep):
    print("\n[parity] %s %s" % (what, json.dumps(rep, sort_keys=True)), flush=True)


class ProjCase:
    def __init__(self, pw, k_flags=0, page_size=0, with_k_out=True, gate_pad=0):
        self.pw, self.k_flags, self.page_size = pw, k_flags, page_size
        kw = pw.key
        T, H = pw.T, pw.H
        self.hidden = dev_bf16(pw.hidden)
        self.weight = dev_bf16(pw.weight)
        gbuf = torch.full((T, H + gate_pad), -1, dtype=torch.int16, device="cuda")
        self.gates = gbuf.view(torch.bfloat16)[:, :H]
        self.k_out = (torch.full((T, ROW), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
                      if with_k_out else None)
        self.pos, self.loc = dev(kw.positions), dev(kw.out_cache_loc)
        self.gamma, self.beta = dev(kw.gamma), dev(kw.beta)
        self.cos, self.sin = dev(kw.cos), dev(kw.sin)
        if k_flags & R.DSAIDX_K_PAGED_CACHE:
            self.cache = torch.full((kw.num_slots * (ROW + 4),), SENTINEL, dtype=torch.uint8, device="cuda")
            self.k_scale = None
        else:
            self.cache = torch.full((kw.num_slots, ROW), SENTINEL, dtype=torch.uint8, device="cuda")
            self.k_scale = torch.full((kw.num_slots,), float("nan"), dtype=torch.float32, device="cuda")

    def ka(self, k=None, cache=None, k_scale=None):
        kw = self.pw.key
        return R.k_args(k, self.gamma, self.beta, kw.eps, self.pos, self.loc,
                        self.cache if cache is None else cache,
                        self.k_scale if k_scale is None else k_scale, flags=self.k_flags,
                        page_size=self.page_size, num_slots=kw.num_slots)

    def rope(self):
        kw = self.pw.key
        return R.rope_args(self.cos, self.sin, kw.rope_dim, kw.style)

    def run(self):
        R.dsaidx_proj_k_norm_rope_quant_store(R.proj_args(self.hidden, self.weight, self.gates, self.k_out),
                                              self.ka(), self.rope())
        torch.cuda.synchronize()

    def cache_host(self):
        kw = self.pw.key
        if self.k_flags & R.DSAIDX_K_PAGED_CACHE:
            return split_paged(self.cache.cpu().numpy(), self.page_size, kw.num_slots)
        return self.cache.cpu().numpy(), self.k_scale.cpu().numpy()


def bits16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def ordinal16(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns to their order on the number line (+0 and -0 equal)."""
    b = np.asarray(b, dtype=np.uint16)
    mag = (b & 0x7FFF).astype(np.int64)
    return np.where(b & 0x8000, -mag, mag)


def check_outputs(got_bits, exact, abs_sum, d, what, rep):
    """got_bits: bf16 bits of the kernel; exact: the float64 sums; abs_sum:
    sum |products|.  The kernel's fp32 sum v lies within E = (d - 1) * 2^-24 *
    abs_sum of the exact sum x (any order of fp32 additions), and its output is
    bf16(v); rounding is monotone, so the output must lie between bf16(x - E)
    and bf16(x + E).  Outputs other than bf16(x) ("flips": near a midpoint, or
    near zero where cancellation leaves few significant bits) are counted.
    Returns the mask of flipped elements."""
    want = P.round_to_bf16_bits(exact)
    flip = got_bits != want
    E = (d - 1) * 2.0 ** -24 * abs_sum
    lo = ordinal16(P.round_to_bf16_bits(exact - E))
    hi = ordinal16(P.round_to_bf16_bits(exact + E))
    g = ordinal16(got_bits)
    ok = (g >= lo) & (g <= hi)
    rep[what] = dict(elements=int(got_bits.size), flipped=int(np.count_nonzero(flip)),
                     outside_bound=int(np.count_nonzero(~ok)))
    if flip.any():
        steps = np.abs(g[flip] - ordinal16(want[flip]))
        rep[what]["max_bf16_steps"] = int(steps.max())
    assert ok.all(), rep[what]
    assert np.count_nonzero(flip) <= 0.001 * got_bits.size, rep[what]
    return flip


def oracle_key_cache(pw, k_bits, k_flags, page_size, rows=None):
    """The key oracle on the oracle's bf16 key (rows: the tokens to run)."""
    kw = pw.key
    pos, loc = kw.positions, kw.out_cache_loc
    if rows is not None:
        k_bits, pos, loc = k_bits[rows], pos[rows], loc[rows]
    mode = bf16_mode_of(k_flags)
    if k_flags & R.DSAIDX_K_PAGED_CACHE:
        buf = np.full(kw.num_slots * (ROW + 4), SENTINEL, np.uint8)
        oracle.k_side_paged(k_bits, kw.gamma, kw.beta, kw.eps, pos, loc, kw.cos, kw.sin, buf, page_size,
                            kw.num_slots, kw.rope_dim, kw.style, mode)
        return split_paged(buf, page_size, kw.num_slots)
    kc = np.full((kw.num_slots, ROW), SENTINEL, np.uint8)
    ks = np.full(kw.num_slots, np.nan, np.float32)
    oracle.k_side(k_bits, kw.gamma, kw.beta, kw.eps, pos, loc, kw.cos, kw.sin, kc, ks, kw.rope_dim,
                  kw.style, mode)
    return kc, ks


def check_case(c: ProjCase):
    pw = c.pw
    rep = dict(T=pw.T, d=pw.d, H=pw.H, rope_dim=pw.key.rope_dim, style=pw.key.style, flags=c.k_flags)
    exact, abs_sum = P.projection_values(pw.hidden, pw.weight)
    check_outputs(bits16(c.gates), exact[:, ROW:], abs_sum[:, ROW:], pw.d, "gates", rep)
    k_bits = P.round_to_bf16_bits(exact[:, :ROW])
    kflip = np.zeros(k_bits.shape, bool)
    if c.k_out is not None:
        kflip = check_outputs(bits16(c.k_out), exact[:, :ROW], abs_sum[:, :ROW], pw.d, "k_out", rep)
    # the key cache against the key oracle on the oracle's bf16 key
    got_kc, got_ks = c.cache_host()
    want_kc, want_ks = oracle_key_cache(pw, k_bits, c.k_flags, c.page_size)
    loc = pw.key.out_cache_loc
    exact_rows = ~kflip.any(axis=1)
    s_ok, s_flip = loc[exact_rows], loc[~exact_rows]
    assert np.array_equal(got_kc[s_ok], want_kc[s_ok]), "key rows with an exact projection"
    assert np.array_equal(got_ks[s_ok].view(np.uint32), want_ks[s_ok].view(np.uint32))
    if s_flip.size:
        dd = np.abs(ordinal(got_kc[s_flip]) - ordinal(want_kc[s_flip]))
        same_scale = got_ks[s_flip] == want_ks[s_flip]
        assert dd[same_scale].max(initial=0) <= 1
        rep["key_rows_with_a_flip"] = int(s_flip.size)
        rep["key_rows_scale_moved"] = int(np.count_nonzero(~same_scale))
        rep["key_codes_differ"] = int(np.count_nonzero(dd))
        assert np.count_nonzero(dd) <= 0.001 * got_kc[loc].size
    touched = np.zeros(pw.key.num_slots, bool)
    touched[loc] = True
    assert np.all(got_kc[~touched] == SENTINEL), "cache rows outside out_cache_loc changed"
    return rep


CASES = [
    # T, d, H, rope_dim, style, flags, page
    (1, 64, 64, 64, W.NEOX, 0, 0),
    (37, 128, 64, 64, W.NEOX, 0, 0),
    (300, 192, 8, 64, W.INTERLEAVED, 0, 0),
    (129, 7168, 64, 64, W.NEOX, 0, 0),
    (1000, 256, 33, 96, W.NEOX, R.DSAIDX_K_PAGED_CACHE, 16),
    (2053, 512, 64, 64, W.NEOX, R.DSAIDX_K_BF16_ROUND_ONCE, 0),
    (513, 320, 64, 24, W.INTERLEAVED, R.DSAIDX_K_BF16_INTERMEDIATE, 0),
    (260, 320, 16, 64, W.NEOX, 0, 0),
    (131, 448, 64, 64, W.NEOX, 0, 0),
    (700, 1024, 1, 128, W.NEOX, 0, 0),
]


@pytest.mark.parametrize("T,d,H,rope_dim,style,flags,page", CASES)
def test_projection_against_oracle(T, d, H, rope_dim, style, flags, page):
    print("\n[case] proj T=%d d=%d H=%d rope_dim=%d style=%d flags=%d" % (T, d, H, rope_dim, style, flags),
          flush=True)
    pw = W.proj_make(T, d, H, seed=T + d + H, name="proj", rope_dim=rope_dim, style=style,
                     table_rows=4096, num_slots=max(4096, T + 8), slot_mode="perm_prefix")
    c = ProjCase(pw, k_flags=flags, page_size=page, gate_pad=8 if H % 2 else 0)
    c.run()
    rep = check_case(c)
    log("proj", rep)


def test_epilogue_equals_key_entry_on_its_own_projection():
    """The cache the epilogue writes equals what dsaidx_k_norm_rope_quant_store
    writes from the kernel's projected key (k_out), byte for byte; without
    k_out the gates and cache are the same."""
    pw = W.proj_make(1500, 384, 64, seed=11, name="proj", table_rows=4096, num_slots=4096,
                     slot_mode="perm_prefix")
    c = ProjCase(pw)
    c.run()
    kc1, ks1 = c.cache_host()
    cache2 = torch.full_like(c.cache, SENTINEL)
    scale2 = torch.full_like(c.k_scale, float("nan"))
    R.dsaidx_k_norm_rope_quant_store(c.ka(k=c.k_out, cache=cache2, k_scale=scale2), c.rope())
    torch.cuda.synchronize()
    assert np.array_equal(kc1, cache2.cpu().numpy())
    assert np.array_equal(ks1.view(np.uint32), scale2.cpu().numpy().view(np.uint32))
    c2 = ProjCase(pw, with_k_out=False)
    c2.run()
    assert np.array_equal(bits16(c.gates), bits16(c2.gates))
    kc3, ks3 = c2.cache_host()
    assert np.array_equal(kc1, kc3) and np.array_equal(ks1.view(np.uint32), ks3.view(np.uint32))


@pytest.mark.parametrize("x_st,w_st", [(448, 520), (1 << 22, 1 << 22)])
def test_projection_strided_rows(x_st, w_st):
    """Hidden and weight rows at strides above d, up to the largest the host
    accepts (2^22 elements): the kernel's byte offsets within a workgroup's 256
    rows then reach 255 * 2^23, just under 2^31.  The results equal those of
    the contiguous call bit for bit (the same sums in the same order)."""
    T, d, H = 300, 256, 24
    pw = W.proj_make(T, d, H, seed=77, name="proj", table_rows=4096, num_slots=4096,
                     slot_mode="perm_prefix")
    ref = ProjCase(pw)
    ref.run()
    c = ProjCase(pw)
    xbig = torch.zeros(((T - 1) * x_st + d,), dtype=torch.bfloat16, device="cuda")
    wbig = torch.zeros(((ROW + H - 1) * w_st + d,), dtype=torch.bfloat16, device="cuda")
    c.hidden = xbig.as_strided((T, d), (x_st, 1))
    c.weight = wbig.as_strided((ROW + H, d), (w_st, 1))
    c.hidden.copy_(ref.hidden)
    c.weight.copy_(ref.weight)
    print("\n[case] proj strided rows x_st=%d w_st=%d (%.1f GB of rows)" %
          (x_st, w_st, (xbig.numel() + wbig.numel()) * 2 / 1e9), flush=True)
    c.run()
    assert np.array_equal(bits16(c.gates), bits16(ref.gates))
    assert np.array_equal(bits16(c.k_out), bits16(ref.k_out))
    kc, ks = c.cache_host()
    kc0, ks0 = ref.cache_host()
    assert np.array_equal(kc, kc0) and np.array_equal(ks.view(np.uint32), ks0.view(np.uint32))
    rep = check_case(c)
    del xbig, wbig, c
    torch.cuda.empty_cache()
    log("proj strided rows", rep)


def test_projection_full_size_sampled():
    """The bench launch: 65536 tokens, d = 7168, H = 64, positions
    196608..262143, a 262144-slot cache.  The oracle runs on 2048 sampled
    tokens and the first and last 64."""
    pw = W.proj_make(65536, 7168, 64, seed=4004, name="proj_long_prefill_T65536", table_rows=262144,
                     pos_mode="contiguous", pos_lo=196608, num_slots=262144, slot_mode="contiguous")
    c = ProjCase(pw)
    c.run()
    rng = np.random.default_rng(9)
    rows = np.unique(np.concatenate([np.arange(64), np.arange(65536 - 64, 65536),
                                     rng.choice(65536, 2048, replace=False)]))
    pws = W.ProjWorkload(name="sample", T=len(rows), d=pw.d, H=pw.H, hidden=pw.hidden[rows],
                         weight=pw.weight, key=pw.key)
    # the key side of the sample: its own positions and slots
    key = W.Workload(**{**pw.key.__dict__})
    key.positions = pw.key.positions[rows]
    key.out_cache_loc = pw.key.out_cache_loc[rows]
    key.T = len(rows)
    pws.key = key
    exact, abs_sum = P.projection_values(pws.hidden, pw.weight)
    rep = dict(T=65536, sampled=int(len(rows)))
    check_outputs(bits16(c.gates)[rows], exact[:, ROW:], abs_sum[:, ROW:], pw.d, "gates", rep)
    kflip = check_outputs(bits16(c.k_out)[rows], exact[:, :ROW], abs_sum[:, :ROW], pw.d, "k_out", rep)
    want_kc, want_ks = oracle_key_cache(pws, P.round_to_bf16_bits(exact[:, :ROW]), 0, 0)
    got_kc, got_ks = c.cache_host()
    loc = key.out_cache_loc
    ok = loc[~kflip.any(axis=1)]
    assert np.array_equal(got_kc[ok], want_kc[ok])
    assert np.array_equal(got_ks[ok].view(np.uint32), want_ks[ok].view(np.uint32))
    rep["key_rows_exact"] = int(ok.size)
    log("proj full size", rep)


def test_empty_and_invalid_projection_calls():
    pw = W.proj_make(4, 64, 64, seed=1, name="proj", table_rows=64, num_slots=16)
    c = ProjCase(pw)
    e = torch.empty
    pa = R.proj_args(e((0, 64), dtype=torch.bfloat16, device="cuda"), c.weight,
                     e((0, 64), dtype=torch.bfloat16, device="cuda"))
    ka = R.k_args(None, c.gamma, c.beta, 1e-6, e((0,), dtype=torch.int64, device="cuda"),
                  e((0,), dtype=torch.int64, device="cuda"), c.cache, c.k_scale)
    R.dsaidx_proj_k_norm_rope_quant_store(pa, ka, c.rope())
    torch.cuda.synchronize()
    assert bool((c.cache == SENTINEL).all())
    bad = R.proj_args(c.hidden, c.weight, c.gates)
    bad.hidden_dim = 96
    with pytest.raises(R.DsaidxError):
        R.dsaidx_proj_k_norm_rope_quant_store(bad, c.ka(), c.rope())
