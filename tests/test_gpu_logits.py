"""GPU parity of dsaidx_mqa_logits against the index-logits oracle.

Tolerance, from the arithmetic of the matrix unit.  Every product of two E4M3
values is exact, but v_mfma_f32_16x16x128_f8f6f4 does not add the 128
products of a dot in IEEE fp32: it aligns them to the largest one and keeps a
limited number of bits, so its error scales with the largest product of the
dot (test_matrix_unit_dot_error below measures this on 51200 dots of random
full-range codes and asserts the allowance: on MI355X the worst seen was
2^-10.65 of the largest product, with no sign bias, and dots whose codes share
a binade came out exact).  The gate multiply and the 64-term head sum are
ordinary fp32.  The test allows, per entry,

  |got - want| <= k_scale * sum_h |w[t, h]| * (2^-8 * max_d |q[t, h, d]| * max_d |k[s, d]|
                                               + 2^-16 * sum_d |q[t, h, d] k[s, d]|)

(2^-8 of an upper bound of the largest product, about 6 times the worst seen,
plus about 256 fp32 roundings of the absolute sum).  Entries past a row's
length must be left untouched."""
import json

import numpy as np
import pytest
import torch

import oracle
import rope_fp8_quant_amd as R
from gpu_util import DeviceCase, logits_bound
from oracle import logits as LG
from rope_fp8_quant_amd import workloads as W

pytestmark = pytest.mark.gpu
SENTINEL = float(np.float32(-12345.5))


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def random_cache(S, rng, row_pad=0):
    codes = rng.integers(0, 256, size=(S, 128 + row_pad)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x00                    # no NaN codes
    scale = np.exp2(rng.integers(-12, -2, size=S)).astype(np.float32)
    return codes, scale


def random_query(T, H, rng):
    q8 = rng.integers(0, 256, size=(T, H, 128)).astype(np.uint8)
    q8[(q8 & 0x7F) == 0x7F] = 0x00
    w = (rng.standard_normal((T, H)) * np.exp2(rng.integers(-10, -4, size=(T, H)))).astype(np.float32)
    return q8, w


def bound(q8, w, codes, scale, slots):
    return logits_bound(q8, w, codes, scale, slots)


def run(q8, w, codes, scale, key_slots=None, lengths=None, N=None, paged_page=0, stride_pad=0):
    T, H, _ = q8.shape
    S = codes.shape[0]
    if N is None:
        N = len(key_slots) if key_slots is not None else S
    dq = torch.from_numpy(q8).cuda()
    dw = torch.from_numpy(w).cuda()
    if paged_page:
        P = paged_page
        buf = np.zeros((S // P, P * 132), np.uint8)
        for s in range(S):
            pg, o = divmod(s, P)
            buf[pg, o * 128:(o + 1) * 128] = codes[s, :128]
            buf[pg, P * 128 + 4 * o:P * 128 + 4 * o + 4] = np.frombuffer(scale[s:s + 1].tobytes(), np.uint8)
        dk = torch.from_numpy(buf.reshape(-1)).cuda()
        dks = None
    else:
        dk = torch.from_numpy(codes).cuda()
        dks = torch.from_numpy(scale).cuda()
    out = torch.full((T, N + stride_pad), SENTINEL, dtype=torch.float32, device="cuda")[:, :N]
    ks = None if key_slots is None else torch.from_numpy(np.asarray(key_slots, np.int32)).cuda()
    ln = None if lengths is None else torch.from_numpy(np.asarray(lengths, np.int32)).cuda()
    args = R.logits_args(dq, dw, dk, out, k_scale=dks, key_slots=ks, lengths=ln,
                         flags=R.DSAIDX_K_PAGED_CACHE if paged_page else 0, page_size=paged_page,
                         num_slots=S if paged_page else None)
    R.dsaidx_mqa_logits(args)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check(got, q8, w, codes, scale, key_slots=None, lengths=None, N=None):
    S = codes.shape[0]
    slots = np.arange(S) if key_slots is None else np.asarray(key_slots, np.int64)
    if N is not None:
        slots = slots[:N]
    valid = (slots >= 0) & (slots < S)
    safe = np.where(valid, slots, 0)
    want = LG.mqa_logits(q8, w, codes, scale, key_slots=safe, lengths=lengths)
    want[:, ~valid] = np.where(np.isnan(want[:, ~valid]), np.nan, 0.0)   # a slot outside the cache scores 0
    tol = bound(q8, w, codes, scale, safe)
    tol[:, ~valid] = 1e-30
    inside = ~np.isnan(want)
    err = np.abs(got.astype(np.float64) - want)
    assert np.all(err[inside] <= tol[inside]), float(np.max(err[inside] / tol[inside]))
    assert np.all(got[~inside] == np.float32(SENTINEL)), "entries past a row's length were written"
    return float(np.max(err[inside] / tol[inside])) if inside.any() else 0.0


@pytest.mark.parametrize("T,H,S", [(64, 64, 4096), (41, 64, 1000), (9, 16, 300), (3, 1, 70),
                                   (17, 33, 129), (8, 63, 64), (5, 64, 1), (33, 8, 15), (64, 64, 257)])
def test_dense_keys(T, H, S):
    """One-token shape (grids of at most 512 workgroups)."""
    assert logits_grid(T, S) <= 512
    rng = np.random.default_rng(T * 1000 + H + S)
    q8, w = random_query(T, H, rng)
    codes, scale = random_cache(S, rng)
    got = run(q8, w, codes, scale)
    r = check(got, q8, w, codes, scale)
    print("\n[parity] logits T=%d H=%d N=%d max err / bound %.3g" % (T, H, S, r), flush=True)


def logits_grid(T, N):
    """Workgroups of a logits call (the host's chunking: about 3072 workgroups
    of 8 tokens, at least 256 keys each); above 512 the kernel runs two
    tokens per wavefront, at or below one."""
    blocks = -(-T // 8)
    want = max(1, min(-(-3072 // blocks), -(-N // 256)))
    chunk = -(-(-(-N // want)) // 128) * 128
    return blocks * -(-N // chunk)


@pytest.mark.parametrize("T,H,S,causal,slots", [(2045, 64, 600, False, False), (1603, 24, 900, True, False),
                                                (1037, 40, 1500, True, True)])
def test_two_tokens_per_wavefront_shape(T, H, S, causal, slots):
    """Calls large enough for the two-token shape, checked in full: a ragged
    token count, heads not a multiple of 16, causal lengths, a slot list with
    entries outside the cache."""
    assert logits_grid(T, S) > 512
    rng = np.random.default_rng(T + H)
    q8, w = random_query(T, H, rng)
    codes, scale = random_cache(S, rng)
    lengths = np.clip(np.arange(T) * S // T + 1, 0, S) if causal else None
    key_slots = None
    if slots:
        key_slots = rng.permutation(S).astype(np.int64)
        key_slots[[0, 7, S // 2, S - 1]] = [-1, S, -(1 << 31), (1 << 31) - 1]
    got = run(q8, w, codes, scale, lengths=lengths, stride_pad=3, key_slots=key_slots)
    r = check(got, q8, w, codes, scale, lengths=lengths, key_slots=key_slots)
    print("\n[parity] logits two-token shape T=%d H=%d N=%d max err / bound %.3g" % (T, H, S, r), flush=True)


def test_causal_lengths_and_ragged_edges():
    rng = np.random.default_rng(5)
    T, H, S = 100, 64, 777
    q8, w = random_query(T, H, rng)
    codes, scale = random_cache(S, rng)
    lengths = np.clip(np.arange(T) * 8 - 13, -3, None)            # negative, short, ragged, > N
    lengths[-1] = 5000
    got = run(q8, w, codes, scale, lengths=lengths, stride_pad=5)
    check(got, q8, w, codes, scale, lengths=lengths)


@pytest.mark.parametrize("T,H,S", [(61, 48, 9000), (64, 64, 16384)])
def test_one_token_shape_ragged_lengths_over_many_chunks(T, H, S):
    """One-token shape with many chunks (a workgroup's keys are every
    chunks-th 16-key block), checked in full: every token a different length
    (zero, negative, multiples of 16 and their neighbours, N, past N), a slot
    list with entries outside the cache, N not a multiple of 16 in the first
    case."""
    assert logits_grid(T, S) <= 512 and -(-S // 256) >= 32
    rng = np.random.default_rng(T * 7 + S)
    q8, w = random_query(T, H, rng)
    codes, scale = random_cache(S, rng)
    lengths = rng.integers(-5, S + 100, size=T)
    lengths[:10] = [0, -1, 1, 15, 16, 17, S - 1, S, 4096, 4097]
    slots = rng.permutation(S).astype(np.int64)
    slots[[2, 99, S // 3, S - 2]] = [-1, S, -(1 << 31), (1 << 31) - 1]
    got = run(q8, w, codes, scale, key_slots=slots, lengths=lengths, stride_pad=7)
    r = check(got, q8, w, codes, scale, key_slots=slots, lengths=lengths)
    print("\n[parity] logits one-token shape T=%d H=%d N=%d ragged max err / bound %.3g" % (T, H, S, r),
          flush=True)


def test_key_slots_and_slots_outside_the_cache():
    rng = np.random.default_rng(6)
    T, H, S = 24, 64, 500
    q8, w = random_query(T, H, rng)
    codes, scale = random_cache(S, rng, row_pad=16)
    slots = rng.permutation(S)[:333].astype(np.int64)
    slots[[3, 50, 200, 201, 332]] = [-1, S, 1 << 30, -(1 << 31), (1 << 31) - 1]   # score 0
    got = run(q8, w, codes, scale, key_slots=slots)
    check(got, q8, w, codes, scale, key_slots=slots)


@pytest.mark.parametrize("page", [2, 64])
def test_page_interleaved_cache(page):
    rng = np.random.default_rng(page)
    T, H, S = 19, 64, 256
    q8, w = random_query(T, H, rng)
    codes, scale = random_cache(S, rng)
    slots = rng.permutation(S)[:200]
    got = run(q8, w, codes, scale, key_slots=slots, paged_page=page)
    check(got, q8, w, codes, scale, key_slots=slots)


def test_single_binade_codes_are_exact_up_to_the_head_sum():
    """Codes of one binade (|values| in [1, 2)): the matrix unit's dots are
    exact, so only the fp32 gate multiply and the 64-term head sum round
    (at most about 70 roundings of 2^-24 of the absolute sum: 2^-17 allowed)."""
    rng = np.random.default_rng(21)
    T, H, S = 32, 64, 512
    q8 = (rng.integers(0, 8, size=(T, H, 128)) | 0x38 | (rng.integers(0, 2, size=(T, H, 128)) << 7)).astype(np.uint8)
    codes = (rng.integers(0, 8, size=(S, 128)) | 0x38 | (rng.integers(0, 2, size=(S, 128)) << 7)).astype(np.uint8)
    scale = np.exp2(rng.integers(-12, -2, size=S)).astype(np.float32)
    w = rng.standard_normal((T, H)).astype(np.float32)
    got = run(q8, w, codes, scale).astype(np.float64)
    want = LG.mqa_logits(q8, w, codes, scale)
    dots = LG.head_dots(q8, codes)
    tol = np.einsum("th,ths->ts", np.abs(w.astype(np.float64)), np.maximum(dots, 0.0))
    tol = tol * scale.astype(np.float64)[None, :] * 2.0 ** -17 + 1e-30
    assert np.all(np.abs(got - want) <= tol), float(np.max(np.abs(got - want) / tol))


def test_extreme_codes():
    """Largest codes (+-448) everywhere: the biggest dots (128 * 448^2) and
    all-negative dots that the ReLU zeroes."""
    T, H, S = 8, 64, 80
    q8 = np.full((T, H, 128), 0x7E, np.uint8)
    q8[:, ::2, :] = 0xFE
    codes = np.full((S, 128), 0x7E, np.uint8)
    codes[::3] = 0x01                                             # smallest subnormal
    scale = np.full(S, 2.0 ** -8, np.float32)
    w = np.ones((T, H), np.float32)
    got = run(q8, w, codes, scale)
    check(got, q8, w, codes, scale)


def test_pipeline_from_the_prep_call():
    """Fused prep call on the device, then logits from its q_fp8, weights_out
    and the index-K cache it wrote, against the oracle applied to the oracle's
    own prep outputs (equal where the prep outputs agree; compared within the
    bound on the device's own prep outputs otherwise)."""
    wl = W.make(40, 64, table_rows=4096, num_slots=512, slot_mode="perm_prefix", seed=77)
    c = DeviceCase(wl)
    c.run("fused")
    q8 = c.q_fp8.cpu().numpy()
    w = c.w_out.cpu().numpy()
    codes = c.cache_full.cpu().numpy()
    scale = c.k_scale.cpu().numpy()
    scale = np.where(np.isnan(scale), np.float32(0), scale)
    codes[np.isnan(c.k_scale.cpu().numpy())] = 0                  # slots no token wrote
    dk = torch.from_numpy(codes).cuda()
    dks = torch.from_numpy(scale).cuda()
    slots = np.asarray(wl.out_cache_loc, np.int64)
    out = torch.full((40, len(slots)), SENTINEL, dtype=torch.float32, device="cuda")
    args = R.logits_args(c.q_fp8, c.w_out, dk, out, k_scale=dks,
                         key_slots=torch.from_numpy(slots.astype(np.int32)).cuda())
    R.dsaidx_mqa_logits(args)
    torch.cuda.synchronize()
    check(out.cpu().numpy(), q8, w, codes, scale, key_slots=slots)
    # and through the oracle's own prep
    oq8, ow, _ = oracle.q_side(wl.q, wl.weights, wl.positions, wl.cos, wl.sin)
    assert np.array_equal(ow, w)
    print("\n[parity] pipeline: prep codes identical on %.4f of query elements"
          % float(np.mean(oq8 == q8)), flush=True)


def test_empty_calls_and_graph_capture():
    rng = np.random.default_rng(9)
    q8, w = random_query(16, 64, rng)
    codes, scale = random_cache(256, rng)
    dq, dw = torch.from_numpy(q8).cuda(), torch.from_numpy(w).cuda()
    dk, dks = torch.from_numpy(codes).cuda(), torch.from_numpy(scale).cuda()
    out = torch.full((16, 256), SENTINEL, dtype=torch.float32, device="cuda")
    R.dsaidx_mqa_logits(R.logits_args(dq[:0], dw[:0], dk, out[:0], k_scale=dks))
    R.dsaidx_mqa_logits(R.logits_args(dq, dw, dk, out[:, :0], k_scale=dks))
    torch.cuda.synchronize()
    assert np.all(out.cpu().numpy() == np.float32(SENTINEL))
    g = torch.cuda.CUDAGraph()
    args = R.logits_args(dq, dw, dk, out, k_scale=dks)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        R.dsaidx_mqa_logits(args)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        R.dsaidx_mqa_logits(args)
    for rep in range(3):
        q8b, wb = random_query(16, 64, np.random.default_rng(100 + rep))
        dq.copy_(torch.from_numpy(q8b))
        dw.copy_(torch.from_numpy(wb))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check(out.cpu().numpy(), q8b, wb, codes, scale)


def test_invalid_arguments():
    rng = np.random.default_rng(10)
    q8, w = random_query(4, 64, rng)
    codes, scale = random_cache(64, rng)
    dq, dw = torch.from_numpy(q8).cuda(), torch.from_numpy(w).cuda()
    dk, dks = torch.from_numpy(codes).cuda(), torch.from_numpy(scale).cuda()
    out = torch.zeros((4, 64), dtype=torch.float32, device="cuda")
    a = R.logits_args(dq, dw, dk, out, k_scale=dks)
    a.num_heads = 65
    with pytest.raises(R.DsaidxError):
        R.dsaidx_mqa_logits(a)
    a = R.logits_args(dq, dw, dk, out, k_scale=dks)
    a.num_keys = 65                                                 # more keys than slots
    a.logits_stride = 65
    with pytest.raises(R.DsaidxError):
        R.dsaidx_mqa_logits(a)


@pytest.mark.parametrize("idx", range(len(W.LOGITS_NAMED)))
def test_named_workloads_sampled_rows(idx):
    """The benchmark's workloads at full size, in the launch the benchmark
    times: every row's untouched tail checked, and sampled rows (first, last
    and random ones) against the oracle entry by entry within the bound."""
    lw = W.logits_named(idx)
    T, H = lw.q_fp8.shape[:2]
    N = len(lw.key_slots)
    print("\n[case] logits %s T=%d H=%d N=%d" % (lw.name, T, H, N), flush=True)
    dq, dw = torch.from_numpy(lw.q_fp8).cuda(), torch.from_numpy(lw.weights).cuda()
    dk, dks = torch.from_numpy(lw.k_cache).cuda(), torch.from_numpy(lw.k_scale).cuda()
    out = torch.full((T, N), SENTINEL, dtype=torch.float32, device="cuda")
    args = R.logits_args(dq, dw, dk, out, k_scale=dks,
                         key_slots=torch.from_numpy(lw.key_slots).cuda(),
                         lengths=torch.from_numpy(lw.lengths).cuda())
    R.dsaidx_mqa_logits(args)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    past = np.arange(N)[None, :] >= lw.lengths[:, None]
    assert np.all(got[past] == np.float32(SENTINEL)), "entries past a row's length were written"
    assert not np.any(got[~past] == np.float32(SENTINEL))
    rng = np.random.default_rng(idx)
    rows = sorted(set([0, T - 1] + [int(x) for x in rng.integers(0, T, 6)]))
    slots = lw.key_slots.astype(np.int64)
    worst = 0.0
    for r in rows:
        want = LG.mqa_logits(lw.q_fp8[r:r + 1], lw.weights[r:r + 1], lw.k_cache, lw.k_scale,
                             key_slots=slots, lengths=lw.lengths[r:r + 1])[0]
        tol = bound(lw.q_fp8[r:r + 1], lw.weights[r:r + 1], lw.k_cache, lw.k_scale, slots)[0]
        n = int(lw.lengths[r])
        err = np.abs(got[r, :n].astype(np.float64) - want[:n])
        assert np.all(err <= tol[:n]), (r, float(np.max(err / tol[:n])))
        worst = max(worst, float(np.max(err / tol[:n])) if n else 0.0)
    print("[parity] %s rows %s: max err / bound %.3g" % (lw.name, rows, worst), flush=True)


def test_matrix_unit_dot_error():
    """The evidence behind the tolerance above: the device's 128-term fp8 dots
    through dsaidx_mqa_logits itself.  One head, gate 1 and key scale 1 make
    each logit relu(dot); the same keys with every sign bit flipped give
    relu(-dot), so the difference is the signed dot as the kernel computes it.
    Over 51200 dots of random full-range codes (400 tokens x 128 keys), the
    error against the exact dot (float64 over the decoded codes: each product
    has at most 8 significant bits, so 128 of them sum exactly) is reported as
    a fraction of the dot's largest |product|, and must stay within the 2^-8
    the tolerance allows (of a bound on that product).  Codes that share one
    binade must give exact dots."""
    rng = np.random.default_rng(6061)
    T, N = 400, 128
    q8, _ = random_query(T, 1, rng)
    codes, _ = random_cache(N, rng)
    w = np.ones((T, 1), np.float32)
    scale = np.ones(N, np.float32)
    pos = run(q8, w, codes, scale)
    neg = run(q8, w, codes ^ np.uint8(0x80), scale)
    got = pos.astype(np.float64) - neg.astype(np.float64)
    dec = LG.decode_table()
    qv = dec[q8[:, 0, :]]                       # [T, 128]
    kv = dec[codes[:, :128]]                    # [N, 128]
    exact = qv @ kv.T
    largest = np.abs(qv)[:, None, :] * np.abs(kv)[None, :, :]
    largest = largest.max(axis=2)
    err = np.abs(got - exact)
    nz = largest > 0
    ratio = np.zeros_like(err)
    ratio[nz] = err[nz] / largest[nz]
    worst = float(ratio.max())
    bias = float(np.mean(np.sign(got - exact)[err > 0])) if np.any(err > 0) else 0.0
    # one binade: codes with the same exponent field (here 0x40..0x47 and signs)
    q1 = (0x40 | rng.integers(0, 8, size=(T, 1, 128)) | (rng.integers(0, 2, size=(T, 1, 128)) << 7)).astype(np.uint8)
    k1 = (0x40 | rng.integers(0, 8, size=(N, 128)) | (rng.integers(0, 2, size=(N, 128)) << 7)).astype(np.uint8)
    g1 = run(q1, w, k1, scale).astype(np.float64) - run(q1, w, k1 ^ np.uint8(0x80), scale).astype(np.float64)
    e1 = dec[q1[:, 0, :]] @ dec[k1].T
    rep = dict(dots=int(err.size), worst_err_over_largest_product=worst,
               log2_worst=float(np.log2(worst)) if worst > 0 else None,
               dots_with_error=int(np.count_nonzero(err)), sign_bias=bias,
               one_binade_max_abs_err=float(np.max(np.abs(g1 - e1))))
    print("\n[parity] mfma fp8 dot error %s" % json.dumps(rep), flush=True)
    assert worst <= 2.0 ** -8, rep
    assert np.array_equal(g1, e1), rep
