// gfx950 kernels for the DSA-indexer Q/K preparation.
//
// Operation ([sglang-fuse] = sglang PR "[AMD] [GLM5] Fuse the DSA indexer Q/K
// rope + quant + K-cache write", sections Motivation and Modifications;
// [vllm-47335] = vLLM PR 47335 "Enable fused indexer-Q RoPE+quant kernel",
// section Summary):
//   query vector (t,h): RoPE -> E4M3FN codes with a power-of-two scale ->
//     scale folded into the head gate;
//   key row t: fp32 LayerNorm -> RoPE -> the same codes -> fp8 row and scale
//     stored at cache slot out_cache_loc[t].
//
// Mapping.  Each 128-wide vector is owned by one 16-lane DPP row of a
// wavefront, eight elements per lane, so one wavefront instruction covers four
// whole vectors.  Two lane layouts:
//   split  lane j holds elements [4j, 4j+4) and [64+4j, 64+4j+4).  Every lane
//          then owns rope elements when rope_dim = 64, so the rotation costs
//          half as many instructions per lane; a NeoX pair (i, i + R/2) sits in
//          lanes j and j + R/8.  Used for NeoX with rope_dim <= 64 and for the
//          interleaved style (pairs never leave a lane).
//   contig lane j holds [8j, 8j+8); used for NeoX with rope_dim 80..128.
//   generic the contig placement with an element-wise rotation, for every other
//          rope_dim (any even value up to 128) and for tables whose rows are
//          not 16-byte aligned: each lane reads the cos/sin entries of its own
//          rope elements, and the partner values come through a small LDS row
//          buffer per wavefront.  Not tuned: the workloads use the two above.
// Row reductions (max |y|, LayerNorm sums) are four DPP row_ror steps; the
// NeoX partner values come from ds_bpermute.  A query work item is one token
// and HPI heads (HPI / 4 passes of 4 vectors): the token's cos/sin sit in
// registers for all of them, and the item's HPI folded head gates are produced
// by one coalesced load and store.  HPI is 16, or 4 for calls of at most 16384
// query rows: a small batch cannot fill the GPU, and more, shorter items cut
// its latency (64 tokens x 64 heads: 2.6 us against 3.0 us per call), while
// for large batches 16-head items move fewer cos/sin rows and gates per byte
// of q.  Large batches of exactly 8 heads (a TP8 rank's share of 64) take
// items of two tokens x 8 heads (query_pair_item).  A key work item is 4
// tokens.  Key and query work items share one dispatch: the last k_blocks
// workgroups take key items (the first ones in small calls of 32 tokens or
// more: the placement template parameter, which also spreads them through
// the grid in 8-head calls of several rounds).
//
// Arithmetic matches the definition row for row: every fp32 product and sum
// is rounded on its own (contraction is off), the LayerNorm sums are fp64 (the
// variance sum by fused multiply-adds, whose fp32-by-fp32 products are exact), and
// the codes come from the gfx950 scaled packed convert, which rounds x / 2^e
// to nearest-even E4M3FN -- the same as multiplying by 2^-e (exact) and
// converting.  No value can exceed 448, as 2^e is chosen from the row max.
#include "dsaidx_prep_device.h"

#pragma clang fp contract(off)

namespace dsaidx {
namespace {

// ---------------------------------------------------------- work items ----

template <int STYLE, int LAYOUT, int HPI>
__device__ __forceinline__ void query_item(const PrepParams& p, int64_t item, int lane) {
    constexpr int kPasses = HPI / kRowsPerWave;
    const int g = lane >> 4;
    const int j = lane & (kLanesPerRow - 1);
    const int64_t t = item / p.head_blocks;
    const int hb = (int)(item - t * p.head_blocks);
    // Head of this row group in pass ps: h0 + 4 * ps.
    const int hbase = hb * HPI;
    const int h0 = hbase + g;
    uint8_t* dst = p.q_fp8 + (t * p.H + h0) * kRow;

    // Every load of the item before any arithmetic: the rows, the HPI head
    // gates (lane l of the first row group takes head hbase + l), the
    // position and the cos/sin row it selects.  Loads return in issue order.
    // A multi-pass item fetches the position and cos/sin first, so pass 0 can
    // start while the later rows are still arriving, and its gates last: a
    // conditional gate load ahead of the rows held them back until it
    // returned (11 % on a 512-token call).  A one-pass item has
    // nothing to overlap: it issues its row and gate first, unconditionally
    // (heads past H clamped to H - 1: computed, never stored), so they travel
    // while the position and then the cos/sin row come back -- two dependent
    // round trips instead of three (3-10 % faster on batches of 41-256; the
    // same order on multi-pass items measured 1-9 % slower on large batches).
    // The multi-pass rows and gate keep their per-lane conditions, though the
    // compiler waits for each such load inside its branch: issuing them all
    // unconditionally (heads clamped) made the 64-head, 65536-token call 6 %
    // slower (279 against 262 us).
    const uint16_t* qt = p.q + t * p.q_st;
    const bool gate_lane = lane < HPI && hbase + lane < p.H;
    uint4 raw[kPasses];
    uint32_t wbits = 0;
    int64_t pos;
    RopeLane rl;
    if (kPasses == 1) {
        raw[0] = load_row<LAYOUT>(qt + (int64_t)min(h0, p.H - 1) * p.q_sh, j);
        wbits = p.w[t * p.w_st + min(hbase + (lane < HPI ? lane : 0), p.H - 1)];
        pos = clamp_position(p.q_pos[t], p.P);
        rl = rope_lane<STYLE, LAYOUT, true>(p, pos, lane);
    } else {
        pos = clamp_position(p.q_pos[t], p.P);
        rl = rope_lane<STYLE, LAYOUT>(p, pos, lane);
        const uint16_t* src = qt + (int64_t)h0 * p.q_sh;
        const int64_t src_pass = (int64_t)kRowsPerWave * p.q_sh;
#pragma unroll
        for (int ps = 0; ps < kPasses; ++ps) {
            raw[ps] = make_uint4(0, 0, 0, 0);
            if (h0 + ps * kRowsPerWave < p.H) raw[ps] = load_row<LAYOUT>(src + ps * src_pass, j);
        }
        if (gate_lane) wbits = p.w[t * p.w_st + hbase + lane];
    }

    int e[kPasses];
#pragma unroll
    for (int ps = 0; ps < kPasses; ++ps) {
        float y[8];
        rope_packed_row<STYLE, LAYOUT>(raw[ps], y, rl);
        e[ps] = scale_exponent(row_max_bits(lane_amax_bits(y)));
        const uint2 codes = encode8(y, exp2_int(e[ps]));
        if (h0 + ps * kRowsPerWave < p.H) store_row<LAYOUT>(dst + ps * (kRowsPerWave * kRow), j, codes);
    }

    // Head gate of head hbase + l on lane l: its exponent was computed in pass
    // l / 4 by row group l % 4.
    const int src_addr = ((lane & 3) << 4) << 2;
    int el = 0;
#pragma unroll
    for (int ps = 0; ps < kPasses; ++ps) {
        const int v = __builtin_amdgcn_ds_bpermute(src_addr, e[ps]);
        if ((lane >> 2) == ps) el = v;
    }
    if (gate_lane) {
        const int64_t row = t * p.H + hbase + lane;
        const float sc = exp2_int(el);
        const float ws = __uint_as_float(wbits << 16) * p.weight_scale;
        p.w_out[row] = ws * sc;
        if (p.q_scale) p.q_scale[row] = sc;
    }
}

// Query work item of two tokens x 8 heads, for calls of exactly 8 heads (a
// TP8 rank's share of 64): 16 rows in 4 passes, passes 0-1 on token t0 and
// 2-3 on token t0 + 1, so that an item moves as many bytes as a 16-head item
// (8-head items of one token left the call 4 % slower; 16-head items of one
// token left half of each wavefront idle).  Each token has its own position
// and cos/sin row; row l of the item (token t0 + l / 8, head l % 8) has its
// gate on lane l, its exponent from pass l / 4, row group l % 4.  A lone last
// token computes its partner's rows from its own (never stored).
template <int STYLE, int LAYOUT>
__device__ __forceinline__ void query_pair_item(const PrepParams& p, int64_t item, int lane) {
    constexpr int kPasses = 4;
    const int g = lane >> 4;
    const int j = lane & (kLanesPerRow - 1);
    const int64_t t0 = item * 2;
    const bool two = t0 + 1 < p.T;
    const int64_t t1 = two ? t0 + 1 : t0;
    auto tok = [&](int ps) -> int64_t { return ps < 2 ? t0 : t1; };
    auto head = [&](int ps) -> int { return 4 * (ps & 1) + g; };

    // The rows and gates first (they depend on nothing), then the positions
    // and the cos/sin rows they select: two dependent round trips.  Every lane
    // reads a gate (lanes 16 and up read token t1's, unused), so no load sits
    // under a per-lane branch.
    uint4 raw[kPasses];
#pragma unroll
    for (int ps = 0; ps < kPasses; ++ps)
        raw[ps] = load_row<LAYOUT>(p.q + tok(ps) * p.q_st + (int64_t)head(ps) * p.q_sh, j);
    const int64_t gt = lane < 8 ? t0 : t1;
    const uint32_t wbits = p.w[gt * p.w_st + (lane & 7)];
    const int64_t pos0 = clamp_position(p.q_pos[t0], p.P);
    const int64_t pos1 = clamp_position(p.q_pos[t1], p.P);
    const RopeLane rl0 = rope_lane<STYLE, LAYOUT>(p, pos0, lane);
    const RopeLane rl1 = rope_lane<STYLE, LAYOUT>(p, pos1, lane);

    int e[kPasses];
#pragma unroll
    for (int ps = 0; ps < kPasses; ++ps) {
        float y[8];
        rope_packed_row<STYLE, LAYOUT>(raw[ps], y, ps < 2 ? rl0 : rl1);
        e[ps] = scale_exponent(row_max_bits(lane_amax_bits(y)));
        const uint2 codes = encode8(y, exp2_int(e[ps]));
        if (ps < 2 || two) store_row<LAYOUT>(p.q_fp8 + (tok(ps) * p.H + head(ps)) * kRow, j, codes);
    }

    const int src_addr = ((lane & 3) << 4) << 2;
    int el = 0;
#pragma unroll
    for (int ps = 0; ps < kPasses; ++ps) {
        const int v = __builtin_amdgcn_ds_bpermute(src_addr, e[ps]);
        if ((lane >> 2) == ps) el = v;
    }
    if (lane < 8 || (lane < 16 && two)) {
        const int64_t row = gt * p.H + (lane & 7);
        const float sc = exp2_int(el);
        const float ws = __uint_as_float(wbits << 16) * p.weight_scale;
        p.w_out[row] = ws * sc;
        if (p.q_scale) p.q_scale[row] = sc;
    }
}

// Key work item: four consecutive tokens, one per DPP row of the wavefront.
template <int STYLE, int LAYOUT>
__device__ __forceinline__ void key_item(const PrepParams& p, int64_t item, int lane) {
    const int g = lane >> 4;
    const int j = lane & (kLanesPerRow - 1);
    const int64_t t = item * kTokensPerKItem + g;
    const bool valid = t < p.T;
    // a row group past T reads token T - 1 (computed, never stored): no load
    // under a per-lane branch.  The position first (the cos/sin row waits for
    // it, and loads retire in issue order), then the row and slot.
    const int64_t tc = valid ? t : p.T - 1;
    const int64_t pos = clamp_position(p.k_pos[tc], p.P);
    const uint4 raw = load_row<LAYOUT>(p.k + tc * p.k_st, j);
    const int64_t slot = p.loc[tc];
    key_row<STYLE, LAYOUT>(p, valid, raw, pos, slot, lane);
}

static_assert(256 / 64 <= kXchgWaves, "rope_generic's exchange buffer covers every wavefront");

// The 8-head instantiation is held to six wavefronts per SIMD (80 VGPRs, no
// spill): 43.0 against 43.7 us at five (92 VGPRs) for 65536 tokens; seven
// spill (51 us).
// Placement of the key workgroups in the grid (template parameter PLACE).
constexpr int kKeysLast = 0;
constexpr int kKeysFirst = 1;
constexpr int kKeysSpread = 2;

template <int STYLE, int LAYOUT, int HPI, int PLACE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(HPI == kHeadsPerItemMid ? 6 : 1)))
void indexer_qk_prep_kernel(PrepParams p) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int waves = (int)(blockDim.x >> 6);
    const int64_t nblocks = gridDim.x;
    const int64_t b = blockIdx.x;
    const int64_t nq = nblocks - p.k_blocks;
    // Where the key workgroups sit.  Calls of several rounds at 8 heads
    // (kKeysSpread) spread them evenly through the grid, one in every
    // k_period workgroups, so that their VALU-bound rows (LayerNorm, RoPE,
    // quantisation: a sixth of the bytes there) overlap the query rows'
    // memory stream.  Otherwise they come last (their work overlaps the query
    // stream's tail), or first (kKeysFirst) in small calls of 32 tokens or
    // more, where the key rows' longer chain of dependent steps is the
    // critical path (64 tokens: 2.46 against 2.57 us per call; with fewer
    // tokens the query rows are).  A template parameter, not a branch: the
    // branch and its parameters alone cost the small calls 0.1 us.
    bool is_key;
    int64_t kb, qb;
    if constexpr (PLACE == kKeysSpread) {
        // workgroup b = j * k_period + i: for j < k_blocks the last of each
        // period (i = k_period - 1) is key workgroup j and the rest query
        // workgroups; past k_blocks periods, query workgroups only.  The grid
        // is below 2^25 workgroups, within the magic division's range.
        const uint32_t bb = (uint32_t)b, per = (uint32_t)p.k_period;
        const uint32_t j = (uint32_t)(((uint64_t)bb * p.k_magic) >> p.k_shift);
        const uint32_t i = bb - j * per;
        if (j < (uint32_t)p.k_blocks) {
            is_key = i == per - 1;
            kb = j;
            qb = (int64_t)j * (per - 1) + i;
        } else {
            is_key = false;
            kb = 0;
            qb = (int64_t)p.k_blocks * (per - 1) + (bb - (uint32_t)p.k_blocks * per);
        }
    } else {
        constexpr bool kFirst = PLACE == kKeysFirst;
        is_key = kFirst ? b < p.k_blocks : b >= nq;
        kb = kFirst ? b : b - nq;
        qb = kFirst ? b - p.k_blocks : b;
    }
    if (is_key) {
        const int64_t stride = (int64_t)p.k_blocks * waves;
        for (int64_t it = kb * waves + wave; it < p.k_items; it += stride)
            key_item<STYLE, LAYOUT>(p, it, lane);
    } else {
        const int64_t stride = nq * waves;
        for (int64_t it = qb * waves + wave; it < p.q_items; it += stride) {
            if constexpr (HPI == kHeadsPerItemMid)
                query_pair_item<STYLE, LAYOUT>(p, it, lane);
            else
                query_item<STYLE, LAYOUT, HPI>(p, it, lane);
        }
    }
}

// Eight consecutive values per lane through the kernels' encoder, with a
// power-of-two scale as a row's ue8m0 scale is passed.
__global__ __launch_bounds__(256) void fp8_encode_selftest_kernel(const float* in, uint8_t* out,
                                                                  int64_t n, float scale) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x * 8;
    for (int64_t base = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8; base < n;
         base += stride) {
        float v[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) v[m] = base + m < n ? in[base + m] : 0.0f;
        const uint2 c = encode8(v, scale);
        if (base + 8 <= n) {
            *reinterpret_cast<uint2*>(out + base) = c;
        } else {
            for (int m = 0; base + m < n; ++m)
                out[base + m] = (uint8_t)(((m < 4 ? c.x : c.y) >> (8 * (m & 3))) & 0xFFu);
        }
    }
}

}  // namespace

hipError_t launch_fp8_selftest(const float* in, uint8_t* out, int64_t n, float scale,
                               unsigned grid, hipStream_t stream) {
    void* args[] = {&in, &out, &n, &scale};
    return hipLaunchKernel(reinterpret_cast<const void*>(&fp8_encode_selftest_kernel), dim3(grid),
                           dim3(256), args, 0, stream);
}

hipError_t launch_prep(const PrepParams& p, int style, unsigned grid, unsigned block,
                       hipStream_t stream) {
    PrepParams copy = p;
    void* args[] = {&copy};
    const int hpi = p.heads_per_item;
    const bool kf = p.k_first != 0 && hpi == kHeadsPerItemSmall;
    const bool spread = p.k_period > 0 && hpi == kHeadsPerItemMid;
    auto pick = [hpi, kf, spread](auto k4f, auto k4, auto k8s, auto k8, auto k16) -> const void* {
        return hpi == kHeadsPerItemSmall ? (kf ? reinterpret_cast<const void*>(k4f)
                                               : reinterpret_cast<const void*>(k4))
               : hpi == kHeadsPerItemMid ? (spread ? reinterpret_cast<const void*>(k8s)
                                                   : reinterpret_cast<const void*>(k8))
                                         : reinterpret_cast<const void*>(k16);
    };
    const void* fn;
    if (p.generic)
        fn = style == 1 ? (hpi == kHeadsPerItemSmall
                               ? reinterpret_cast<const void*>(
                                     &indexer_qk_prep_kernel<1, kGeneric, kHeadsPerItemSmall, kKeysLast>)
                               : reinterpret_cast<const void*>(
                                     &indexer_qk_prep_kernel<1, kGeneric, kHeadsPerItem, kKeysLast>))
                        : (hpi == kHeadsPerItemSmall
                               ? reinterpret_cast<const void*>(
                                     &indexer_qk_prep_kernel<0, kGeneric, kHeadsPerItemSmall, kKeysLast>)
                               : reinterpret_cast<const void*>(
                                     &indexer_qk_prep_kernel<0, kGeneric, kHeadsPerItem, kKeysLast>));
    else if (style == 1)
        fn = pick(&indexer_qk_prep_kernel<1, kSplit, kHeadsPerItemSmall, kKeysFirst>,
                  &indexer_qk_prep_kernel<1, kSplit, kHeadsPerItemSmall, kKeysLast>,
                  &indexer_qk_prep_kernel<1, kSplit, kHeadsPerItemMid, kKeysSpread>,
                  &indexer_qk_prep_kernel<1, kSplit, kHeadsPerItemMid, kKeysLast>,
                  &indexer_qk_prep_kernel<1, kSplit, kHeadsPerItem, kKeysLast>);
    else if (p.R <= 64)
        fn = pick(&indexer_qk_prep_kernel<0, kSplit, kHeadsPerItemSmall, kKeysFirst>,
                  &indexer_qk_prep_kernel<0, kSplit, kHeadsPerItemSmall, kKeysLast>,
                  &indexer_qk_prep_kernel<0, kSplit, kHeadsPerItemMid, kKeysSpread>,
                  &indexer_qk_prep_kernel<0, kSplit, kHeadsPerItemMid, kKeysLast>,
                  &indexer_qk_prep_kernel<0, kSplit, kHeadsPerItem, kKeysLast>);
    else
        fn = pick(&indexer_qk_prep_kernel<0, kContig, kHeadsPerItemSmall, kKeysFirst>,
                  &indexer_qk_prep_kernel<0, kContig, kHeadsPerItemSmall, kKeysLast>,
                  &indexer_qk_prep_kernel<0, kContig, kHeadsPerItemMid, kKeysSpread>,
                  &indexer_qk_prep_kernel<0, kContig, kHeadsPerItemMid, kKeysLast>,
                  &indexer_qk_prep_kernel<0, kContig, kHeadsPerItem, kKeysLast>);
    return hipLaunchKernel(fn, dim3(grid), dim3(block), args, 0, stream);
}

}  // namespace dsaidx
