// Device code shared by the gfx950 kernels that prepare index-K rows: the
// preparation kernel (dsaidx_kernels.hip) and the projection kernel whose
// epilogue prepares the rows it has just computed (dsaidx_proj.hip).
//
// Memory helpers, the per-row arithmetic (bf16 unpacking, DPP row reductions,
// the ue8m0 exponent, the scaled fp8 convert), the RoPE lane layouts and the
// key row itself (LayerNorm, RoPE, quantisation, cache store).  The mapping
// and the arithmetic are described at the top of dsaidx_kernels.hip.
#pragma once

#include "dsaidx_internal.h"

#pragma clang fp contract(off)

// Cache policy of the streamed rows: every q/k row is read once and every code
// row written once, so they carry the nontemporal hint and do not displace the
// cos/sin rows, head gates and LayerNorm parameters, which are reused.
#ifndef DSAIDX_NT_LOADS
#define DSAIDX_NT_LOADS 1
#endif
#ifndef DSAIDX_NT_STORES
#define DSAIDX_NT_STORES 1
#endif

namespace dsaidx {
namespace {

constexpr int kContig = 0;
constexpr int kSplit = 1;
constexpr int kGeneric = 2;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));

// DPP controls (row = 16 lanes): row_ror:n reads lane (l - n) mod 16 of the row.
constexpr int kRowRor1 = 0x121;
constexpr int kRowRor2 = 0x122;
constexpr int kRowRor4 = 0x124;
constexpr int kRowRor8 = 0x128;

// ------------------------------------------------------------ memory ----

__device__ __forceinline__ uint4 load16(const uint16_t* p) {
    const u32x4* v = reinterpret_cast<const u32x4*>(p);
#if DSAIDX_NT_LOADS
    const u32x4 r = __builtin_nontemporal_load(v);
#else
    const u32x4 r = *v;
#endif
    return make_uint4(r.x, r.y, r.z, r.w);
}

__device__ __forceinline__ uint2 load8(const uint16_t* p) {
    const u32x2* v = reinterpret_cast<const u32x2*>(p);
#if DSAIDX_NT_LOADS
    const u32x2 r = __builtin_nontemporal_load(v);
#else
    const u32x2 r = *v;
#endif
    return make_uint2(r.x, r.y);
}

__device__ __forceinline__ void store8(uint8_t* p, uint2 c) {
    u32x2* v = reinterpret_cast<u32x2*>(p);
    const u32x2 w = {c.x, c.y};
#if DSAIDX_NT_STORES
    __builtin_nontemporal_store(w, v);
#else
    *v = w;
#endif
}

__device__ __forceinline__ void store4(uint8_t* p, uint32_t c) {
    uint32_t* v = reinterpret_cast<uint32_t*>(p);
#if DSAIDX_NT_STORES
    __builtin_nontemporal_store(c, v);
#else
    *v = c;
#endif
}

// The lane's eight bf16 values of one 128-element row (layout order).
template <int LAYOUT>
__device__ __forceinline__ uint4 load_row(const uint16_t* row, int j) {
    if (LAYOUT != kSplit) return load16(row + 8 * j);
    const uint2 a = load8(row + 4 * j);
    const uint2 b = load8(row + 64 + 4 * j);
    return make_uint4(a.x, a.y, b.x, b.y);
}

// The lane's eight codes of one 128-byte code row.
template <int LAYOUT>
__device__ __forceinline__ void store_row(uint8_t* row, int j, uint2 c) {
    if (LAYOUT != kSplit) {
        store8(row + 8 * j, c);
    } else {
        store4(row + 4 * j, c.x);
        store4(row + 64 + 4 * j, c.y);
    }
}

// The lane's eight fp32 LayerNorm parameters (layout order).
template <int LAYOUT>
__device__ __forceinline__ void load_params(const float* v, int j, float out[8]) {
    const float4* p = reinterpret_cast<const float4*>(v);
    const float4 a = LAYOUT != kSplit ? p[2 * j] : p[j];
    const float4 b = LAYOUT != kSplit ? p[2 * j + 1] : p[16 + j];
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

// --------------------------------------------------------- arithmetic ----

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

__device__ __forceinline__ void unpack8(const uint4& r, float x[8]) {
    x[0] = bf16_lo(r.x); x[1] = bf16_hi(r.x);
    x[2] = bf16_lo(r.y); x[3] = bf16_hi(r.y);
    x[4] = bf16_lo(r.z); x[5] = bf16_hi(r.z);
    x[6] = bf16_lo(r.w); x[7] = bf16_hi(r.w);
}

// row_ror reads a lane of the same row, always valid, so bound_ctrl changes
// nothing; it lets the move fold into the consuming op (v_max_u32_dpp).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}

// (mov_dpp rather than update_dpp with an old value: every lane is enabled
// and row_ror reads inside the row, so no old value is ever kept, and none
// has to be written into the destination first.)
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
    const unsigned long long u = (unsigned long long)__double_as_longlong(v);
    const int lo = __builtin_amdgcn_mov_dpp((int)(u & 0xFFFFFFFFull), CTRL, 0xF, 0xF, true);
    const int hi = __builtin_amdgcn_mov_dpp((int)(u >> 32), CTRL, 0xF, 0xF, true);
    return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo));
}

// Max over the 16 lanes of a DPP row of non-negative fp32 values given as bit
// patterns (for x, y >= 0 the unsigned order of the bits is the order of the
// values); every lane gets the result.
__device__ __forceinline__ uint32_t row_max_bits(uint32_t v) {
    v = max(v, dpp_u32<kRowRor8>(v));
    v = max(v, dpp_u32<kRowRor4>(v));
    v = max(v, dpp_u32<kRowRor2>(v));
    v = max(v, dpp_u32<kRowRor1>(v));
    return v;
}

// Sum over the 16 lanes of a DPP row (butterfly: every lane ends with the
// same bits, since each step adds the same two operands in either order).
__device__ __forceinline__ double row_sum(double v) {
    v = v + dpp_f64<kRowRor8>(v);
    v = v + dpp_f64<kRowRor4>(v);
    v = v + dpp_f64<kRowRor2>(v);
    v = v + dpp_f64<kRowRor1>(v);
    return v;
}

// Lane-local max |y| of eight values, as bits.
__device__ __forceinline__ uint32_t lane_amax_bits(const float y[8]) {
    float am = 0.0f;
#pragma unroll
    for (int m = 0; m < 8; ++m) am = fmaxf(am, fabsf(y[m]));
    return __float_as_uint(am);
}

// Scale exponent: the smallest e with max(amax, 1e-4) <= 448 * 2^e.  For a
// normal g = 1.f * 2^E, 448 = 1.75 * 2^8 gives e = E - 8 + [f > 0.75].  The
// floor (zero-row guard) is applied on the bits, which order like the values.
__device__ __forceinline__ int scale_exponent(uint32_t amax_bits) {
    const uint32_t b = max(amax_bits, __float_as_uint(1e-4f));
    return (int)(b >> 23) - 127 - 8 + ((b & 0x7FFFFFu) > 0x600000u ? 1 : 0);
}

// fp32 -> nearest bf16 (ties to even), kept as fp32; finite inputs.
__device__ __forceinline__ float round_bf16(float v) {
    uint32_t u = __float_as_uint(v);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return __uint_as_float(u & 0xFFFF0000u);
}

__device__ __forceinline__ float exp2_int(int e) {
    return __uint_as_float((uint32_t)(127 + e) << 23);
}

// Eight values -> eight E4M3FN bytes of y / scale (scale a power of two that
// brings every |y| within 448); element m lands in byte m of the pair of words.
__device__ __forceinline__ uint2 encode8(const float y[8], float scale) {
    // The first convert of each word writes its low half; the old operand's
    // bits are all replaced by the second convert, so any register serves.
    i16x2 lo = __builtin_bit_cast(i16x2, __float_as_uint(y[0]));
    i16x2 hi = __builtin_bit_cast(i16x2, __float_as_uint(y[4]));
    lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, y[0], y[1], scale, false);
    lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, y[2], y[3], scale, true);
    hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(hi, y[4], y[5], scale, false);
    hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(hi, y[6], y[7], scale, true);
    return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

// ---------------------------------------------------------------- rope ----

// Per-lane RoPE state for one table row.
//   contig NeoX: lanes j < R/16 hold first-half elements, R/16 <= j < R/8 the
//     second half; c[m], s[m] for the lane's element m.
//   split NeoX (R <= 64): lanes j < R/8 hold first-half elements in their
//     first four values, R/8 <= j < R/4 the second half; c[0..3], s[0..3].
//   split interleaved: the first four values hold pairs 2j, 2j+1 (c[0..1],
//     s[0..1]) when 4j < R, the last four pairs 32+2j, 33+2j (c[2..3],
//     s[2..3]) when 64 + 4j < R.
//   generic: c[m], s[m] for the lane's element m = 8j + m when it is below R
//     (bit m of mask), for either style.
// For NeoX the sine carries the pair's sign: a*c - b*s == a*c + b*(-s) exactly
// (in the generic layout for both styles).
struct RopeLane {
    float c[8];
    float s[8];
    int partner_addr;  // ds_bpermute byte address of the NeoX partner lane
    bool active;       // NeoX: the lane rotates; interleaved: first four values rotate
    bool active_hi;    // interleaved: last four values rotate
    uint32_t mask;     // generic: the lane's elements that rotate
    int rdim;          // rope_dim (generic layout; interleaved: whether any lane rotates its last four)
};

template <int STYLE, int LAYOUT, bool LANE_BRANCH = false>
__device__ __forceinline__ RopeLane rope_lane(const PrepParams& p, int64_t pos, int lane) {
    RopeLane r;
    const int j = lane & (kLanesPerRow - 1);
    const int R = p.R;
    const float* crow = p.cos + pos * p.rs;
    const float* srow = p.sin + pos * p.rs;
    r.active_hi = false;
    r.partner_addr = lane << 2;
    r.mask = 0;
    r.rdim = R;
    if constexpr (LAYOUT == kGeneric) {
        // element e = 8j + m rotates with pair i: NeoX i = e mod R/2 (the
        // first half carries -sin), interleaved i = e / 2 (even e carries -sin)
        const int half = R >> 1;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const int e = 8 * j + m;
            r.c[m] = 0.0f;
            r.s[m] = 0.0f;
            if (e < R) {
                const bool first = STYLE == 0 ? e < half : (e & 1) == 0;
                const int i = STYLE == 0 ? (first ? e : e - half) : (e >> 1);
                r.c[m] = crow[i];
                r.s[m] = first ? -srow[i] : srow[i];
                r.mask |= 1u << m;
            }
        }
        return r;
    }
    // Every lane loads (a lane outside the rope slice reads the row's first
    // entries and never uses them): a load under a per-lane condition sits in
    // a divergent branch, where the compiler waits for it before the branch
    // ends, holding back every load issued after it.  LANE_BRANCH keeps the
    // NeoX loads under the lane's condition, for one-pass query items: there
    // the cos/sin row is the item's last load, nothing queues behind it, and
    // the branch measured faster (2.03 against 2.19 us for a one-token call,
    // 2.26 against 2.37 us for 64 tokens).
    if (STYLE == 0) {
        // lanes per half of the rope slice
        const int hl = LAYOUT == kContig ? (R >> 4) : (R >> 3);
        r.active = j < 2 * hl;
        const bool first = j < hl;
        const int pj = first ? j + hl : j - hl;
        r.partner_addr = ((lane & ~(kLanesPerRow - 1)) | (r.active ? pj : j)) << 2;
        if (!LANE_BRANCH || r.active) {
            const float sg = first ? -1.0f : 1.0f;
            if (LAYOUT == kContig) {
                const int base = r.active ? 8 * (first ? j : j - hl) : 0;
                const float4 c0 = *reinterpret_cast<const float4*>(crow + base);
                const float4 c1 = *reinterpret_cast<const float4*>(crow + base + 4);
                const float4 s0 = *reinterpret_cast<const float4*>(srow + base);
                const float4 s1 = *reinterpret_cast<const float4*>(srow + base + 4);
                r.c[0] = c0.x; r.c[1] = c0.y; r.c[2] = c0.z; r.c[3] = c0.w;
                r.c[4] = c1.x; r.c[5] = c1.y; r.c[6] = c1.z; r.c[7] = c1.w;
                r.s[0] = sg * s0.x; r.s[1] = sg * s0.y; r.s[2] = sg * s0.z; r.s[3] = sg * s0.w;
                r.s[4] = sg * s1.x; r.s[5] = sg * s1.y; r.s[6] = sg * s1.z; r.s[7] = sg * s1.w;
            } else {
                const int base = r.active ? 4 * (first ? j : j - hl) : 0;
                const float4 c0 = *reinterpret_cast<const float4*>(crow + base);
                const float4 s0 = *reinterpret_cast<const float4*>(srow + base);
                r.c[0] = c0.x; r.c[1] = c0.y; r.c[2] = c0.z; r.c[3] = c0.w;
                r.s[0] = sg * s0.x; r.s[1] = sg * s0.y; r.s[2] = sg * s0.z; r.s[3] = sg * s0.w;
            }
        }
    } else {
        r.active = 4 * j < R;
        r.active_hi = 64 + 4 * j < R;
        const int lo = r.active ? 2 * j : 0;
        const float2 c0 = *reinterpret_cast<const float2*>(crow + lo);
        const float2 s0 = *reinterpret_cast<const float2*>(srow + lo);
        r.c[0] = c0.x; r.c[1] = c0.y; r.s[0] = s0.x; r.s[1] = s0.y;
        r.c[2] = r.c[3] = r.s[2] = r.s[3] = 0.0f;
        if (R > 64) {   // the same for every lane: only then does any lane rotate its last four
            const int hi = r.active_hi ? 32 + 2 * j : 0;
            const float2 c1 = *reinterpret_cast<const float2*>(crow + hi);
            const float2 s1 = *reinterpret_cast<const float2*>(srow + hi);
            r.c[2] = c1.x; r.c[3] = c1.y; r.s[2] = s1.x; r.s[3] = s1.y;
        }
    }
    return r;
}

__device__ __forceinline__ int64_t clamp_position(int64_t pos, int64_t P) {
    return pos < 0 ? 0 : (pos >= P ? P - 1 : pos);
}

// One rotated pair: (a, b) -> (a*c - b*s, b*c + a*s).
__device__ __forceinline__ void rotate_pair(float& a, float& b, float c, float s) {
    const float ac = a * c;
    const float bs = b * s;
    const float bc = b * c;
    const float as = a * s;
    a = ac - bs;
    b = bc + as;
}

// NeoX rotation of the lane's first N values given the partner's N values,
// on lanes of the rope slice.
template <int N>
__device__ __forceinline__ void rotate_neox(float x[8], const float xp[8], const RopeLane& r) {
    if (!r.active) return;
#pragma unroll
    for (int m = 0; m < N; ++m) {
        const float xc = x[m] * r.c[m];
        const float ps = xp[m] * r.s[m];
        x[m] = xc + ps;
    }
}

// One interleaved pair, rotated where `on` (computed on every lane and
// selected).
__device__ __forceinline__ void rotate_pair_if(float& a, float& b, float c, float s, bool on) {
    float ra = a, rb = b;
    rotate_pair(ra, rb, c, s);
    a = on ? ra : a;
    b = on ? rb : b;
}

// Element-wise RoPE of the generic layout.  Each DPP row of the wavefront
// writes its vector to its own 128-float slot of an LDS buffer and reads the
// partners back by index (NeoX: e +- R/2; interleaved: e ^ 1).  Only the
// wavefront's own slots are touched, and a wavefront's LDS accesses complete
// in issue order, so no workgroup barrier is involved: the wave barriers only
// keep the compiler from moving the accesses across each other.
// Wavefronts per workgroup the exchange buffer of rope_generic serves (every
// kernel that reaches it asserts that its workgroups are no larger).
constexpr int kXchgWaves = 4;

template <int STYLE>
__device__ __forceinline__ void rope_generic(float x[8], const RopeLane& rl) {
    __shared__ __align__(16) float xchg[kXchgWaves][kRowsPerWave][kRow];
    const int lane = threadIdx.x & 63;
    const int j = lane & (kLanesPerRow - 1);
    float* row = xchg[threadIdx.x >> 6][lane >> 4];
    *reinterpret_cast<float4*>(row + 8 * j) = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4*>(row + 8 * j + 4) = make_float4(x[4], x[5], x[6], x[7]);
    __builtin_amdgcn_wave_barrier();
    const int half = rl.rdim >> 1;
    float xp[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int e = 8 * j + m;
        const int partner = STYLE == 0 ? (e < half ? e + half : e - half) : (e ^ 1);
        xp[m] = (rl.mask >> m) & 1u ? row[partner] : 0.0f;
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        if ((rl.mask >> m) & 1u) {
            const float xc = x[m] * rl.c[m];
            const float ps = xp[m] * rl.s[m];
            x[m] = xc + ps;
        }
    }
}

// RoPE of one row held as eight fp32 values per lane.
template <int STYLE, int LAYOUT>
__device__ __forceinline__ void rope_row(float x[8], const RopeLane& rl) {
    if constexpr (LAYOUT == kGeneric) {
        rope_generic<STYLE>(x, rl);
        return;
    }
    if (STYLE == 0) {
        float xp[8];
        if (LAYOUT == kContig) {
#pragma unroll
            for (int m = 0; m < 8; ++m)
                xp[m] = __int_as_float(__builtin_amdgcn_ds_bpermute(rl.partner_addr, __float_as_int(x[m])));
            rotate_neox<8>(x, xp, rl);
        } else {
#pragma unroll
            for (int m = 0; m < 4; ++m)
                xp[m] = __int_as_float(__builtin_amdgcn_ds_bpermute(rl.partner_addr, __float_as_int(x[m])));
            rotate_neox<4>(x, xp, rl);
        }
    } else {
        rotate_pair_if(x[0], x[1], rl.c[0], rl.s[0], rl.active);
        rotate_pair_if(x[2], x[3], rl.c[1], rl.s[1], rl.active);
        if (rl.rdim > 64) {
            rotate_pair_if(x[4], x[5], rl.c[2], rl.s[2], rl.active_hi);
            rotate_pair_if(x[6], x[7], rl.c[3], rl.s[3], rl.active_hi);
        }
    }
}

// Same, for a query row still packed as bf16: the NeoX exchange moves the
// packed words (half as many permutes as fp32 values).
template <int STYLE, int LAYOUT>
__device__ __forceinline__ void rope_packed_row(const uint4& raw, float x[8], const RopeLane& rl) {
    unpack8(raw, x);
    if constexpr (LAYOUT == kGeneric) {
        rope_generic<STYLE>(x, rl);
        return;
    }
    if (STYLE == 0) {
        uint4 pr = raw;
        pr.x = (uint32_t)__builtin_amdgcn_ds_bpermute(rl.partner_addr, (int)raw.x);
        pr.y = (uint32_t)__builtin_amdgcn_ds_bpermute(rl.partner_addr, (int)raw.y);
        if (LAYOUT == kContig) {
            pr.z = (uint32_t)__builtin_amdgcn_ds_bpermute(rl.partner_addr, (int)raw.z);
            pr.w = (uint32_t)__builtin_amdgcn_ds_bpermute(rl.partner_addr, (int)raw.w);
        }
        float xp[8];
        unpack8(pr, xp);
        if (LAYOUT == kContig)
            rotate_neox<8>(x, xp, rl);
        else
            rotate_neox<4>(x, xp, rl);
    } else {
        rope_row<STYLE, LAYOUT>(x, rl);
    }
}

// One key row: LayerNorm, RoPE, quantisation and the cache store.  raw holds
// the lane's eight bf16 values of the row (layout order), pos its clamped
// table row and slot its cache slot; a row with valid == false computes on
// whatever it holds and stores nothing.  The caller issues the loads
// (position first: the cos/sin row waits for it, and loads retire in issue
// order; then the row and slot).
template <int STYLE, int LAYOUT>
__device__ __forceinline__ void key_row(const PrepParams& p, bool valid, uint4 raw, int64_t pos,
                                        int64_t slot, int lane) {
    const int j = lane & (kLanesPerRow - 1);
    // the LayerNorm parameters first: they depend on nothing, the cos/sin row
    // on the position
    float gam[8], bet[8];
    load_params<LAYOUT>(p.gamma, j, gam);
    load_params<LAYOUT>(p.beta, j, bet);
    const RopeLane rl = rope_lane<STYLE, LAYOUT>(p, pos, lane);

    float x[8];
    unpack8(raw, x);
    // LayerNorm: fp64 sums, fp32 mean / variance / reciprocal root.
    double s1 = 0.0;
#pragma unroll
    for (int m = 0; m < 8; ++m) s1 += (double)x[m];
    s1 = row_sum(s1);
    const float mu = (float)(s1 * (1.0 / kRow));
    float d[8];
    double s2 = 0.0;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        d[m] = x[m] - mu;
        // the product of two fp32 values is exact in fp64, so one fused
        // multiply-add rounds exactly as the product and the sum did
        s2 = __builtin_fma((double)d[m], (double)d[m], s2);
    }
    s2 = row_sum(s2);
    const float var = (float)(s2 * (1.0 / kRow));
    const float r = (float)(1.0 / sqrt((double)var + (double)p.eps));
    float n[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const float dn = d[m] * r;
        const float dg = dn * gam[m];
        n[m] = dg + bet[m];
    }

    // The unfused K-cache writer of [sglang-fuse] Accuracy rounds to bf16
    // before quantising: at both kernel boundaries (LayerNorm output and RoPE
    // output) or once, on the finished value, depending on the flag.
    const bool bf16_steps = (p.k_flags & kKeyBf16Intermediate) != 0;
    if (bf16_steps) {
#pragma unroll
        for (int m = 0; m < 8; ++m) n[m] = round_bf16(n[m]);
    }
    rope_row<STYLE, LAYOUT>(n, rl);
    if (bf16_steps || (p.k_flags & kKeyBf16Once) != 0) {
#pragma unroll
        for (int m = 0; m < 8; ++m) n[m] = round_bf16(n[m]);
    }
    const int e = scale_exponent(row_max_bits(lane_amax_bits(n)));
    const uint2 codes = encode8(n, exp2_int(e));
    if (valid && slot >= 0 && slot < p.S) {
        if (p.page_size > 0) {
            // page-interleaved cache: [page_size code rows | page_size fp32 scales]
            const int64_t page = slot / p.page_size;
            const int64_t off = slot - page * p.page_size;
            uint8_t* base = p.k_cache + page * p.page_size * (kRow + kPagedScaleBytes);
            store_row<LAYOUT>(base + off * kRow, j, codes);
            if (j == 0)
                *reinterpret_cast<float*>(base + p.page_size * kRow + off * kPagedScaleBytes) =
                    exp2_int(e);
        } else {
            store_row<LAYOUT>(p.k_cache + slot * p.k_row_stride, j, codes);
            if (j == 0) p.k_scale[slot] = exp2_int(e);
        }
    }
}

}  // namespace
}  // namespace dsaidx
