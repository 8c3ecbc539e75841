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
// wavefront: lane j holds elements [8j, 8j+8) from a single 16-byte load, so a
// wavefront instruction moves four whole 256-byte vectors.  Row reductions
// (max |y|, LayerNorm sums) are four DPP row_ror steps; the NeoX partner of
// lane j (elements i and i + rope_dim/2 live rope_dim/16 lanes apart) comes
// from ds_bpermute.  A query work item is one token and 16 heads (4 passes of
// 4 vectors): the token's cos/sin sit in registers for all 16 heads.  A key
// work item is 4 tokens.  One dispatch runs key items on its first k_blocks
// workgroups and query items on the rest, with grid-stride loops.
//
// Arithmetic matches the definition row for row: every fp32 product and sum
// is rounded on its own (contraction is off), the LayerNorm sums are fp64,
// and the fp8 codes come from the hardware packed convert (round to nearest
// even; no value can exceed 448 because the scale is chosen from the row max).
#include "dsaidx_internal.h"

#pragma clang fp contract(off)

namespace dsaidx {
namespace {

constexpr int kPasses = kHeadsPerItem / kRowsPerWave;  // 4

// DPP controls (row = 16 lanes): row_ror:n reads lane (l - n) mod 16 of the row.
constexpr int kRowRor1 = 0x121;
constexpr int kRowRor2 = 0x122;
constexpr int kRowRor4 = 0x124;
constexpr int kRowRor8 = 0x128;

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

__device__ __forceinline__ void unpack8(const uint4& r, float x[8]) {
    x[0] = bf16_lo(r.x); x[1] = bf16_hi(r.x);
    x[2] = bf16_lo(r.y); x[3] = bf16_hi(r.y);
    x[4] = bf16_lo(r.z); x[5] = bf16_hi(r.z);
    x[6] = bf16_lo(r.w); x[7] = bf16_hi(r.w);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
    const unsigned long long u = (unsigned long long)__double_as_longlong(v);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(u & 0xFFFFFFFFull), CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(u >> 32), CTRL, 0xF, 0xF, false);
    return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo));
}

// Max over the 16 lanes of a DPP row; every lane gets the result.
__device__ __forceinline__ float row_max(float v) {
    v = fmaxf(v, dpp_f32<kRowRor8>(v));
    v = fmaxf(v, dpp_f32<kRowRor4>(v));
    v = fmaxf(v, dpp_f32<kRowRor2>(v));
    v = fmaxf(v, dpp_f32<kRowRor1>(v));
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

// Scale exponent: the smallest e with max(amax, 1e-4) <= 448 * 2^e.  For a
// normal g = 1.f * 2^E, 448 = 1.75 * 2^8 gives e = E - 8 + [f > 0.75].
__device__ __forceinline__ int scale_exponent(float amax) {
    const uint32_t b = __float_as_uint(fmaxf(amax, 1e-4f));
    return (int)(b >> 23) - 127 - 8 + ((b & 0x7FFFFFu) > 0x600000u ? 1 : 0);
}

__device__ __forceinline__ float exp2_int(int e) {
    return __uint_as_float((uint32_t)(127 + e) << 23);
}

// Eight fp32 values (already in [-448, 448]) -> eight E4M3FN bytes, element m
// in byte m.
__device__ __forceinline__ uint2 encode8(const float v[8]) {
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], lo, true);
    int hi = __builtin_amdgcn_cvt_pk_fp8_f32(v[4], v[5], 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(v[6], v[7], hi, true);
    return make_uint2((uint32_t)lo, (uint32_t)hi);
}

// Per-lane RoPE state for one table row.
//   NeoX: lanes j < R/16 hold first-half elements, lanes R/16 <= j < R/8 the
//     matching second half; c[m], s[m] are the angles of the lane's element m
//     with the sign of the sine folded in (a*c - b*s == a*c + b*(-s) exactly).
//   Interleaved: lanes j < R/8 hold four whole pairs; c[0..3], s[0..3].
struct RopeLane {
    float c[8];
    float s[8];
    int partner_addr;  // ds_bpermute byte address of the NeoX partner lane
    bool active;
};

template <int STYLE>
__device__ __forceinline__ RopeLane rope_lane(const PrepParams& p, int64_t pos, int lane) {
    RopeLane r;
    const int j = lane & (kLanesPerRow - 1);
    const int R = p.R;
    const int64_t rowoff = pos * p.rs;
    if (STYLE == 0) {
        const int hl = R >> 4;  // lanes per half of the rope slice
        r.active = j < 2 * hl;
        const bool first = j < hl;
        const int pj = first ? j + hl : j - hl;
        r.partner_addr = ((lane & ~(kLanesPerRow - 1)) | (r.active ? pj : j)) << 2;
        if (r.active) {
            const int base = 8 * (first ? j : j - hl);
            const float4* cp = reinterpret_cast<const float4*>(p.cos + rowoff + base);
            const float4* sp = reinterpret_cast<const float4*>(p.sin + rowoff + base);
            const float4 c0 = cp[0], c1 = cp[1], s0 = sp[0], s1 = sp[1];
            r.c[0] = c0.x; r.c[1] = c0.y; r.c[2] = c0.z; r.c[3] = c0.w;
            r.c[4] = c1.x; r.c[5] = c1.y; r.c[6] = c1.z; r.c[7] = c1.w;
            const float sg = first ? -1.0f : 1.0f;
            r.s[0] = sg * s0.x; r.s[1] = sg * s0.y; r.s[2] = sg * s0.z; r.s[3] = sg * s0.w;
            r.s[4] = sg * s1.x; r.s[5] = sg * s1.y; r.s[6] = sg * s1.z; r.s[7] = sg * s1.w;
        }
    } else {
        r.active = j < (R >> 3);
        r.partner_addr = lane << 2;
        if (r.active) {
            const float4 c0 = *reinterpret_cast<const float4*>(p.cos + rowoff + 4 * j);
            const float4 s0 = *reinterpret_cast<const float4*>(p.sin + rowoff + 4 * j);
            r.c[0] = c0.x; r.c[1] = c0.y; r.c[2] = c0.z; r.c[3] = c0.w;
            r.s[0] = s0.x; r.s[1] = s0.y; r.s[2] = s0.z; r.s[3] = s0.w;
        }
    }
    return r;
}

__device__ __forceinline__ int64_t clamp_position(int64_t pos, int64_t P) {
    return pos < 0 ? 0 : (pos >= P ? P - 1 : pos);
}

// NeoX rotation of the lane's eight values, given the partner lane's eight.
__device__ __forceinline__ void rotate_neox(float x[8], const float xp[8], const RopeLane& r) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const float xc = x[m] * r.c[m];
        const float ps = xp[m] * r.s[m];
        x[m] = xc + ps;
    }
}

// Interleaved rotation of the lane's four pairs.
__device__ __forceinline__ void rotate_interleaved(float x[8], const RopeLane& r) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const float a = x[2 * m], b = x[2 * m + 1];
        const float ac = a * r.c[m];
        const float bs = b * r.s[m];
        const float bc = b * r.c[m];
        const float as = a * r.s[m];
        x[2 * m] = ac - bs;
        x[2 * m + 1] = bc + as;
    }
}

// Row max -> exponent -> codes for the lane's eight values.
__device__ __forceinline__ uint2 quantize8(const float y[8], int& e_out) {
    float am = 0.0f;
#pragma unroll
    for (int m = 0; m < 8; ++m) am = fmaxf(am, fabsf(y[m]));
    am = row_max(am);
    const int e = scale_exponent(am);
    const float inv = exp2_int(-e);
    float v[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) v[m] = y[m] * inv;
    e_out = e;
    return encode8(v);
}

template <int STYLE>
__device__ __forceinline__ void query_item(const PrepParams& p, int64_t item, int lane) {
    const int g = lane >> 4;
    const int j = lane & (kLanesPerRow - 1);
    const int64_t t = item / p.head_blocks;
    const int hb = (int)(item - t * p.head_blocks);
    const int64_t pos = clamp_position(p.q_pos[t], p.P);
    const RopeLane rl = rope_lane<STYLE>(p, pos, lane);

    // Issue every load of the item before any arithmetic.
    uint4 raw[kPasses];
    uint32_t wbits[kPasses];
#pragma unroll
    for (int ps = 0; ps < kPasses; ++ps) {
        const int h = hb * kHeadsPerItem + ps * kRowsPerWave + g;
        raw[ps] = make_uint4(0, 0, 0, 0);
        wbits[ps] = 0;
        if (h < p.H) {
            raw[ps] = *reinterpret_cast<const uint4*>(p.q + t * p.q_st + (int64_t)h * p.q_sh + 8 * j);
            if (j == 0) wbits[ps] = p.w[t * p.w_st + h];
        }
    }

#pragma unroll
    for (int ps = 0; ps < kPasses; ++ps) {
        const int h = hb * kHeadsPerItem + ps * kRowsPerWave + g;
        float x[8];
        unpack8(raw[ps], x);
        if (STYLE == 0) {
            uint4 pr;
            pr.x = (uint32_t)__builtin_amdgcn_ds_bpermute(rl.partner_addr, (int)raw[ps].x);
            pr.y = (uint32_t)__builtin_amdgcn_ds_bpermute(rl.partner_addr, (int)raw[ps].y);
            pr.z = (uint32_t)__builtin_amdgcn_ds_bpermute(rl.partner_addr, (int)raw[ps].z);
            pr.w = (uint32_t)__builtin_amdgcn_ds_bpermute(rl.partner_addr, (int)raw[ps].w);
            float xp[8];
            unpack8(pr, xp);
            if (rl.active) rotate_neox(x, xp, rl);
        } else {
            if (rl.active) rotate_interleaved(x, rl);
        }
        int e;
        const uint2 codes = quantize8(x, e);
        if (h < p.H) {
            const int64_t row = t * p.H + h;
            *reinterpret_cast<uint2*>(p.q_fp8 + row * kRow + 8 * j) = codes;
            if (j == 0) {
                const float sc = exp2_int(e);
                const float ws = __uint_as_float(wbits[ps] << 16) * p.weight_scale;
                p.w_out[row] = ws * sc;
                if (p.q_scale) p.q_scale[row] = sc;
            }
        }
    }
}

template <int STYLE>
__device__ __forceinline__ void key_item(const PrepParams& p, int64_t item, int lane) {
    const int g = lane >> 4;
    const int j = lane & (kLanesPerRow - 1);
    const int64_t t = item * kTokensPerKItem + g;
    const bool valid = t < p.T;

    uint4 raw = make_uint4(0, 0, 0, 0);
    int64_t pos = 0, slot = -1;
    if (valid) {
        raw = *reinterpret_cast<const uint4*>(p.k + t * p.k_st + 8 * j);
        pos = clamp_position(p.k_pos[t], p.P);
        slot = p.loc[t];
    }
    const RopeLane rl = rope_lane<STYLE>(p, pos, lane);
    const float4 g0 = reinterpret_cast<const float4*>(p.gamma)[2 * j];
    const float4 g1 = reinterpret_cast<const float4*>(p.gamma)[2 * j + 1];
    const float4 b0 = reinterpret_cast<const float4*>(p.beta)[2 * j];
    const float4 b1 = reinterpret_cast<const float4*>(p.beta)[2 * j + 1];
    const float gam[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    const float bet[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};

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
        s2 += (double)d[m] * (double)d[m];
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

    if (STYLE == 0) {
        float np[8];
#pragma unroll
        for (int m = 0; m < 8; ++m)
            np[m] = __int_as_float(__builtin_amdgcn_ds_bpermute(rl.partner_addr, __float_as_int(n[m])));
        if (rl.active) rotate_neox(n, np, rl);
    } else {
        if (rl.active) rotate_interleaved(n, rl);
    }
    int e;
    const uint2 codes = quantize8(n, e);
    if (valid && slot >= 0 && slot < p.S) {
        *reinterpret_cast<uint2*>(p.k_cache + slot * p.k_row_stride + 8 * j) = codes;
        if (j == 0) p.k_scale[slot] = exp2_int(e);
    }
}

template <int STYLE>
__global__ __launch_bounds__(256) void indexer_qk_prep_kernel(PrepParams p) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int waves = (int)(blockDim.x >> 6);
    if ((int)blockIdx.x < p.k_blocks) {
        const int64_t stride = (int64_t)p.k_blocks * waves;
        for (int64_t it = (int64_t)blockIdx.x * waves + wave; it < p.k_items; it += stride)
            key_item<STYLE>(p, it, lane);
    } else {
        const int64_t qb = (int64_t)blockIdx.x - p.k_blocks;
        const int64_t stride = ((int64_t)gridDim.x - p.k_blocks) * waves;
        for (int64_t it = qb * waves + wave; it < p.q_items; it += stride)
            query_item<STYLE>(p, it, lane);
    }
}

// Eight consecutive values per lane through the same encode8 as the kernels.
__global__ __launch_bounds__(256) void fp8_encode_selftest_kernel(const float* in, uint8_t* out,
                                                                  int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x * 8;
    for (int64_t base = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8; base < n;
         base += stride) {
        float v[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) v[m] = base + m < n ? in[base + m] : 0.0f;
        const uint2 c = encode8(v);
        if (base + 8 <= n) {
            *reinterpret_cast<uint2*>(out + base) = c;
        } else {
            for (int m = 0; base + m < n; ++m)
                out[base + m] = (uint8_t)(((m < 4 ? c.x : c.y) >> (8 * (m & 3))) & 0xFFu);
        }
    }
}

}  // namespace

hipError_t launch_fp8_selftest(const float* in, uint8_t* out, int64_t n, unsigned grid,
                               hipStream_t stream) {
    void* args[] = {&in, &out, &n};
    return hipLaunchKernel(reinterpret_cast<const void*>(&fp8_encode_selftest_kernel), dim3(grid),
                           dim3(256), args, 0, stream);
}

hipError_t launch_prep(const PrepParams& p, int style, unsigned grid, unsigned block,
                       hipStream_t stream) {
    PrepParams copy = p;
    void* args[] = {&copy};
    const void* fn = style == 0 ? reinterpret_cast<const void*>(&indexer_qk_prep_kernel<0>)
                                : reinterpret_cast<const void*>(&indexer_qk_prep_kernel<1>);
    return hipLaunchKernel(fn, dim3(grid), dim3(block), args, 0, stream);
}

}  // namespace dsaidx
