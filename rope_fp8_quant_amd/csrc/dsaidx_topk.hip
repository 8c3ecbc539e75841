// gfx950 kernel for the top-k selection per row that follows the index logits:
// each query keeps the index_topk highest-scoring keys ([sglang-fuse] = sglang
// PR "[AMD] [GLM5] Fuse the DSA indexer Q/K rope + quant + K-cache write",
// section Benchmark; the top-k-per-row decode launch after the paged MQA
// logits, vLLM PR 47335 "Enable fused indexer-Q RoPE+quant kernel", section
// Kernel-level evidence).
//
// One workgroup of 1024 threads per row:
//   0. min and max of the row's finite logits (workgroup reduction);
//   1. a 2048-bin histogram of a coarse bin index that is a monotone function
//      of the value: linear between min and max, -inf in the first bin, +inf
//      in the last.  Spreading by value (not by the top bits of the float,
//      which pile normal-looking data into a few dozen bins) keeps the LDS
//      atomics nearly conflict-free.  A scan from the top finds the bin B1
//      holding the k-th largest logit;
//   2. one more pass: logits in bins above B1 are certainly selected and are
//      written out at once; the logits of B1 (typically a few hundred) are
//      compacted into LDS with their indices;
//   3. an exact radix select over the compacted candidates on order-preserving
//      32-bit keys (the float bits with the sign flipped for positives and all
//      bits flipped for negatives): digits of 11, 11 and 10 bits, an LDS
//      histogram and a scan each; then the final pick: keys above the
//      threshold, and as many keys equal to it as are needed.
// Output slots are claimed with one atomic per wavefront (ballot + popcount).
// The row is read twice (three times with the min/max pass); rows up to 8192
// or 24576 logits are copied into LDS first and read from there.  When B1
// holds more logits than LDS takes (heavy ties), step 3 runs over the row.
#include "dsaidx_internal.h"

namespace dsaidx {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 2048;

__device__ __forceinline__ uint32_t order_key(float v) {
    const uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum over the 1024 threads of the workgroup (thread order).
__device__ __forceinline__ uint32_t block_inclusive_scan(uint32_t v, uint32_t* wave_totals) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t o = __shfl_up(v, d, 64);
        if (lane >= d) v += o;
    }
    if (lane == 63) wave_totals[wave] = v;
    __syncthreads();
    uint32_t before = 0;
    for (int w = 0; w < wave; ++w) before += wave_totals[w];
    __syncthreads();
    return v + before;
}

struct Shared {
    uint32_t hist[kBins];
    uint32_t wave_totals[kWaves];
    float wave_min[kWaves], wave_max[kWaves];
    uint32_t sel_prefix, sel_remaining, cnt_out, cnt_eq, cnt_cand;
    float lo, scale;
};

// Slot for this lane among the lanes of its wavefront with pred set, taken
// from *counter with one atomic per wavefront.  Every active lane calls it.
__device__ __forceinline__ uint32_t wave_append(uint32_t* counter, bool pred) {
    const unsigned long long mask = __ballot(pred);
    if (mask == 0) return 0;
    const int leader = __ffsll((long long)mask) - 1;
    uint32_t base = 0;
    if ((int)(threadIdx.x & 63) == leader) base = atomicAdd(counter, (uint32_t)__popcll(mask));
    base = __shfl(base, leader, 64);
    const uint32_t rank =
        __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
    return base + rank;
}

// After a histogram of nbins bins (keys matching `prefix` only), pick the bin
// holding the key of rank `remaining` from the top; every thread returns the
// prefix extended by that bin (<< shift) and the rank inside it.
__device__ __forceinline__ void pick_bin(Shared& sh, int nbins, int shift, uint32_t& prefix,
                                         uint32_t& remaining) {
    const int tid = threadIdx.x;
    const int bhi = nbins - 1 - 2 * tid;  // thread t owns bins bhi, bhi - 1 (descending)
    const int blo = bhi - 1;
    const uint32_t chi = bhi >= 0 ? sh.hist[bhi] : 0u;
    const uint32_t clo = blo >= 0 ? sh.hist[blo] : 0u;
    const uint32_t incl = block_inclusive_scan(chi + clo, sh.wave_totals);
    const uint32_t excl = incl - chi - clo;
    if (excl < remaining && remaining <= incl) {
        if (excl + chi >= remaining) {
            sh.sel_prefix = prefix | ((uint32_t)bhi << shift);
            sh.sel_remaining = remaining - excl;
        } else {
            sh.sel_prefix = prefix | ((uint32_t)blo << shift);
            sh.sel_remaining = remaining - excl - chi;
        }
    }
    __syncthreads();
    prefix = sh.sel_prefix;
    remaining = sh.sel_remaining;
    __syncthreads();
}

__device__ __forceinline__ void clear_hist(Shared& sh, int nbins) {
    for (int b = threadIdx.x; b < nbins; b += kThreads) sh.hist[b] = 0;
    __syncthreads();
}

// Calls f(valid, index, value) for every element slot of the row, 16 bytes at
// a time; all lanes of a wavefront call f together (valid may be false).
template <typename F>
__device__ __forceinline__ void for_each_value(const float4* src, int64_t len, F f) {
    const int64_t chunks = (len + 3) >> 2;
    const int64_t rounds = (chunks + kThreads - 1) / kThreads;
    for (int64_t rd = 0; rd < rounds; ++rd) {
        const int64_t c = rd * kThreads + threadIdx.x;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (c < chunks) v = src[c];
        const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int m = 0; m < 4; ++m) f(c < chunks && 4 * c + m < len, 4 * c + m, e[m]);
    }
}

// Coarse bin of a value: monotone non-decreasing in the value.
__device__ __forceinline__ uint32_t coarse_bin(float v, float lo, float scale) {
    if (v == -INFINITY) return 0;
    if (v == INFINITY) return kBins - 1;
    const float t = (v - lo) * scale;
    const int b = (int)t;
    return b < 0 ? 0u : (b > kBins - 1 ? (uint32_t)(kBins - 1) : (uint32_t)b);
}

template <int CACHE_FLOATS, int CAND>
__global__ __launch_bounds__(kThreads) void topk_per_row_kernel(const float* logits,
                                                                int64_t row_stride,
                                                                const int32_t* lengths,
                                                                int64_t cols, int32_t k,
                                                                int32_t* out) {
    __shared__ Shared sh;
    __shared__ uint32_t cand_key[CAND];
    __shared__ int32_t cand_idx[CAND];
    __shared__ float4 row_cache[CACHE_FLOATS > 0 ? CACHE_FLOATS / 4 : 1];

    const int tid = threadIdx.x;
    const int64_t r = blockIdx.x;
    int32_t* dst = out + r * (int64_t)k;
    int64_t len = cols;
    if (lengths) {
        const int64_t l = lengths[r];
        len = l < 0 ? 0 : (l < cols ? l : cols);
    }
    if (len <= k) {
        for (int64_t i = tid; i < k; i += kThreads) dst[i] = i < len ? (int32_t)i : -1;
        return;
    }
    const float4* src = reinterpret_cast<const float4*>(logits + r * row_stride);
    if (CACHE_FLOATS > 0) {
        const int64_t chunks = (len + 3) >> 2;
        for (int64_t c = tid; c < chunks; c += kThreads) row_cache[c] = src[c];
        src = row_cache;
    }

    // 0. finite min and max
    float mn = INFINITY, mx = -INFINITY;
    for_each_value(src, len, [&](bool ok, int64_t, float v) {
        if (ok && v > -INFINITY && v < INFINITY) {
            mn = fminf(mn, v);
            mx = fmaxf(mx, v);
        }
    });
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
        mn = fminf(mn, __shfl_xor(mn, d, 64));
        mx = fmaxf(mx, __shfl_xor(mx, d, 64));
    }
    if ((tid & 63) == 0) {
        sh.wave_min[tid >> 6] = mn;
        sh.wave_max[tid >> 6] = mx;
    }
    if (tid == 0) {
        sh.cnt_out = 0;
        sh.cnt_eq = 0;
        sh.cnt_cand = 0;
    }
    __syncthreads();
    if (tid == 0) {
        float a = INFINITY, b = -INFINITY;
        for (int w = 0; w < kWaves; ++w) {
            a = fminf(a, sh.wave_min[w]);
            b = fmaxf(b, sh.wave_max[w]);
        }
        // A finite scale keeps (v - lo) * scale in [0, 2048] for every finite v;
        // otherwise (one distinct finite value, or a span too small or too
        // large for fp32) all finite values share one bin.
        const float span = b - a;
        const float sc = (a < b && span < INFINITY) ? (float)kBins / span : 0.0f;
        sh.lo = a;
        sh.scale = sc < INFINITY ? sc : 0.0f;
    }
    clear_hist(sh, kBins);
    const float lo = sh.lo, scale = sh.scale;

    // 1. coarse histogram, bin B1 of the k-th largest
    for_each_value(src, len, [&](bool ok, int64_t, float v) {
        if (ok) atomicAdd(&sh.hist[coarse_bin(v, lo, scale)], 1u);
    });
    __syncthreads();
    uint32_t b1 = 0, rem = (uint32_t)k;
    pick_bin(sh, kBins, 0, b1, rem);

    // 2. bins above B1 go out; B1 becomes the candidates
    for_each_value(src, len, [&](bool ok, int64_t i, float v) {
        const uint32_t b = ok ? coarse_bin(v, lo, scale) : 0u;
        const bool take = ok && b > b1;
        const bool cand = ok && b == b1;
        const uint32_t o = wave_append(&sh.cnt_out, take);
        if (take) dst[o] = (int32_t)i;
        const uint32_t c = wave_append(&sh.cnt_cand, cand);
        if (cand && c < (uint32_t)CAND) {
            cand_key[c] = order_key(v);
            cand_idx[c] = (int32_t)i;
        }
    });
    __syncthreads();
    const uint32_t ncand = sh.cnt_cand;
    const bool compact = ncand <= (uint32_t)CAND;

    // 3. exact radix select of rank `rem` among the B1 logits
    uint32_t prefix = 0;
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
        const int bits = pass < 2 ? 11 : 10;
        const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
        const int nbins = 1 << bits;
        const uint32_t hi_mask = pass == 0 ? 0u : (0xFFFFFFFFu << (shift + bits));
        clear_hist(sh, nbins);
        if (compact) {
            for (uint32_t c = tid; c < ncand; c += kThreads) {
                const uint32_t key = cand_key[c];
                if ((key & hi_mask) == prefix)
                    atomicAdd(&sh.hist[(key >> shift) & (uint32_t)(nbins - 1)], 1u);
            }
        } else {
            for_each_value(src, len, [&](bool ok, int64_t, float v) {
                const uint32_t key = order_key(v);
                if (ok && coarse_bin(v, lo, scale) == b1 && (key & hi_mask) == prefix)
                    atomicAdd(&sh.hist[(key >> shift) & (uint32_t)(nbins - 1)], 1u);
            });
        }
        __syncthreads();
        pick_bin(sh, nbins, shift, prefix, rem);
    }

    // prefix is the k-th largest key: the B1 keys above it go out, then `rem`
    // keys equal to it fill [k - rem, k).
    const uint32_t above = (uint32_t)k - rem;
    if (compact) {
        const uint32_t rounds = (ncand + kThreads - 1) / kThreads;
        for (uint32_t rd = 0; rd < rounds; ++rd) {
            const uint32_t c = rd * kThreads + tid;
            const bool ok = c < ncand;
            const uint32_t key = ok ? cand_key[c] : 0u;
            const bool gt = ok && key > prefix, eq = ok && key == prefix;
            const uint32_t o = wave_append(&sh.cnt_out, gt);
            if (gt) dst[o] = cand_idx[c];
            const uint32_t q = wave_append(&sh.cnt_eq, eq);
            if (eq && q < rem) dst[above + q] = cand_idx[c];
        }
    } else {
        for_each_value(src, len, [&](bool ok, int64_t i, float v) {
            const uint32_t key = order_key(v);
            const bool in_b1 = ok && coarse_bin(v, lo, scale) == b1;
            const bool gt = in_b1 && key > prefix, eq = in_b1 && key == prefix;
            const uint32_t o = wave_append(&sh.cnt_out, gt);
            if (gt) dst[o] = (int32_t)i;
            const uint32_t q = wave_append(&sh.cnt_eq, eq);
            if (eq && q < rem) dst[above + q] = (int32_t)i;
        });
    }
}

}  // namespace

hipError_t launch_topk(const float* logits, int64_t row_stride, const int32_t* lengths,
                       int64_t rows, int64_t cols, int32_t k, int32_t* out, hipStream_t stream) {
    void* args[] = {&logits, &row_stride, &lengths, &cols, &k, &out};
    const void* fn;
    if (cols <= 8192)
        fn = reinterpret_cast<const void*>(&topk_per_row_kernel<8192, 2048>);
    else if (cols <= 24576)
        fn = reinterpret_cast<const void*>(&topk_per_row_kernel<24576, 4096>);
    else
        fn = reinterpret_cast<const void*>(&topk_per_row_kernel<0, 16384>);
    return hipLaunchKernel(fn, dim3((unsigned)rows), dim3(kThreads), args, 0, stream);
}

}  // namespace dsaidx
