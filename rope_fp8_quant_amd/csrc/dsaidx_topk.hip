// gfx950 kernels for the top-k selection per row that follows the index
// logits: each query keeps the index_topk highest-scoring keys ([sglang-fuse] =
// sglang PR "[AMD] [GLM5] Fuse the DSA indexer Q/K rope + quant + K-cache
// write", section Benchmark; the top-k-per-row decode launch after the paged
// MQA logits, vLLM PR 47335 "Enable fused indexer-Q RoPE+quant kernel", section
// Kernel-level evidence).
//
// Register-resident selection (topk_reg_kernel): one workgroup per segment of
// at most T*V logits, each thread holding V of them in registers for the whole
// selection, so the row is read from HBM exactly once and LDS holds only two
// 2048-bin histograms:
//   1. min and max of the finite logits (workgroup reduction);
//   2. a 2048-bin histogram of a coarse bin index that is a monotone function
//      of the value (linear between min and max, -inf first, +inf last): the
//      spread keeps the LDS atomics nearly conflict-free.  A scan from the top
//      finds the bin B1 holding the k-th largest logit and its rank in B1;
//   3. an exact radix select inside B1 on order-preserving 32-bit keys (the
//      float bits with the sign flipped for positives, all bits flipped for
//      negatives), taken relative to the smallest key in B1 so that only the
//      bits that differ are examined: digits of up to 11 bits, most often two
//      passes, none when B1 holds one distinct value;
//   4. with the k-th largest key K known, the logits above K and the first
//      needed ones equal to K are written to slots given by one workgroup
//      prefix sum (no atomics, deterministic).
// Segments are whole rows (rows up to 32768 logits), or, for longer rows, two
// launches: chunks of 16384 logits each keep their own top-k (values and
// indices into a caller workspace), then one workgroup per row selects the
// top-k of those candidates.
//
// Rows and k outside those shapes take topk_generic_kernel: one 1024-thread
// workgroup per row that streams the row (from LDS when it fits) through the
// same coarse histogram, compacts B1 into LDS, and radix-selects there (or over
// the row when B1 does not fit).
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

// Inverse of order_key.
__device__ __forceinline__ float key_value(uint32_t key) {
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
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
__global__ __launch_bounds__(kThreads) void topk_generic_kernel(const float* logits,
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


// ------------------------------------------------ register-resident path ----

// Wavefront helpers on DPP: row_shr:n is 0x110 + n (source lane - n inside a
// row of 16, zero where that leaves the row), row_ror:n is 0x120 + n.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_or_zero(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_rot(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}

// Inclusive prefix sum over the 64 lanes (every lane active).
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t v) {
    v += dpp_or_zero<0x111>(v);
    v += dpp_or_zero<0x112>(v);
    v += dpp_or_zero<0x114>(v);
    v += dpp_or_zero<0x118>(v);
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 15);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 31);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 47);
    const int row = (threadIdx.x & 63) >> 4;
    return v + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
}

// Wavefront-uniform reduction of 32-bit patterns with `op` (every lane active).
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t v, Op op) {
    v = op(v, dpp_rot<0x128>(v));
    v = op(v, dpp_rot<0x124>(v));
    v = op(v, dpp_rot<0x122>(v));
    v = op(v, dpp_rot<0x121>(v));
    const uint32_t a = op((uint32_t)__builtin_amdgcn_readlane((int)v, 0),
                          (uint32_t)__builtin_amdgcn_readlane((int)v, 16));
    const uint32_t b = op((uint32_t)__builtin_amdgcn_readlane((int)v, 32),
                          (uint32_t)__builtin_amdgcn_readlane((int)v, 48));
    return op(a, b);
}

struct MinF { __device__ uint32_t operator()(uint32_t a, uint32_t b) const {
    return __float_as_uint(fminf(__uint_as_float(a), __uint_as_float(b))); } };
struct MaxF { __device__ uint32_t operator()(uint32_t a, uint32_t b) const {
    return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b))); } };
struct MinU { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a < b ? a : b; } };
struct MaxU { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a > b ? a : b; } };

// Inclusive prefix sum over the T threads of the workgroup.  part[] holds one
// word per wavefront; it must not be read by a previous call after the last
// barrier before this one.  Ends with every thread past one barrier.
template <int T>
__device__ __forceinline__ uint32_t block_inclusive_sum(uint32_t v, uint32_t* part) {
    constexpr int W = T / 64;
    const int wave = threadIdx.x >> 6;
    const uint32_t incl = wave_inclusive_sum(v);
    if ((threadIdx.x & 63) == 63) part[wave] = incl;
    __syncthreads();
    uint32_t before = 0;
#pragma unroll
    for (int w = 0; w < W; ++w) before += w < wave ? part[w] : 0u;
    return incl + before;
}

// Bins of `hist` are ranked from the top (bin kBins-1 first).  Finds the bin
// holding the element of rank `want` (1-based, from the top) and the rank of
// that element inside its bin; every thread returns both.  Thread t owns the
// kBins/T bins just below kBins - t*kBins/T.  Three barriers.
template <int T>
__device__ __forceinline__ void select_bin(const uint32_t* hist, uint32_t want, uint32_t* part,
                                           uint32_t* sel, uint32_t& bin, uint32_t& rank) {
    constexpr int BPT = kBins / T;
    static_assert(BPT >= 1 && BPT * T == kBins, "bins per thread");
    const int base = kBins - (threadIdx.x + 1) * BPT;
    uint32_t h[BPT];
    uint32_t sum = 0;
#pragma unroll
    for (int q = 0; q < BPT; ++q) {
        h[q] = hist[base + q];
        sum += h[q];
    }
    const uint32_t incl = block_inclusive_sum<T>(sum, part);
    uint32_t acc = incl - sum;
    if (acc < want && want <= incl) {
#pragma unroll
        for (int q = BPT - 1; q >= 0; --q) {
            if (acc < want && want <= acc + h[q]) {
                sel[0] = (uint32_t)(base + q);
                sel[1] = want - acc;
            }
            acc += h[q];
        }
    }
    __syncthreads();
    bin = sel[0];
    rank = sel[1];
}

enum SegMode { kSegRows = 0, kSegChunks = 1, kSegMerge = 2 };

struct RegArgs {
    const float* logits;
    int64_t row_stride;
    const int32_t* lengths;
    int64_t cols;
    int32_t k;
    int32_t chunk;           // kSegChunks / kSegMerge: logits per chunk (> k, multiple of 4)
    int32_t chunks;          // chunks per row
    int32_t* out;            // [rows, k]
    float* ws_val;           // [rows, chunks, k]
    int32_t* ws_idx;         // [rows, chunks, k]
};

__device__ __forceinline__ int64_t row_length(const RegArgs& a, int64_t r) {
    if (!a.lengths) return a.cols;
    const int64_t l = a.lengths[r];
    return l < 0 ? 0 : (l < a.cols ? l : a.cols);
}

constexpr int kCand = 1024;   // B1 logits kept in an LDS list (more: they stay in registers)

// MODE kSegRows: one segment per row.  kSegChunks: one per (row, chunk), top-k
// values and global indices go to the workspace.  kSegMerge: one per row over
// the chunk results of its row.  T threads, V logits per thread (V % 4 == 0).
template <int MODE, int T, int V>
__global__ __launch_bounds__(T) void topk_reg_kernel(RegArgs a) {
    static_assert(V % 4 == 0 && V <= 32, "V");
    constexpr int W = T / 64;
    __shared__ uint32_t hist0[kBins + 64];   // coarse bins, then radix digits; 64 spare bins
    __shared__ uint32_t hist1[kBins];        // radix digits
    __shared__ uint32_t cand_key[kCand];
    __shared__ int32_t cand_pos[kCand];
    __shared__ uint32_t part[W];
    __shared__ uint32_t red[2][W];
    __shared__ uint32_t sel[2];
    __shared__ uint32_t cnt[3];              // list length, B1 outputs above / equal to the k-th

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int32_t k = a.k;

    // ---- the segment
    int64_t r, len;
    const float* src;
    int32_t* dst = nullptr;
    float* wv = nullptr;
    int32_t* wi = nullptr;
    const int32_t* map = nullptr;
    int64_t idx_base = 0;
    if (MODE == kSegChunks) {
        r = blockIdx.x / a.chunks;
        const int64_t j = blockIdx.x - r * a.chunks;
        const int64_t lr = row_length(a, r);
        if (lr <= k) return;                    // the merge launch writes such rows
        idx_base = j * a.chunk;
        len = lr - idx_base;
        if (len <= 0) return;
        if (len > a.chunk) len = a.chunk;
        src = a.logits + r * a.row_stride + idx_base;
        wv = a.ws_val + (r * a.chunks + j) * k;
        wi = a.ws_idx + (r * a.chunks + j) * k;
        if (len <= k) {                         // the whole chunk is a candidate
            for (int64_t p = tid; p < len; p += T) {
                wv[p] = src[p];
                wi[p] = (int32_t)(idx_base + p);
            }
            return;
        }
    } else {
        r = blockIdx.x;
        const int64_t lr = row_length(a, r);
        dst = a.out + r * (int64_t)k;
        if (lr <= k) {
            for (int64_t i = tid; i < k; i += T) dst[i] = i < lr ? (int32_t)i : -1;
            return;
        }
        if (MODE == kSegRows) {
            len = lr;
            src = a.logits + r * a.row_stride;
        } else {
            // full chunks give k candidates each; the last one min(k, rest)
            const int64_t full = lr / a.chunk, rest = lr - full * a.chunk;
            len = full * k + (rest < k ? rest : k);
            src = a.ws_val + r * a.chunks * (int64_t)k;
            map = a.ws_idx + r * a.chunks * (int64_t)k;
            if (len <= k) {
                for (int64_t i = tid; i < k; i += T) dst[i] = i < len ? map[i] : -1;
                return;
            }
        }
    }
    const int32_t n = (int32_t)len;          // <= T * V, checked on the host

    // Slot i of thread t holds logit pos(i); live(i) is false (for the whole
    // workgroup) when no thread's slot i is inside the segment.
    auto pos = [&](int i) -> int32_t {
        if (MODE == kSegMerge) return tid + i * T;
        return 4 * (tid + (i >> 2) * T) + (i & 3);
    };
    auto live = [&](int i) -> bool {
        if (MODE == kSegMerge) return i * T < n;
        return (i >> 2) * T * 4 < n;
    };
    auto write = [&](uint32_t slot, int32_t p, float v) {
        if (slot >= (uint32_t)k) return;
        if (MODE == kSegRows) {
            dst[slot] = p;
        } else if (MODE == kSegChunks) {
            wv[slot] = v;
            wi[slot] = (int32_t)(idx_base + p);
        } else {
            dst[slot] = map[p];
        }
    };

    // ---- load, as order keys; key 0 marks a slot outside the segment (no
    // logit that is not NaN has key 0)
    uint32_t key[V];
    if (MODE == kSegMerge) {
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const int32_t p = pos(i);
            key[i] = (live(i) && p < n) ? order_key(src[p]) : 0u;
        }
    } else {
        const float4* s4 = reinterpret_cast<const float4*>(src);
#pragma unroll
        for (int j = 0; j < V / 4; ++j) {
            const int32_t c = tid + j * T;
            float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
            if (live(4 * j) && 4 * c < n) f = s4[c];
            key[4 * j + 0] = 4 * c + 0 < n ? order_key(f.x) : 0u;
            key[4 * j + 1] = 4 * c + 1 < n ? order_key(f.y) : 0u;
            key[4 * j + 2] = 4 * c + 2 < n ? order_key(f.z) : 0u;
            key[4 * j + 3] = 4 * c + 3 < n ? order_key(f.w) : 0u;
        }
    }

    // ---- 1. keys of the finite min and max: finite keys lie strictly
    // between those of -inf (0x007FFFFF) and +inf (0xFF800000)
    for (int b = tid; b < kBins + 64; b += T) hist0[b] = 0;
    for (int b = tid; b < kBins; b += T) hist1[b] = 0;
    if (tid < 3) cnt[tid] = 0;
    if (tid == 0) {
        sel[0] = 0;
        sel[1] = 1;
    }
    uint32_t fmn = 0xFFFFFFFFu, fmx = 0u;
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const bool fin = key[i] - 0x00800000u < 0xFF000000u;
        fmn = min(fmn, fin ? key[i] : 0xFFFFFFFFu);
        fmx = max(fmx, fin ? key[i] : 0u);
    }
    {
        const uint32_t wmn = wave_reduce(fmn, MinU());
        const uint32_t wmx = wave_reduce(fmx, MaxU());
        if (lane == 0) {
            red[0][wave] = wmn;
            red[1][wave] = wmx;
        }
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < W; ++w) {
        fmn = min(fmn, red[0][w]);
        fmx = max(fmx, red[1][w]);
    }
    // Bins are linear in the value clamped to [lo, hi], the finite min and
    // max (-inf shares the first bin, +inf the last).  With no finite span,
    // or one too small or too large for a finite fp32 scale, every logit
    // shares bin 0.  Monotone non-decreasing either way.
    const bool any_finite = fmn <= fmx;
    const float lo = any_finite ? key_value(fmn) : 0.0f;
    const float hi = any_finite ? key_value(fmx) : 0.0f;
    const float span = hi - lo;
    float scale = (lo < hi && span < INFINITY) ? (float)kBins / span : 0.0f;
    if (!(scale < INFINITY)) scale = 0.0f;
    auto bin_of = [&](uint32_t kk) -> uint32_t {
        const float t = (__builtin_amdgcn_fmed3f(key_value(kk), lo, hi) - lo) * scale;
        return min((uint32_t)t, (uint32_t)(kBins - 1));
    };

    // ---- 2. coarse histogram (slots outside the segment count in a spare
    // bin of their lane) and the bin B1 of the k-th largest
    uint32_t bins[(V + 1) / 2];
#pragma unroll
    for (int i = 0; i < (V + 1) / 2; ++i) bins[i] = 0;
#pragma unroll
    for (int i = 0; i < V; ++i) {
        if (live(i)) {
            const uint32_t b = key[i] ? bin_of(key[i]) : (uint32_t)(kBins + lane);
            atomicAdd(&hist0[b], 1u);
            bins[i >> 1] |= b << (16 * (i & 1));
        }
    }
    __syncthreads();
    uint32_t b1, rem;
    select_bin<T>(hist0, (uint32_t)k, part, sel, b1, rem);
    b1 = min(b1, (uint32_t)(kBins - 1));
    const uint32_t n1 = hist0[b1];           // logits in B1
    const uint32_t rem0 = rem;
    auto bin_at = [&](int i) -> uint32_t { return (bins[i >> 1] >> (16 * (i & 1))) & 0xFFFFu; };

    // ---- 3. bins above B1 go out at once; B1 goes to the LDS list.  Spare
    // bins lie above kBins - 1, so the key test keeps them out.
    uint32_t n_gt = 0;
#pragma unroll
    for (int i = 0; i < V; ++i) {
        if (live(i)) {
            const uint32_t b = bin_at(i);
            n_gt += (key[i] && b > b1) ? 1u : 0u;
            if (b == b1 && n1 <= (uint32_t)kCand) {
                const uint32_t c = atomicAdd(&cnt[0], 1u);
                if (c < (uint32_t)kCand) {
                    cand_key[c] = key[i];
                    cand_pos[c] = pos(i);
                }
            }
        }
    }
    {
        uint32_t o = block_inclusive_sum<T>(n_gt, part) - n_gt;
#pragma unroll
        for (int i = 0; i < V; ++i)
            if (live(i) && key[i] && bin_at(i) > b1) write(o++, pos(i), key_value(key[i]));
    }
    const uint32_t above0 = (uint32_t)k - rem0;  // slots taken by the bins above B1
    const bool listed = n1 <= (uint32_t)kCand;

    // ---- 4a. a short list: one wavefront ranks it directly
    if (n1 <= 64) {
        if (wave == 0) {
            const bool mine = (uint32_t)lane < n1;
            const uint32_t key = mine ? cand_key[lane] : 0u;
            uint32_t rank = 0;
            for (uint32_t j = 0; j < n1; ++j) {
                const uint32_t kj = cand_key[j];
                rank += (kj > key || (kj == key && j < (uint32_t)lane)) ? 1u : 0u;
            }
            if (mine && rank < rem0) write(above0 + rank, cand_pos[lane], key_value(key));
        }
        return;
    }

    // ---- 4b. exact rank-`rem` key inside B1 by radix select, over the list
    // or, when B1 overflows it, over the registers
    auto for_b1 = [&](auto f) {
        if (listed) {
            for (uint32_t c = tid; c < n1; c += T) f(cand_key[c], cand_pos[c]);
        } else {
#pragma unroll
            for (int i = 0; i < V; ++i)
                if (live(i) && bin_at(i) == b1) f(key[i], pos(i));
        }
    };
    uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
    for_b1([&](uint32_t key, int32_t) {
        kmn = key < kmn ? key : kmn;
        kmx = key > kmx ? key : kmx;
    });
    for (int b = tid; b < kBins; b += T) hist0[b] = 0;       // n1 and select_bin read it before
    {
        const uint32_t wmn = wave_reduce(kmn, MinU());
        const uint32_t wmx = wave_reduce(kmx, MaxU());
        if (lane == 0) {
            red[0][wave] = wmn;
            red[1][wave] = wmx;
        }
    }
    __syncthreads();
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
    for (int w = 0; w < W; ++w) {
        kmin = red[0][w] < kmin ? red[0][w] : kmin;
        kmax = red[1][w] > kmax ? red[1][w] : kmax;
    }
    const uint32_t kspan = kmax - kmin;
    int top = kspan ? 32 - __clz(kspan) : 0;                 // relative keys fit in `top` bits
    uint32_t pfx = 0;                                        // their digits chosen so far
    int pass = 0;
#pragma unroll 1
    while (top > 0) {
        const int db = top < 11 ? top : 11;
        const int sh = top - db;
        uint32_t* h = (pass & 1) ? hist0 : hist1;
        for_b1([&](uint32_t key, int32_t) {
            const uint32_t rk = key - kmin;
            if (top >= 32 || (rk >> top) == pfx) atomicAdd(&h[(rk >> sh) & ((1u << db) - 1u)], 1u);
        });
        __syncthreads();
        uint32_t digit;
        select_bin<T>(h, rem, part, sel, digit, rem);
        for (int b = tid; b < kBins; b += T) h[b] = 0;
        pfx = (pfx << db) | digit;
        top = sh;
        ++pass;
    }
    const uint32_t kth = kmin + pfx;

    // ---- 5. B1 outputs: keys above kth fill [above0, k - rem), then `rem`
    // keys equal to kth fill [k - rem, k)
    const uint32_t above = (uint32_t)k - rem;
    for_b1([&](uint32_t key, int32_t p) {
        if (key > kth) {
            write(above0 + atomicAdd(&cnt[1], 1u), p, key_value(key));
        } else if (key == kth) {
            const uint32_t q = atomicAdd(&cnt[2], 1u);
            if (q < rem) write(above + q, p, key_value(key));
        }
    });
}

}  // namespace

// Kernel choice for a call; topk_workspace_bytes and launch_topk share it.
struct TopkPlan {
    int kind;          // 0: one register-resident launch per row, 1: chunks + merge, 2: generic
    int variant;       // kind 0: row shape 0..3;  kind 1: merge shape 0..2
    int64_t chunks;    // kind 1: chunks per row
    int64_t ws_bytes;  // kind 1: workspace bytes
};

// Workgroup shapes (threads x logits per thread) of the one-pass row kernel
// for rows of up to 4096, 8192, 16384 and 32768 logits.
#ifndef DSAIDX_TOPK_R4K
#define DSAIDX_TOPK_R4K 256, 16
#endif
#ifndef DSAIDX_TOPK_R8K
#define DSAIDX_TOPK_R8K 512, 16
#endif
#ifndef DSAIDX_TOPK_R16K
#define DSAIDX_TOPK_R16K 1024, 16
#endif
#ifndef DSAIDX_TOPK_R32K
#define DSAIDX_TOPK_R32K 1024, 32
#endif
// Longest row of the one-pass path; longer rows go through chunks.
#ifndef DSAIDX_TOPK_ONE_PASS_MAX
#define DSAIDX_TOPK_ONE_PASS_MAX 32768
#endif
#ifndef DSAIDX_TOPK_CHUNK_T
#define DSAIDX_TOPK_CHUNK_T 1024
#endif
#ifndef DSAIDX_TOPK_CHUNK_V
#define DSAIDX_TOPK_CHUNK_V 16
#endif
constexpr int64_t kChunk = int64_t(DSAIDX_TOPK_CHUNK_T) * DSAIDX_TOPK_CHUNK_V;
constexpr int64_t kMergeMax = 1024 * 32;   // candidates per row the merge takes

template <int T, int V>
constexpr int64_t cap() { return int64_t(T) * V; }

static TopkPlan plan_topk(int64_t rows, int64_t cols, int32_t k) {
    TopkPlan p{2, 0, 0, 0};
    if (cols <= DSAIDX_TOPK_ONE_PASS_MAX) {
        p.kind = 0;
        p.variant = cols <= cap<DSAIDX_TOPK_R4K>() ? 0
                  : cols <= cap<DSAIDX_TOPK_R8K>() ? 1
                  : cols <= cap<DSAIDX_TOPK_R16K>() ? 2 : 3;
        return p;
    }
    const int64_t chunks = (cols + kChunk - 1) / kChunk;
    if (k < kChunk && chunks * k <= kMergeMax && rows * chunks < (int64_t(1) << 31)) {
        p.kind = 1;
        p.variant = chunks * k <= 8192 ? 0 : (chunks * k <= 16384 ? 1 : 2);
        p.chunks = chunks;
        p.ws_bytes = rows * chunks * (int64_t)k * 8;
    }
    return p;
}
static_assert(cap<DSAIDX_TOPK_R4K>() >= 4096 && cap<DSAIDX_TOPK_R8K>() >= 8192 &&
                  cap<DSAIDX_TOPK_R16K>() >= 16384 && cap<DSAIDX_TOPK_R32K>() >= 32768 &&
                  DSAIDX_TOPK_ONE_PASS_MAX <= 32768,
              "row shapes must cover their row lengths");

int64_t topk_workspace_bytes(int64_t rows, int64_t cols, int32_t k) {
    return plan_topk(rows, cols, k).ws_bytes;
}

template <int MODE, int T, int V>
static hipError_t launch_reg(RegArgs& a, int64_t grid, hipStream_t stream) {
    void* args[] = {&a};
    return hipLaunchKernel(reinterpret_cast<const void*>(&topk_reg_kernel<MODE, T, V>),
                           dim3((unsigned)grid), dim3(T), args, 0, stream);
}

hipError_t launch_topk(const float* logits, int64_t row_stride, const int32_t* lengths,
                       int64_t rows, int64_t cols, int32_t k, int32_t* out, void* workspace,
                       hipStream_t stream) {
    const TopkPlan p = plan_topk(rows, cols, k);
    if (p.kind == 2) {
        void* args[] = {&logits, &row_stride, &lengths, &cols, &k, &out};
        const void* fn;
        if (cols <= 8192)
            fn = reinterpret_cast<const void*>(&topk_generic_kernel<8192, 2048>);
        else if (cols <= 24576)
            fn = reinterpret_cast<const void*>(&topk_generic_kernel<24576, 4096>);
        else
            fn = reinterpret_cast<const void*>(&topk_generic_kernel<0, 16384>);
        return hipLaunchKernel(fn, dim3((unsigned)rows), dim3(kThreads), args, 0, stream);
    }
    RegArgs a{};
    a.logits = logits;
    a.row_stride = row_stride;
    a.lengths = lengths;
    a.cols = cols;
    a.k = k;
    a.out = out;
    if (p.kind == 0) {
        switch (p.variant) {
            case 0: return launch_reg<kSegRows, DSAIDX_TOPK_R4K>(a, rows, stream);
            case 1: return launch_reg<kSegRows, DSAIDX_TOPK_R8K>(a, rows, stream);
            case 2: return launch_reg<kSegRows, DSAIDX_TOPK_R16K>(a, rows, stream);
            default: return launch_reg<kSegRows, DSAIDX_TOPK_R32K>(a, rows, stream);
        }
    }
    a.chunk = (int32_t)kChunk;
    a.chunks = (int32_t)p.chunks;
    a.ws_val = static_cast<float*>(workspace);
    a.ws_idx = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + p.ws_bytes / 2);
    const hipError_t e =
        launch_reg<kSegChunks, DSAIDX_TOPK_CHUNK_T, DSAIDX_TOPK_CHUNK_V>(a, rows * p.chunks, stream);
    if (e != hipSuccess) return e;
    switch (p.variant) {
        case 0: return launch_reg<kSegMerge, 512, 16>(a, rows, stream);
        case 1: return launch_reg<kSegMerge, 1024, 16>(a, rows, stream);
        default: return launch_reg<kSegMerge, 1024, 32>(a, rows, stream);
    }
}

}  // namespace dsaidx
