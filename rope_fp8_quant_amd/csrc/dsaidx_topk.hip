// gfx950 kernels for the top-k selection per row that follows the index
// logits: each query keeps the index_topk highest-scoring keys ([sglang-fuse] =
// sglang PR "[AMD] [GLM5] Fuse the DSA indexer Q/K rope + quant + K-cache
// write", section Benchmark; the top-k-per-row decode launch after the paged
// MQA logits, vLLM PR 47335 "Enable fused indexer-Q RoPE+quant kernel", section
// Kernel-level evidence).
//
// Both paths select on order-preserving 32-bit keys: the float bits with the
// sign flipped for positives and all bits flipped for negatives, so unsigned
// key order is value order (-0 just below +0; NaN is outside the contract).
//
// Rows of up to 32768 logits (topk_row_kernel): one workgroup per row, each
// thread holding V of the row's logits in registers for the whole selection,
// so the row is read from HBM once and LDS holds only two 2048-bin histograms
// and a short list.  The per-logit work is kept to integer compares on the
// keys:
//   1. a 2048-bin histogram of the keys' top 11 bits (sign, exponent, two
//      mantissa bits); wavefront 0 scans it from the top for the bin B1 that
//      holds the k-th largest logit and its rank in B1;
//   2. logits in bins above B1 are written, and B1's logits appended to an
//      LDS list, at offsets from one workgroup prefix sum of both counts (no
//      atomics);
//   3. a list of at most 64 is ranked by one wavefront directly.  A longer
//      one is radix-selected on the 21 bits below B1's prefix, 11 then 10
//      bits: in calls of many rows by wavefront 0 alone (no workgroup
//      barriers; the other wavefronts leave the compute unit to other rows),
//      in smaller calls by every wavefront adding to the digit histograms and
//      wavefront 0 choosing each digit.  When B1 overflows the list (a narrow
//      value range), the workgroup selects over the registers, on keys
//      relative to B1's smallest key.  The list's keys above the k-th and the
//      needed keys equal to it fill the remaining slots.
// Linear bins between the row's min and max adapt better to a narrow value
// range, but cost a min/max pass and about eight more instructions per logit:
// 14.5 against 12.5 us for 64 rows of 16384, 75 against 72 us for the causal
// 8192-row prefill (measured when adopted).
// Longer rows take the split-row path below (four dispatches over a caller
// workspace), which spreads one row over many workgroups.
#include "dsaidx_internal.h"

#include <atomic>

namespace dsaidx {
namespace {

constexpr int kBins = 2048;

__device__ __forceinline__ uint32_t order_key(float v) {
    const uint32_t u = __float_as_uint(v);
    return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
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

// Bins are ranked from the top (bin kBins-1 first); thread t owns the
// kBins/T bins just below kBins - t*kBins/T, given in h[] (lowest first).
// Finds the bin holding the element of rank `want` (1-based, from the top)
// and the rank of that element inside its bin; every thread returns both.
// Two barriers.
template <int T>
__device__ __forceinline__ void select_bin_regs(const uint32_t (&h)[kBins / T], uint32_t want,
                                                uint32_t* part, uint32_t* sel, uint32_t& bin,
                                                uint32_t& rank) {
    constexpr int BPT = kBins / T;
    static_assert(BPT >= 1 && BPT * T == kBins, "bins per thread");
    const int base = kBins - (threadIdx.x + 1) * BPT;
    uint32_t sum = 0;
#pragma unroll
    for (int q = 0; q < BPT; ++q) sum += h[q];
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

// This thread's bins of a histogram (LDS or global), for select_bin_regs.
template <int T>
__device__ __forceinline__ void load_bins(const uint32_t* hist, uint32_t (&h)[kBins / T]) {
    constexpr int BPT = kBins / T;
    const int base = kBins - (threadIdx.x + 1) * BPT;
#pragma unroll
    for (int q = 0; q < BPT; ++q) h[q] = hist[base + q];
}

template <int T>
__device__ __forceinline__ void select_bin(const uint32_t* hist, uint32_t want, uint32_t* part,
                                           uint32_t* sel, uint32_t& bin, uint32_t& rank) {
    uint32_t h[kBins / T];
    load_bins<T>(hist, h);
    select_bin_regs<T>(h, want, part, sel, bin, rank);
}

// Lanes of this wavefront below this one whose bit is set in m.
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Orders this wavefront's earlier LDS writes and atomics before its later LDS
// reads by other lanes (a wavefront's LDS operations complete in order).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One wavefront, every lane active: the bin of an NB-bin LDS histogram
// (ranked from the top) that holds the element of rank `want` (1-based, at
// most the histogram's total), and that element's rank inside the bin.
// Lane l sums the NB/64 bins below NB - l*NB/64; a wavefront scan finds the
// lane whose bins hold rank `want`, then the first NB/64 lanes scan that
// lane's bins one each.
template <int NB>
__device__ __forceinline__ void wave_select(const uint32_t* h, uint32_t want, uint32_t& bin,
                                            uint32_t& rank) {
    constexpr int PL = NB / 64;
    static_assert(PL % 4 == 0 && PL <= 64 && (PL & (PL - 1)) == 0, "bins per lane");
    const int lane = threadIdx.x & 63;
    // Each lane starts at another 16-byte piece of its bins, so that the
    // lanes of one load spread over the LDS banks (lanes PL words apart would
    // otherwise all hit the same banks).
    uint32_t s = 0;
#pragma unroll
    for (int q = 0; q < PL; q += 4) {
        const int qs = (q + 4 * lane) & (PL - 1);
        const uint4 v = *reinterpret_cast<const uint4*>(&h[NB - (lane + 1) * PL + qs]);
        s += v.x + v.y + v.z + v.w;
    }
    const uint32_t incl = wave_inclusive_sum(s);
    const uint64_t m = __builtin_amdgcn_ballot_w64(incl >= want);
    const int L = m ? (int)__builtin_ctzll(m) : 63;
    const uint32_t above = (uint32_t)__builtin_amdgcn_readlane((int)(incl - s), L);
    const int top = NB - 1 - L * PL;                      // lane L's highest bin
    const uint32_t c = lane < PL ? h[top - lane] : 0u;
    const uint32_t ci = wave_inclusive_sum(c);
    const uint64_t m2 = __builtin_amdgcn_ballot_w64(lane < PL && above + ci >= want);
    const int j = m2 ? (int)__builtin_ctzll(m2) : PL - 1;
    bin = (uint32_t)(top - j);
    rank = want - above - (uint32_t)__builtin_amdgcn_readlane((int)(ci - c), j);
}

struct RowArgs {
    const float* logits;
    int64_t row_stride;
    const int32_t* lengths;
    int64_t cols;
    int32_t k;
    int32_t* out;            // [rows, k]
    int32_t many_rows;       // nonzero: several row workgroups per compute unit (see kManyRows)
};

constexpr int kCand = 1024;   // B1 logits kept in an LDS list (more: they stay in registers)

// One workgroup per row of at most T * V logits (V % 4 == 0).  MINW: waves
// per SIMD the register allocation must leave room for (1: no constraint).
template <int T, int V, int MINW>
__global__ __launch_bounds__(T, MINW) void topk_row_kernel(RowArgs a) {
    static_assert(V % 4 == 0 && V <= 32, "V");
    constexpr int W = T / 64;
    __shared__ __align__(16) uint32_t hist0[kBins + 64];   // coarse bins, then radix digits; 64 spare bins
    __shared__ __align__(16) uint32_t hist1[kBins];        // radix digits
    __shared__ uint32_t cand_key[kCand];
    __shared__ int32_t cand_pos[kCand];
    __shared__ uint32_t part[W];
    __shared__ uint32_t red[2][W];
    __shared__ uint32_t sel[2];
    __shared__ uint32_t cnt[2];              // B1 outputs above / equal to the k-th

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int32_t k = a.k;
    const int64_t r = blockIdx.x;
    const float4* s4 = reinterpret_cast<const float4*>(a.logits + r * a.row_stride);
    // Thread t's register group j holds logits 4 * (t + j * T) + 0..3.  In a
    // call of few rows the groups are loaded before the row's length is
    // known, up to the column count (one memory round trip less on the
    // row's critical path); in a call of many rows only up to the length.
    float4 f[V / 4];
    if (!a.many_rows) {
        const int32_t cols4 = (int32_t)((a.cols + 3) / 4);   // rows hold whole float4s
#pragma unroll
        for (int j = 0; j < V / 4; ++j) {
            const int32_t c = tid + j * T;
            f[j] = c < cols4 ? s4[c] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
    int64_t len = a.cols;
    if (a.lengths) {
        const int64_t l = a.lengths[r];
        len = l < 0 ? 0 : (l < a.cols ? l : a.cols);
    }
    int32_t* dst = a.out + r * (int64_t)k;
    if (len <= k) {
        for (int64_t i = tid; i < k; i += T) dst[i] = i < len ? (int32_t)i : -1;
        return;
    }
    const int32_t n = (int32_t)len;          // <= T * V, checked on the host

    // Slot i of thread t holds logit pos(i); live(i) is false (for the whole
    // workgroup) when no thread's slot i is inside the row.
    auto pos = [&](int i) -> int32_t { return 4 * (tid + (i >> 2) * T) + (i & 3); };
    auto live = [&](int i) -> bool { return (i >> 2) * T * 4 < n; };
    auto write = [&](uint32_t slot, int32_t p) {
        if (slot < (uint32_t)k) dst[slot] = p;
    };

    // ---- order keys; key 0 marks a slot outside the row (no logit that is
    // not NaN has key 0), so the count and write passes below need no bound
    // checks.  Register group j is full when all its slots lie inside the
    // row, the same for the whole workgroup: only the group that straddles
    // the row's end pays for per-slot checks.
    auto full = [&](int j) -> bool { return (j + 1) * T * 4 <= n; };
    uint32_t key[V];
    {
        if (a.many_rows) {
#pragma unroll
            for (int j = 0; j < V / 4; ++j) {
                const int32_t c = tid + j * T;
                f[j] = make_float4(0.f, 0.f, 0.f, 0.f);
                if (full(j) || (live(4 * j) && 4 * c < n)) f[j] = s4[c];
            }
        }
#pragma unroll
        for (int j = 0; j < V / 4; ++j) {
            key[4 * j + 0] = order_key(f[j].x);
            key[4 * j + 1] = order_key(f[j].y);
            key[4 * j + 2] = order_key(f[j].z);
            key[4 * j + 3] = order_key(f[j].w);
        }
#pragma unroll
        for (int j = 0; j < V / 4; ++j) {
            if (!full(j)) {
                const int32_t c = tid + j * T;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (!live(4 * j) || 4 * c + e >= n) key[4 * j + e] = 0u;
            }
        }
    }

    {
        const uint4 z = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int b = 4 * tid; b < kBins; b += 4 * T) {
            *reinterpret_cast<uint4*>(&hist0[b]) = z;
            *reinterpret_cast<uint4*>(&hist1[b]) = z;
        }
        if (tid < 16) *reinterpret_cast<uint4*>(&hist0[kBins + 4 * tid]) = z;
    }
    if (tid < 2) cnt[tid] = 0;
    if (tid == 0) {
        sel[0] = 0;
        sel[1] = 1;
    }
    __syncthreads();
    // ---- 1. histogram of the keys' top 11 bits (slots outside the row count
    // in a spare bin of their lane) and the bin B1 of the k-th largest
#pragma unroll
    for (int j = 0; j < V / 4; ++j) {
        if (full(j)) {
#pragma unroll
            for (int e = 0; e < 4; ++e) atomicAdd(&hist0[key[4 * j + e] >> 21], 1u);
        } else if (live(4 * j)) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t kk = key[4 * j + e];
                atomicAdd(&hist0[kk ? kk >> 21 : (uint32_t)(kBins + lane)], 1u);
            }
        }
    }
    __syncthreads();
    if (wave == 0) {
        uint32_t bin, rank;
        wave_select<kBins>(hist0, (uint32_t)k, bin, rank);
        if (lane == 0) {
            sel[0] = bin;
            sel[1] = rank;
        }
    }
    __syncthreads();
    const uint32_t b1 = sel[0];
    uint32_t rem = sel[1];
    const uint32_t n1 = hist0[b1];           // logits in B1
    const uint32_t rem0 = rem;
    // Keys above hi_m1 are in bins above B1 (none when B1 is the top bin);
    // keys above lo_m1 are in B1 or above.  Key 0 is above neither: B1 is
    // never bin 0, which holds no logit that is not NaN.
    const uint32_t hi_m1 = ((b1 + 1) << 21) - 1u;
    const uint32_t lo_m1 = (b1 << 21) - 1u;
    auto bin_at = [&](int i) -> uint32_t { return key[i] >> 21; };

    // ---- 2. bins above B1 go out at once and B1 goes to the LDS list, at
    // offsets from one workgroup prefix sum of both counts (above B1 in the
    // low half-word, in B1 in the high one; each total is at most 32768)
    const bool listed = n1 <= (uint32_t)kCand;
    {
        uint32_t n_gt = 0, n_ge = 0;
#pragma unroll
        for (int i = 0; i < V; ++i) {
            n_gt += key[i] > hi_m1 ? 1u : 0u;
            n_ge += key[i] > lo_m1 ? 1u : 0u;
        }
        const uint32_t packed = n_gt | ((n_ge - n_gt) << 16);
        const uint32_t before = block_inclusive_sum<T>(packed, part) - packed;
        // Compare again below rather than keep 2V lane masks alive across the
        // prefix sum (they would spill to VGPR lanes).
#pragma unroll
        for (int i = 0; i < V; ++i) asm volatile("" : "+v"(key[i]));
        uint32_t o_gt = before & 0xFFFFu;
        if (listed) {
            uint32_t o_b1 = before >> 16;
#pragma unroll
            for (int i = 0; i < V; ++i) {
                if (key[i] > hi_m1) {
                    dst[o_gt++] = pos(i);
                } else if (key[i] > lo_m1) {
                    cand_key[o_b1] = key[i];
                    cand_pos[o_b1] = pos(i);
                    ++o_b1;
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < V; ++i)
                if (key[i] > hi_m1) dst[o_gt++] = pos(i);
        }
    }
    const uint32_t above0 = (uint32_t)k - rem0;  // slots taken by the bins above B1
    __syncthreads();                             // the list is complete

    // ---- 3a. a short list: wavefront 0 ranks it directly
    if (n1 <= 64) {
        if (wave == 0) {
            const bool mine = (uint32_t)lane < n1;
            const uint32_t key = mine ? cand_key[lane] : 0u;
            uint32_t rank = 0;
            for (uint32_t j = 0; j < n1; ++j) {
                const uint32_t kj = cand_key[j];
                rank += (kj > key || (kj == key && j < (uint32_t)lane)) ? 1u : 0u;
            }
            if (mine && rank < rem0) write(above0 + rank, cand_pos[lane]);
        }
        return;
    }

    // ---- 3b. a longer list, when many rows share each compute unit:
    // wavefront 0 alone resolves it with no further workgroup barriers, and
    // the other wavefronts leave the compute unit to other rows.  B1's keys
    // share their top 11 bits; two radix passes on the 21 bits below (11,
    // then 10) give the rank-rem0 key.  Bin indices are masked so that they
    // stay inside the histograms whatever the list holds.
    if (listed && a.many_rows) {
        if (wave != 0) return;
        const uint32_t base = b1 << 21;
        for (uint32_t c = lane; c < n1; c += 64)
            atomicAdd(&hist1[((cand_key[c] - base) >> 10) & (kBins - 1)], 1u);
        {
            const uint4 z = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
            for (int b = 4 * lane; b < 1024; b += 4 * 64) *reinterpret_cast<uint4*>(&hist0[b]) = z;
        }
        wave_lds_sync();
        uint32_t d1, r1;
        wave_select<kBins>(hist1, rem0, d1, r1);
        for (uint32_t c = lane; c < n1; c += 64) {
            const uint32_t rk = cand_key[c] - base;
            if (((rk >> 10) & (kBins - 1)) == d1) atomicAdd(&hist0[rk & 1023u], 1u);
        }
        wave_lds_sync();
        uint32_t d2, r2;
        wave_select<1024>(hist0, r1, d2, r2);
        const uint32_t kth = base + (d1 << 10) + d2;
        // keys above kth fill [above0, k - r2); the first r2 keys equal to it
        // fill [k - r2, k)
        uint32_t n_above = 0, n_eq = 0;
        for (uint32_t c0 = 0; c0 < n1; c0 += 64) {
            const uint32_t c = c0 + lane;
            const bool ok = c < n1;
            const uint32_t key = ok ? cand_key[c] : 0u;
            const bool gt = ok && key > kth;
            const bool eq = ok && key == kth;
            const uint64_t mg = __builtin_amdgcn_ballot_w64(gt);
            const uint64_t me = __builtin_amdgcn_ballot_w64(eq);
            if (gt) write(above0 + n_above + lanes_below(mg), cand_pos[c]);
            if (eq) {
                const uint32_t q = n_eq + lanes_below(me);
                if (q < r2) write((uint32_t)k - r2 + q, cand_pos[c]);
            }
            n_above += (uint32_t)__builtin_popcountll(mg);
            n_eq += (uint32_t)__builtin_popcountll(me);
        }
        return;
    }

    // ---- 4. a longer list in a smaller call: the same two radix passes, with
    // every wavefront adding to the digit histograms and wavefront 0 choosing
    // each digit (one barrier to publish it), then every wavefront writes
    if (listed) {
        const uint32_t base = b1 << 21;
        for (uint32_t c = tid; c < n1; c += T)
            atomicAdd(&hist1[((cand_key[c] - base) >> 10) & (kBins - 1)], 1u);
        {
            const uint4 z = make_uint4(0u, 0u, 0u, 0u);
            for (int b = 4 * tid; b < 1024; b += 4 * T) *reinterpret_cast<uint4*>(&hist0[b]) = z;
        }
        __syncthreads();
        if (wave == 0) {
            uint32_t d, r;
            wave_select<kBins>(hist1, rem0, d, r);
            if (lane == 0) {
                sel[0] = d;
                sel[1] = r;
            }
        }
        __syncthreads();
        const uint32_t d1 = sel[0], r1 = sel[1];
        for (uint32_t c = tid; c < n1; c += T) {
            const uint32_t rk = cand_key[c] - base;
            if (((rk >> 10) & (kBins - 1)) == d1) atomicAdd(&hist0[rk & 1023u], 1u);
        }
        __syncthreads();                                     // also: every thread has read sel
        if (wave == 0) {
            uint32_t d, r;
            wave_select<1024>(hist0, r1, d, r);
            if (lane == 0) {
                sel[0] = d;
                sel[1] = r;
            }
        }
        __syncthreads();
        const uint32_t kth = base + (d1 << 10) + sel[0];
        const uint32_t r2 = sel[1];
        // keys above kth fill [above0, k - r2); r2 keys equal to it fill [k - r2, k)
        for (uint32_t c = tid; c < n1; c += T) {
            const uint32_t key = cand_key[c];
            if (key > kth) {
                write(above0 + atomicAdd(&cnt[0], 1u), cand_pos[c]);
            } else if (key == kth) {
                const uint32_t q = atomicAdd(&cnt[1], 1u);
                if (q < r2) write((uint32_t)k - r2 + q, cand_pos[c]);
            }
        }
        return;
    }

    // ---- 5. B1 overflowed the list (a narrow value range): every wavefront
    // takes part in a radix select over the registers for the exact rank-`rem`
    // key inside B1, on keys relative to B1's smallest key (its span decides
    // the digits, so a narrow range spreads over the bins; none for a tie
    // group)
    auto for_b1 = [&](auto f) {
#pragma unroll
        for (int i = 0; i < V; ++i)
            if (live(i) && key[i] && bin_at(i) == b1) f(key[i], pos(i));
    };
    uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
    for_b1([&](uint32_t key, int32_t) {
        kmn = key < kmn ? key : kmn;
        kmx = key > kmx ? key : kmx;
    });
    for (int b = tid; b < kBins; b += T) hist0[b] = 0;       // last read before the step-2 barrier
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
        asm volatile("" : "+v"(kmin));   // keeps key - kmin inside the loop (no 2V-register hoist)
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

    // B1 outputs: keys above kth fill [above0, k - rem), then `rem` keys
    // equal to kth fill [k - rem, k)
    const uint32_t above = (uint32_t)k - rem;
    for_b1([&](uint32_t key, int32_t p) {
        if (key > kth) {
            write(above0 + atomicAdd(&cnt[0], 1u), p);
        } else if (key == kth) {
            const uint32_t q = atomicAdd(&cnt[1], 1u);
            if (q < rem) write(above + q, p);
        }
    });
}


// ------------------------------------------------------ split-row path ----
// Rows spread over one workgroup per chunk of 4096 logits, in four
// dispatches over a caller workspace (the dispatch boundaries make each
// step's global writes visible to the next; no fences or waits in kernels):
//   zero:   the row's 2048-bin histogram and counters;
//   hist:   each chunk adds the histogram of its keys' top 11 bits (digit 1);
//   select: each chunk finds the bin B1 of the k-th largest from the row's
//           histogram, writes its logits above B1 at slots taken with one
//           global atomic per workgroup and appends its B1 logits (key and
//           index) to the row's list;
//   finish: one workgroup per row finds the next 11 bits (digit 2) and then
//           the last 10 from LDS histograms over the list, and writes the
//           list's selected entries.  When B1 overflowed the list (its
//           capacity is max(4096, cols / 16)), the finish streams the row
//           instead.
// The select step adds nothing to a global digit-2 histogram: those device
// atomics, contended by the row's chunks, cost it 2.1 of 15.1 us, more than
// the finish's extra pass over the list.
constexpr int kSplitT = 256;
constexpr int kSplitV = 16;
constexpr int kSplitChunk = kSplitT * kSplitV;
constexpr int kStateWords = kBins + 8;        // digit-1 histogram, counters: placed, listed

struct SplitArgs {
    const float* logits;
    int64_t row_stride;
    const int32_t* lengths;
    int64_t cols;
    int32_t k;
    int32_t chunks;        // per row: ceil(cols / kSplitChunk)
    int32_t* out;          // [rows, k]
    uint32_t* state;       // [rows, kStateWords]
    uint32_t* list_key;    // [rows, list_stride]
    int32_t* list_pos;     // [rows, list_stride]
    int64_t list_stride;   // list capacity per row
};

// List capacity per row: B1 usually holds a few percent of a row; a larger B1
// (heavy ties, a narrow value range) is finished by streaming the row.
__host__ __device__ constexpr int64_t split_list_cap(int64_t cols) {
    return ((cols / 16 > 4096 ? cols / 16 : 4096) + 3) / 4 * 4;
}

__device__ __forceinline__ int64_t split_row_length(const SplitArgs& a, int64_t r) {
    if (!a.lengths) return a.cols;
    const int64_t l = a.lengths[r];
    return l < 0 ? 0 : (l < a.cols ? l : a.cols);
}

// Keys of logits [0, n) of a chunk; slot i of thread t is logit
// 4 * (t + (i / 4) * kSplitT) + i % 4; key 0 marks a slot past n.
__device__ __forceinline__ void load_chunk_keys(const float* src, int32_t n, uint32_t (&key)[kSplitV]) {
    const float4* s4 = reinterpret_cast<const float4*>(src);
#pragma unroll
    for (int j = 0; j < kSplitV / 4; ++j) {
        const int32_t c = threadIdx.x + j * kSplitT;
        float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
        if (4 * c < n) f = s4[c];
        key[4 * j + 0] = 4 * c + 0 < n ? order_key(f.x) : 0u;
        key[4 * j + 1] = 4 * c + 1 < n ? order_key(f.y) : 0u;
        key[4 * j + 2] = 4 * c + 2 < n ? order_key(f.z) : 0u;
        key[4 * j + 3] = 4 * c + 3 < n ? order_key(f.w) : 0u;
    }
}

__device__ __forceinline__ int32_t chunk_pos(int i) {
    return 4 * (threadIdx.x + (i >> 2) * kSplitT) + (i & 3);
}

__global__ __launch_bounds__(kSplitT) void topk_split_zero_kernel(SplitArgs a) {
    uint32_t* st = a.state + blockIdx.x * (int64_t)kStateWords;
    for (int i = threadIdx.x; i < kStateWords; i += kSplitT) st[i] = 0;
}

// The digit-1 histogram uses the selection's chunks; chunks of 16384 logits
// (1024 threads) measured slower: fewer workgroups to overlap, more LDS
// contention in each.
__global__ __launch_bounds__(kSplitT) void topk_split_hist_kernel(SplitArgs a) {
    __shared__ uint32_t hist[kBins];
    const int64_t r = blockIdx.x / a.chunks;
    const int64_t base = (blockIdx.x - r * a.chunks) * (int64_t)kSplitChunk;
    const int64_t lr = split_row_length(a, r);
    if (lr <= a.k || base >= lr) return;
    const int32_t n = (int32_t)(lr - base < kSplitChunk ? lr - base : kSplitChunk);
    for (int b = threadIdx.x; b < kBins; b += kSplitT) hist[b] = 0;
    uint32_t key[kSplitV];
    load_chunk_keys(a.logits + r * a.row_stride + base, n, key);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kSplitV; ++i)
        if (key[i]) atomicAdd(&hist[key[i] >> 21], 1u);
    __syncthreads();
    uint32_t* g1 = a.state + r * kStateWords;
    for (int b = threadIdx.x; b < kBins; b += kSplitT) {
        const uint32_t c = hist[b];
        if (c) atomicAdd(&g1[b], c);
    }
}

// Eight waves per SIMD: all chunk workgroups of 64 rows of 131072 are
// resident at once (the register budget otherwise leaves seven).
__global__ __launch_bounds__(kSplitT, 8) void topk_split_select_kernel(SplitArgs a) {
    constexpr int T = kSplitT;
    constexpr int W = T / 64;
    __shared__ uint32_t part[W];
    __shared__ uint32_t sel[2];
    __shared__ uint32_t shared_base[2];

    const int tid = threadIdx.x;
    const int32_t k = a.k;
    const int64_t r = blockIdx.x / a.chunks;
    const int64_t j = blockIdx.x - r * a.chunks;
    const int64_t lr = split_row_length(a, r);
    int32_t* dst = a.out + r * (int64_t)k;
    if (lr <= k) {
        if (j == 0)
            for (int64_t i = tid; i < k; i += T) dst[i] = i < lr ? (int32_t)i : -1;
        return;
    }
    const int64_t base = j * kSplitChunk;
    if (base >= lr) return;
    const int32_t n = (int32_t)(lr - base < kSplitChunk ? lr - base : kSplitChunk);
    uint32_t* g1 = a.state + r * kStateWords;
    uint32_t* ctrl = g1 + kBins;
    uint32_t* lk = a.list_key + r * a.list_stride;
    int32_t* lp = a.list_pos + r * a.list_stride;

    if (tid == 0) {
        sel[0] = 0;
        sel[1] = 1;
    }
    uint32_t key[kSplitV];
    load_chunk_keys(a.logits + r * a.row_stride + base, n, key);
    uint32_t h1[kBins / T];
    load_bins<T>(g1, h1);

    // B1 and the rank in it, from the row's digit-1 histogram
    uint32_t b1, rem;
    select_bin_regs<T>(h1, (uint32_t)k, part, sel, b1, rem);
    b1 = min(b1, (uint32_t)(kBins - 1));

    uint32_t n_gt = 0, n_eq = 0;
#pragma unroll
    for (int i = 0; i < kSplitV; ++i) {
        if (key[i]) {
            const uint32_t d1 = key[i] >> 21;
            n_gt += d1 > b1 ? 1u : 0u;
            n_eq += d1 == b1 ? 1u : 0u;
        }
    }
    const uint32_t packed = n_gt | (n_eq << 16);             // chunk totals < 2^13
    const uint32_t excl = block_inclusive_sum<T>(packed, part) - packed;
    if (tid == 0) {
        uint32_t tot = 0;
#pragma unroll
        for (int w = 0; w < W; ++w) tot += part[w];
        // both running counts in one 64-bit word: placed (low), listed (high)
        const unsigned long long old = atomicAdd(reinterpret_cast<unsigned long long*>(ctrl),
                                                 (unsigned long long)(tot & 0xFFFFu) |
                                                     ((unsigned long long)(tot >> 16) << 32));
        shared_base[0] = (uint32_t)old;
        shared_base[1] = (uint32_t)(old >> 32);
    }
    __syncthreads();
    uint32_t og = shared_base[0] + (excl & 0xFFFFu);
    uint32_t oe = shared_base[1] + (excl >> 16);
#pragma unroll
    for (int i = 0; i < kSplitV; ++i) {
        if (key[i]) {
            const uint32_t d1 = key[i] >> 21;
            if (d1 > b1) {
                if (og < (uint32_t)k) dst[og] = (int32_t)(base + chunk_pos(i));
                ++og;
            } else if (d1 == b1) {
                if (oe < (uint64_t)a.list_stride) {
                    lk[oe] = key[i];
                    lp[oe] = (int32_t)(base + chunk_pos(i));
                }
                ++oe;
            }
        }
    }
}

// One workgroup per row: rank `rem` among the n1 listed B1 logits, from the
// digit-2 histogram and an LDS histogram of the last 10 bits.
constexpr int kFinishT = 1024;

__global__ __launch_bounds__(kFinishT) void topk_split_finish_kernel(SplitArgs a) {
    constexpr int T = kFinishT;
    constexpr int W = T / 64;
    __shared__ __align__(16) uint32_t hist2[kBins];
    __shared__ __align__(16) uint32_t hist3[1024];
    __shared__ uint32_t part[W];
    __shared__ uint32_t sel[2];
    __shared__ uint32_t cnt[2];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int32_t k = a.k;
    const int64_t r = blockIdx.x;
    if (split_row_length(a, r) <= k) return;
    int32_t* dst = a.out + r * (int64_t)k;
    const uint32_t* g1 = a.state + r * kStateWords;
    const uint32_t* lk = a.list_key + r * a.list_stride;
    const int32_t* lp = a.list_pos + r * a.list_stride;

    {
        const uint4 z = make_uint4(0u, 0u, 0u, 0u);
        for (int b = 4 * tid; b < kBins; b += 4 * T) *reinterpret_cast<uint4*>(&hist2[b]) = z;
        for (int b = 4 * tid; b < 1024; b += 4 * T) *reinterpret_cast<uint4*>(&hist3[b]) = z;
    }
    if (tid < 2) cnt[tid] = 0;
    if (tid == 0) {
        sel[0] = 0;
        sel[1] = 1;
    }
    uint32_t h1[kBins / T];
    load_bins<T>(g1, h1);
    uint32_t b1, rem;
    select_bin_regs<T>(h1, (uint32_t)k, part, sel, b1, rem);
    b1 = min(b1, (uint32_t)(kBins - 1));
    const uint32_t n1 = g1[b1];                              // every B1 logit of the row
    const bool listed = n1 <= (uint64_t)a.list_stride;
    const uint32_t above1 = (uint32_t)k - rem;
    // The B1 logits: from the list, or, when it overflowed, by streaming the row.
    const int64_t lr = split_row_length(a, r);
    const float4* row4 = reinterpret_cast<const float4*>(a.logits + r * a.row_stride);
    // A list of up to kFinishRegs entries per thread is read into registers
    // once (all its loads in flight together) for the three passes below.
    constexpr int kFinishRegs = 8;
    const bool in_regs = listed && n1 <= (uint32_t)(kFinishRegs * T);
    uint32_t rk[kFinishRegs];
    int32_t rp[kFinishRegs];
    if (in_regs) {
#pragma unroll
        for (int i = 0; i < kFinishRegs; ++i) {
            const uint32_t c = tid + i * T;
            rk[i] = c < n1 ? lk[c] : 0u;
            rp[i] = c < n1 ? lp[c] : 0;
        }
    }
    auto for_b1 = [&](auto f) {
        if (in_regs) {
#pragma unroll
            for (int i = 0; i < kFinishRegs; ++i)
                if ((uint32_t)(tid + i * T) < n1) f(rk[i], rp[i]);
        } else if (listed) {
            for (uint32_t c = tid; c < n1; c += T) f(lk[c], lp[c]);
        } else {
            for (int64_t c = tid; 4 * c < lr; c += T) {
                const float4 v = row4[c];
                const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const uint32_t kk = order_key(e[m]);
                    if (4 * c + m < lr && (kk >> 21) == b1) f(kk, (int32_t)(4 * c + m));
                }
            }
        }
    };
    // digit 2 (bits 20..10) and digit 3 (bits 9..0) of the rank-rem key; each
    // digit is chosen by wavefront 0 and published behind one barrier (bin
    // indices masked so that they stay inside the histograms)
    for_b1([&](uint32_t kk, int32_t) { atomicAdd(&hist2[(kk >> 10) & (kBins - 1)], 1u); });
    __syncthreads();                                         // also: every thread has read sel
    if (wave == 0) {
        uint32_t d, q;
        wave_select<kBins>(hist2, rem, d, q);
        if (lane == 0) {
            sel[0] = d;
            sel[1] = q;
        }
    }
    __syncthreads();
    const uint32_t b2 = sel[0], rem2 = sel[1];
    for_b1([&](uint32_t kk, int32_t) {
        if (((kk >> 10) & (kBins - 1)) == b2) atomicAdd(&hist3[kk & 1023u], 1u);
    });
    __syncthreads();                                         // also: every thread has read sel
    if (wave == 0) {
        uint32_t d, q;
        wave_select<1024>(hist3, rem2, d, q);
        if (lane == 0) {
            sel[0] = d;
            sel[1] = q;
        }
    }
    __syncthreads();
    const uint32_t b3 = sel[0], rem3 = sel[1];
    const uint32_t kth = (b1 << 21) | (b2 << 10) | (b3 & 1023u);
    const uint32_t above = (uint32_t)k - rem3;
    for_b1([&](uint32_t kk, int32_t pos) {
        if (kk > kth) {
            const uint32_t slot = above1 + atomicAdd(&cnt[0], 1u);
            if (slot < (uint32_t)k) dst[slot] = pos;
        } else if (kk == kth) {
            const uint32_t q = atomicAdd(&cnt[1], 1u);
            if (q < rem3) dst[above + q] = pos;
        }
    });
}

}  // namespace

// Kernel choice for a call; topk_workspace_bytes and launch_topk share it.
struct TopkPlan {
    int split;         // 0: one row kernel launch, 1: the split-row path
    int variant;       // row kernel shape 0..3
    int64_t chunks;    // split: chunks of kSplitChunk per row
    int64_t ws_bytes;  // split: workspace bytes
};

// Workgroup shapes (threads, logits per thread, waves per SIMD to leave room
// for) of the row kernel for rows of up to 4096, 8192, 16384 and 32768 logits.
// Capping the 512-thread shapes at 64 VGPRs (8 waves per SIMD) measured 4 %
// faster on the causal prefill; the 1024-thread shapes spill under that cap
// and run slower.  For rows of up to 4096 logits 512 x 8 beat 256 x 16 (which
// LDS holds to six workgroups per compute unit): 18.9 against 23.5 us for
// 4096 causal rows, equal on 64 rows.
#define DSAIDX_TOPK_R4K 512, 8, 8
#define DSAIDX_TOPK_R8K 512, 16, 8
#define DSAIDX_TOPK_R16K 1024, 16, 1
#define DSAIDX_TOPK_R32K 1024, 32, 1
constexpr int64_t kRowMax = 32768;       // longest row of the row kernel
// From this many rows (several row workgroups per compute unit) the row
// kernel works for throughput: a row's loads stop at its length, and a long
// B1 list is resolved by one wavefront, which frees the compute unit for other
// rows sooner.  With fewer rows compute units idle, and it works for latency:
// the loads go out before the length is known, and every wavefront of the
// row's workgroup shares the list work.
constexpr int64_t kManyRows = 1024;

static TopkPlan plan_topk(int64_t rows, int64_t cols, int32_t) {
    TopkPlan p{0, 0, 0, 0};
    if (cols <= kRowMax) {
        p.variant = cols <= 4096 ? 0 : (cols <= 8192 ? 1 : (cols <= 16384 ? 2 : 3));
        return p;
    }
    p.split = 1;
    p.chunks = (cols + kSplitChunk - 1) / kSplitChunk;
    // the grid holds rows * chunks workgroups; that bound also keeps the
    // workspace size far inside int64
    if (rows * p.chunks >= (int64_t(1) << 31)) {
        p.ws_bytes = -1;
        return p;
    }
    p.ws_bytes = rows * (int64_t(kStateWords) * 4 + 8 * split_list_cap(cols));
    return p;
}

int64_t topk_workspace_bytes(int64_t rows, int64_t cols, int32_t k) {
    return plan_topk(rows, cols, k).ws_bytes;
}

template <int T, int V, int MINW>
static hipError_t launch_row(RowArgs& a, int64_t rows, hipStream_t stream) {
    static_assert(T * V >= 4096, "row shape");
    void* args[] = {&a};
    return hipLaunchKernel(reinterpret_cast<const void*>(&topk_row_kernel<T, V, MINW>),
                           dim3((unsigned)rows), dim3(T), args, 0, stream);
}

// A dispatch counts its work-items in 32 bits: rows are launched in batches
// whose workgroups * threads stay below 2^32 (one batch, so one or four
// dispatches, for any call of up to 4194303 rows; more only beyond that).
constexpr int64_t kMaxItems = (int64_t(1) << 32) - 1;

static hipError_t launch_rows(const RowArgs& base, int variant, int64_t rows, hipStream_t stream) {
    constexpr int kThreads[4] = {512, 512, 1024, 1024};   // DSAIDX_TOPK_R4K .. R32K
    const int64_t batch = kMaxItems / kThreads[variant];
    hipError_t e = hipSuccess;
    for (int64_t r0 = 0; r0 < rows && e == hipSuccess; r0 += batch) {
        const int64_t n = rows - r0 < batch ? rows - r0 : batch;
        RowArgs a = base;
        a.logits = base.logits + r0 * base.row_stride;
        a.lengths = base.lengths ? base.lengths + r0 : nullptr;
        a.out = base.out + r0 * base.k;
        switch (variant) {
            case 0: e = launch_row<DSAIDX_TOPK_R4K>(a, n, stream); break;
            case 1: e = launch_row<DSAIDX_TOPK_R8K>(a, n, stream); break;
            case 2: e = launch_row<DSAIDX_TOPK_R16K>(a, n, stream); break;
            default: e = launch_row<DSAIDX_TOPK_R32K>(a, n, stream); break;
        }
    }
    return e;
}

hipError_t launch_topk(const float* logits, int64_t row_stride, const int32_t* lengths,
                       int64_t rows, int64_t cols, int32_t k, int32_t* out, void* workspace,
                       hipStream_t stream) {
    const TopkPlan p = plan_topk(rows, cols, k);
    if (!p.split) {
        RowArgs a{logits, row_stride, lengths, cols, k, out, rows >= kManyRows ? 1 : 0};
        return launch_rows(a, p.variant, rows, stream);
    }
    const int64_t cap = split_list_cap(cols);
    uint32_t* state = static_cast<uint32_t*>(workspace);
    uint32_t* list_key = state + rows * kStateWords;
    int32_t* list_pos = reinterpret_cast<int32_t*>(list_key + rows * cap);
    // rows * chunks workgroups of kSplitT threads, rows of kFinishT
    int64_t batch = kMaxItems / (kSplitT * p.chunks);
    if (batch > kMaxItems / kFinishT) batch = kMaxItems / kFinishT;
    hipError_t e = hipSuccess;
    for (int64_t r0 = 0; r0 < rows && e == hipSuccess; r0 += batch) {
        const int64_t n = rows - r0 < batch ? rows - r0 : batch;
        SplitArgs sa{};
        sa.logits = logits + r0 * row_stride;
        sa.row_stride = row_stride;
        sa.lengths = lengths ? lengths + r0 : nullptr;
        sa.cols = cols;
        sa.k = k;
        sa.chunks = (int32_t)p.chunks;
        sa.out = out + r0 * k;
        sa.state = state + r0 * kStateWords;
        sa.list_key = list_key + r0 * cap;
        sa.list_pos = list_pos + r0 * cap;
        sa.list_stride = cap;
        void* args[] = {&sa};
        const dim3 grid((unsigned)(n * p.chunks));
        e = hipLaunchKernel(reinterpret_cast<const void*>(&topk_split_zero_kernel),
                            dim3((unsigned)n), dim3(kSplitT), args, 0, stream);
        if (e == hipSuccess)
            e = hipLaunchKernel(reinterpret_cast<const void*>(&topk_split_hist_kernel), grid,
                                dim3(kSplitT), args, 0, stream);
        if (e == hipSuccess)
            e = hipLaunchKernel(reinterpret_cast<const void*>(&topk_split_select_kernel), grid,
                                dim3(kSplitT), args, 0, stream);
        if (e == hipSuccess)
            e = hipLaunchKernel(reinterpret_cast<const void*>(&topk_split_finish_kernel),
                                dim3((unsigned)n), dim3(kFinishT), args, 0, stream);
    }
    return e;
}

// ------------------------------------------- allocation-free workspace ----
// The workspace of dsaidx_topk_per_row_noalloc: a file-scope device array,
// part of this code object, so each GPU the library runs on holds its own
// copy until the process ends.  Host code never uses the array's name as an
// address (on the host it is only a stand-in for the symbol): the device
// address comes from hipGetSymbolAddress, called once per device with that
// device current, and is kept in a per-device table.
static __device__ __align__(256) unsigned char scratch[kTopkScratchBytes];

hipError_t topk_scratch(int device, void** ptr) {
    static std::atomic<void*> table[kTopkScratchDevices];
    if (device < 0 || device >= kTopkScratchDevices) return hipErrorInvalidDevice;
    void* p = table[device].load(std::memory_order_acquire);
    if (!p) {
        // the caller made `device` current; concurrent first calls on one
        // device look up the same address
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        table[device].store(p, std::memory_order_release);
    }
    *ptr = p;
    return hipSuccess;
}

}  // namespace dsaidx
