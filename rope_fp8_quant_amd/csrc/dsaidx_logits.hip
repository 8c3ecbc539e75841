// gfx950 kernel for the index logits: the consumer of the prepared query
// (fp8 codes and folded head gates) and of the index-K cache, between the
// indexer prep and the top-k ([vllm-47335] = vLLM PR 47335 "Enable fused
// indexer-Q RoPE+quant kernel", section Kernel-level evidence, where the fp8
// paged MQA-logits launch sits between the two).  The pages name the step but
// do not write out its arithmetic; the reading taken is the one under which
// folding the per-head query scale into the gate is exact (a ReLU on each
// head's dot, which commutes with a positive factor, then a gate-weighted sum
// over the heads):
//
//   logit[t][s] = k_scale(slot) * sum_h w[t][h] * max(0, q[t][h][:] . k[slot][:])
//
// The dots are one dense contraction over 128 fp8 codes, so they run on the
// matrix cores: v_mfma_f32_16x16x128_f8f6f4 with both operands E4M3 computes
// a 16 (heads) x 16 (keys) block of dots in one instruction.  Products of two
// E4M3 values are exact in fp32; the 128-term sums and the head sum are fp32.
//
// Work: a workgroup of 4 wavefronts takes 8 query tokens (2 per wavefront,
// their q rows and gates held in registers for the whole call) and one chunk
// of keys.  Keys are staged through LDS 64 at a time (double-buffered, one
// barrier per stage), so each 16-key block read from L2 feeds 8 tokens x 4
// head blocks of MFMAs.  Per block: ReLU and gate on the 4 results of each
// lane, a sum over the lane groups (two cross-lane exchanges), the key scale
// and a store by 16 lanes.
#include "dsaidx_internal.h"

namespace dsaidx {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kLgThreads = 256;                   // 4 wavefronts
constexpr int kLgTokensPerWave = kLogitsTokensPerBlock / 4;
constexpr int kLgStage = kLogitsStageKeys;        // keys per LDS stage
constexpr int kLgRowPitch = 144;                  // LDS bytes per staged key row (128 + 16: no bank conflicts)
constexpr int kLgHeadBlocks = kLogitsMaxHeads / 16;

// 16 x 16 x 128 block of dots over E4M3 codes (format 0 for both operands,
// no block scales).  Lane l supplies row l % 16 of A and column l % 16 of B,
// each as the 32 bytes [32 (l / 16), 32 (l / 16) + 32) of the 128; lane l
// receives rows 4 (l / 16) + e, column l % 16, in element e.  (Which 32
// bytes a lane group carries only has to agree between A and B.)
__device__ __forceinline__ v4f dots16(v8i a, v8i b) {
    const v4f z = {0.f, 0.f, 0.f, 0.f};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ v8i load32(const uint8_t* p) {
    const uint4 a = *reinterpret_cast<const uint4*>(p);
    const uint4 b = *reinterpret_cast<const uint4*>(p + 16);
    v8i r;
    r[0] = (int)a.x; r[1] = (int)a.y; r[2] = (int)a.z; r[3] = (int)a.w;
    r[4] = (int)b.x; r[5] = (int)b.y; r[6] = (int)b.z; r[7] = (int)b.w;
    return r;
}

__device__ __forceinline__ int64_t clamp_len(const LogitsParams& p, int64_t t) {
    if (t >= p.T) return 0;
    if (!p.lengths) return p.N;
    const int64_t l = p.lengths[t];
    return l < 0 ? 0 : (l < p.N ? l : p.N);
}

__global__ __launch_bounds__(kLgThreads) void mqa_logits_kernel(LogitsParams p) {
    __shared__ __align__(16) uint8_t kbuf[2][kLgStage * kLgRowPitch];
    __shared__ float kscl[2][kLgStage];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = lane >> 4;                      // lane group: bytes [32 g, 32 g + 32)
    const int64_t tb = blockIdx.x / p.chunks;
    const int64_t key0 = (blockIdx.x - tb * p.chunks) * p.chunk;
    const int64_t t_first = tb * kLogitsTokensPerBlock;

    // keys past every token's length are skipped (the same for the workgroup)
    int64_t kmax = 0;
#pragma unroll
    for (int i = 0; i < kLogitsTokensPerBlock; ++i) {
        const int64_t l = clamp_len(p, t_first + i);
        kmax = l > kmax ? l : kmax;
    }
    const int64_t key1 = key0 + p.chunk < p.N ? key0 + p.chunk : p.N;
    const int64_t kend = key1 < kmax ? key1 : kmax;
    if (kend <= key0) return;

    // this wavefront's tokens: q rows (A operands) and gates, zero past H or T
    int64_t tok[kLgTokensPerWave], len[kLgTokensPerWave];
    v8i A[kLgTokensPerWave][kLgHeadBlocks];
    float G[kLgTokensPerWave][kLgHeadBlocks][4];
#pragma unroll
    for (int i = 0; i < kLgTokensPerWave; ++i) {
        const int64_t t = t_first + wave * kLgTokensPerWave + i;
        tok[i] = t;
        len[i] = clamp_len(p, t);
#pragma unroll
        for (int hb = 0; hb < kLgHeadBlocks; ++hb) {
            const int h = hb * 16 + (lane & 15);
            A[i][hb] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
            if (t < p.T && h < p.H) A[i][hb] = load32(p.q + ((t * p.H + h) * 128 + 32 * g));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int hh = hb * 16 + 4 * g + e;
                G[i][hb][e] = (t < p.T && hh < p.H) ? p.w[t * p.H + hh] : 0.f;
            }
        }
    }

    // stage loader: thread tid brings key tid / 4 of a stage, bytes
    // [32 (tid % 4), +32) as four 8-byte loads, and lanes 0..63 the scales;
    // a key past kend or with a slot outside the cache is all zeros
    const int sk = tid >> 2, sp = tid & 3;
    uint2 sreg[4];
    float sscale = 0.f;
    auto fetch = [&](int64_t s0) {
        const int64_t s = s0 + sk;
        int64_t slot = -1;
        if (s < kend) slot = p.key_slots ? (int64_t)p.key_slots[s] : s;
        const bool ok = slot >= 0 && slot < p.S;
        const uint8_t* row = nullptr;
        if (ok) {
            if (p.page_size) {
                const int64_t pg = slot / p.page_size, o = slot - pg * p.page_size;
                row = p.k_cache + pg * p.page_size * 132 + o * 128;
            } else {
                row = p.k_cache + slot * p.k_row_stride;
            }
        }
#pragma unroll
        for (int m = 0; m < 4; ++m)
            sreg[m] = ok ? *reinterpret_cast<const uint2*>(row + 32 * sp + 8 * m) : make_uint2(0u, 0u);
        if (tid < kLgStage) {
            const int64_t s2 = s0 + tid;
            int64_t slot2 = -1;
            if (s2 < kend) slot2 = p.key_slots ? (int64_t)p.key_slots[s2] : s2;
            sscale = 0.f;
            if (slot2 >= 0 && slot2 < p.S) {
                if (p.page_size) {
                    const int64_t pg = slot2 / p.page_size, o = slot2 - pg * p.page_size;
                    sscale = *reinterpret_cast<const float*>(p.k_cache + pg * p.page_size * 132 +
                                                             p.page_size * 128 + o * 4);
                } else {
                    sscale = p.k_scale[slot2];
                }
            }
        }
    };
    auto stash = [&](int buf) {
        uint8_t* d = &kbuf[buf][sk * kLgRowPitch + 32 * sp];
#pragma unroll
        for (int m = 0; m < 4; ++m) *reinterpret_cast<uint2*>(d + 8 * m) = sreg[m];
        if (tid < kLgStage) kscl[buf][tid] = sscale;
    };

    fetch(key0);
    int buf = 0;
#pragma unroll 1
    for (int64_t s0 = key0; s0 < kend; s0 += kLgStage, buf ^= 1) {
        stash(buf);
        __syncthreads();        // the stage is in LDS; every wavefront is done with the other buffer
        if (s0 + kLgStage < kend) fetch(s0 + kLgStage);
#pragma unroll
        for (int kb = 0; kb < kLgStage / 16; ++kb) {
            if (s0 + kb * 16 >= kend) break;
            const v8i B = load32(&kbuf[buf][(kb * 16 + (lane & 15)) * kLgRowPitch + 32 * g]);
            float acc[kLgTokensPerWave];
#pragma unroll
            for (int i = 0; i < kLgTokensPerWave; ++i) {
                acc[i] = 0.f;
#pragma unroll
                for (int hb = 0; hb < kLgHeadBlocks; ++hb) {
                    if (hb * 16 >= p.H) break;
                    const v4f c = dots16(A[i][hb], B);
                    acc[i] += G[i][hb][0] * fmaxf(c[0], 0.f) + G[i][hb][1] * fmaxf(c[1], 0.f) +
                              G[i][hb][2] * fmaxf(c[2], 0.f) + G[i][hb][3] * fmaxf(c[3], 0.f);
                }
            }
#pragma unroll
            for (int i = 0; i < kLgTokensPerWave; ++i) {
                float v = acc[i];
                v += __shfl_xor(v, 16);
                v += __shfl_xor(v, 32);
                const int64_t s = s0 + kb * 16 + (lane & 15);
                if (lane < 16 && s < kend && s < len[i])
                    p.out[tok[i] * p.out_stride + s] = v * kscl[buf][kb * 16 + lane];
            }
        }
    }
}

}  // namespace

hipError_t launch_logits(const LogitsParams& p, hipStream_t stream) {
    LogitsParams a = p;
    const int64_t tb = (p.T + kLogitsTokensPerBlock - 1) / kLogitsTokensPerBlock;
    void* args[] = {&a};
    return hipLaunchKernel(reinterpret_cast<const void*>(&mqa_logits_kernel),
                           dim3((unsigned)(tb * p.chunks)), dim3(kLgThreads), args, 0, stream);
}

}  // namespace dsaidx
