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
// Work: a workgroup takes 8 query tokens (their q rows and gates held in
// registers for the whole call) and one chunk of keys: 4 wavefronts of 2
// tokens, or, for calls whose grid is one resident round (decode), 8
// wavefronts of 1 token, which hold four wavefronts per SIMD and issue each
// block's MFMAs before the previous block's epilogue.  Keys are staged
// through LDS 128 at a time (double-buffered, one barrier per stage; each
// thread brings 32 bytes of one or two key rows), so each 16-key block read
// from L2 feeds 8 tokens x 4 head blocks of MFMAs.  Per
// block (two tokens): the 8 MFMAs of a wavefront, the next block's key
// operand read from LDS behind them, then ReLU and gate on the 4 results of
// each lane, a sum over the lane groups for both tokens together (two
// lane-swap instructions), the key scale and one store of 16 keys per token.
//
// Time on gfx950 goes to the matrix unit and the VALU in turn rather than
// side by side, and the epilogue costs two VALU operations per dot (ReLU and
// gate FMA): 64 per block and lane, as many cycles as the block's 8 MFMAs.
#include "dsaidx_internal.h"

namespace dsaidx {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kLgStage = kLogitsStageKeys;        // keys per LDS stage
constexpr int kLgRowPitch = 144;                  // LDS bytes per staged key row (128 + 16: no bank conflicts)
constexpr int kLgHeadBlocks = kLogitsMaxHeads / 16;

// Workgroup shape for TPW query tokens per wavefront: kLogitsTokensPerBlock
// tokens per workgroup, so TPW = 2 is 4 wavefronts and TPW = 1 is 8; each
// thread stages KPT key rows of a stage.  Register budgets: three wavefronts
// per SIMD for two tokens (168 VGPRs); four for one (128 VGPRs: with the
// pipelined blocks this leaves no room to read each key operand a block
// ahead, so one token reads it just before its MFMAs).
template <int TPW>
struct LgShape {
    static_assert(TPW == 1 || TPW == 2, "one or two tokens per wavefront");
    static constexpr int kWaves = kLogitsTokensPerBlock / TPW;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kKPT = kLgStage / (kThreads / 4);
    static_assert(kKPT * (kThreads / 4) == kLgStage, "stage rows per thread");
    static constexpr int kMinWaves = TPW == 2 ? 3 : 4;
    static constexpr bool kReadAhead = TPW == 2;
};

// 16 x 16 x 128 block of dots over E4M3 codes (format 0 for both operands,
// no block scales).  Lane l supplies row l % 16 of A and column l % 16 of B,
// each as the 32 bytes [32 (l / 16), 32 (l / 16) + 32) of the 128; lane l
// receives rows 4 (l / 16) + e, column l % 16, in element e.  (Which 32
// bytes a lane group carries only has to agree between A and B.)
__device__ __forceinline__ v4f dots16(v8i a, v8i b) {
    const v4f z = {0.f, 0.f, 0.f, 0.f};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 0, 0, 0);
}

// max(x, 0) in one instruction (v_med3_f32); the dots are finite.
__device__ __forceinline__ float relu(float x) { return __builtin_amdgcn_fmed3f(x, 0.f, 3.0e38f); }

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

template <int TPW>
__global__ __launch_bounds__(LgShape<TPW>::kThreads)
__attribute__((amdgpu_waves_per_eu(LgShape<TPW>::kMinWaves)))
void mqa_logits_kernel(LogitsParams p) {
    constexpr int kLgTokensPerWave = TPW;
    constexpr int TPB = kLogitsTokensPerBlock;
    __shared__ __align__(16) uint8_t kbuf[2][kLgStage * kLgRowPitch];
    __shared__ float kscl[2][kLgStage];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = lane >> 4;                      // lane group: bytes [32 g, 32 g + 32)
    // token blocks from the last: under causal lengths the longest rows go
    // first, so the short ones fill in behind them instead of trailing
    const int64_t nb = (p.T + TPB - 1) / TPB;
    // The 8 XCDs take consecutive workgroups in turn.  Chunk-major order
    // (consecutive workgroups: neighbouring token blocks of one chunk) gives
    // every XCD its share of every chunk whatever the chunk count, which
    // matters when chunks carry unequal work (causal lengths); token-major
    // order (consecutive workgroups: the chunks of one token block) keeps each
    // chunk's keys on one XCD when there are few token blocks and many chunks.
    int64_t tb, key0;
    if (p.chunk_major) {
        const int64_t ci = blockIdx.x / nb;
        tb = nb - 1 - (blockIdx.x - ci * nb);
        key0 = ci * p.chunk;
    } else {
        const int64_t bi = blockIdx.x / p.chunks;
        tb = nb - 1 - bi;
        key0 = (blockIdx.x - bi * p.chunks) * p.chunk;
    }
    const int64_t t_first = tb * TPB;

    // keys past every token's length are skipped (the same for the workgroup)
    int64_t kmax = 0;
#pragma unroll
    for (int i = 0; i < TPB; ++i) {
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
            if (p.w_vec) {
                // the lane's four gates are adjacent: one 16-byte load
                float4 gv = make_float4(0.f, 0.f, 0.f, 0.f);
                if (t < p.T && hb * 16 + 4 * g < p.H)
                    gv = *reinterpret_cast<const float4*>(p.w + t * p.H + hb * 16 + 4 * g);
                G[i][hb][0] = gv.x; G[i][hb][1] = gv.y; G[i][hb][2] = gv.z; G[i][hb][3] = gv.w;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int hh = hb * 16 + 4 * g + e;
                    G[i][hb][e] = (t < p.T && hh < p.H) ? p.w[t * p.H + hh] : 0.f;
                }
            }
        }
    }

    // stage loader: thread tid brings keys tid / 4 + 64 j (j < KPT) of a
    // stage, bytes [32 (tid % 4), +32) of each as four 8-byte loads, and the
    // thread with tid % 4 = 0 their scales; a key past kend or with a slot
    // outside the cache is all zeros.  The slot list is read one stage ahead
    // into 32-bit registers and widened only when the rows are fetched, so
    // the wavefront does not wait on it in the stage that loads it.
    const int sk = tid >> 2, sp = tid & 3;
    constexpr int KPT = LgShape<TPW>::kKPT;
    auto slot_of = [&](int64_t s, int32_t raw) -> int64_t {
        if (s >= kend) return -1;
        return p.key_slots ? (int64_t)raw : s;
    };
    uint2 sreg[KPT][4];
    float sscale[KPT];
    auto fetch = [&](int64_t s0, const int32_t (&raw)[KPT]) {
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const int64_t slot = slot_of(s0 + 64 * j + sk, raw[j]);
            const bool ok = slot >= 0 && slot < p.S;
            const uint8_t* row = nullptr;
            const float* scl = nullptr;
            if (ok) {
                if (p.page_size) {
                    const uint32_t pg = (uint32_t)(((uint64_t)slot * p.page_magic) >> p.page_shift);
                    const int64_t o = slot - (int64_t)pg * p.page_size;
                    const uint8_t* page = p.k_cache + (int64_t)pg * p.page_size * 132;
                    row = page + o * 128;
                    scl = reinterpret_cast<const float*>(page + p.page_size * 128) + o;
                } else {
                    row = p.k_cache + slot * p.k_row_stride;
                    scl = p.k_scale + slot;
                }
            }
#pragma unroll
            for (int m = 0; m < 4; ++m)
                sreg[j][m] = ok ? *reinterpret_cast<const uint2*>(row + 32 * sp + 8 * m) : make_uint2(0u, 0u);
            sscale[j] = 0.f;
            if (sp == 0) sscale[j] = ok ? *scl : 0.f;
        }
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            uint8_t* d = &kbuf[buf][(sk + 64 * j) * kLgRowPitch + 32 * sp];
#pragma unroll
            for (int m = 0; m < 4; ++m) *reinterpret_cast<uint2*>(d + 8 * m) = sreg[j][m];
            if (sp == 0) kscl[buf][sk + 64 * j] = sscale[j];
        }
    };
    auto slots_at = [&](int64_t s0, int32_t (&out)[KPT]) {
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const int64_t s = s0 + 64 * j + sk;
            out[j] = (p.key_slots && s < kend) ? p.key_slots[s] : -1;
        }
    };

    // output: after the reduction lanes 0..15 hold token 0's sums and (two
    // tokens) lanes 32..47 token 1's, for the 16 keys of a block (lane % 16);
    // key offsets from here on are relative to key0 (below the chunk size,
    // 32-bit)
    const int oi = TPW == 2 ? lane >> 5 : 0;
    const bool writer = TPW == 2 ? (lane & 16) == 0 : lane < 16;
    const int64_t otok = oi ? tok[TPW - 1] : tok[0];
    const int64_t olen = oi ? len[TPW - 1] : len[0];
    const int64_t ostop = (olen < kend ? olen : kend) - key0;
    const int lim = writer && ostop > 0 ? (int)ostop : 0;     // this lane stores keys rel < lim
    float* const obase = p.out + (otok < p.T ? otok : 0) * p.out_stride + key0;
    const int nkeys = (int)(kend - key0);

    // ReLU, gate and head sum of one block's dots, then the sum over the four
    // lane groups: with two tokens, for both at once (the 32-lane swap pairs
    // token 0's upper half with token 1's lower half), with one, of its two
    // halves; the 16-lane swap then folds the remaining pair of groups; key
    // scale and store
    auto epilogue = [&](const v4f (&C)[kLgTokensPerWave][kLgHeadBlocks], float ks, int rel) {
        float acc[kLgTokensPerWave];
#pragma unroll
        for (int i = 0; i < kLgTokensPerWave; ++i) {
            acc[i] = 0.f;
#pragma unroll
            for (int hb = 0; hb < kLgHeadBlocks; ++hb)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc[i] = __builtin_fmaf(G[i][hb][e], relu(C[i][hb][e]), acc[i]);
        }
        const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[0]),
                                                        __float_as_uint(acc[TPW - 1]), false, false);
        const float v2 = __uint_as_float(h[0]) + __uint_as_float(h[1]);
        const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(v2), __float_as_uint(v2),
                                                        false, false);
        const float v = __uint_as_float(q[0]) + __uint_as_float(q[1]);
        if (rel < lim) obase[rel] = v * ks;
    };

    int32_t slot_cur[KPT], slot_next[KPT];
    slots_at(key0, slot_cur);
    fetch(key0, slot_cur);
    slots_at(key0 + kLgStage, slot_next);
    int buf = 0;
    // One token per wavefront: each block's MFMAs are issued before the
    // previous block's epilogue (its results held over in Cp), so the matrix
    // unit works on one block while the VALU finishes the other, across the
    // stage barriers too.  Two tokens run each block's MFMAs and epilogue in
    // turn (their registers leave no room for a second set of results).
    v4f Cp[kLgTokensPerWave][kLgHeadBlocks];
    float ksp = 0.f;
    int relp = 0;
    bool havep = false;
#pragma unroll 1
    for (int r0 = 0; r0 < nkeys; r0 += kLgStage, buf ^= 1) {
        stash(buf);
        __syncthreads();        // the stage is in LDS; every wavefront is done with the other buffer
        if (r0 + kLgStage < nkeys) {
            fetch(key0 + r0 + kLgStage, slot_next);
            slots_at(key0 + r0 + 2 * kLgStage, slot_next);
        }
        // each block's key operand and scale are read from LDS one block ahead,
        // so their latency hides behind the epilogue of the block before
        constexpr bool kAhead = LgShape<TPW>::kReadAhead;
        v8i Bn = load32(&kbuf[buf][(lane & 15) * kLgRowPitch + 32 * g]);
        float ksn = kscl[buf][lane & 15];
#pragma unroll
        for (int kb = 0; kb < kLgStage / 16; ++kb) {
            if (!kAhead && kb > 0) {
                Bn = load32(&kbuf[buf][(kb * 16 + (lane & 15)) * kLgRowPitch + 32 * g]);
                ksn = kscl[buf][kb * 16 + (lane & 15)];
            }
            const v8i B = Bn;
            const float ks = ksn;
            const int rel = r0 + kb * 16 + (lane & 15);
            // heads past H have zero rows and gates and keys past kend zero
            // rows, so they add nothing
            v4f C[kLgTokensPerWave][kLgHeadBlocks];
#pragma unroll
            for (int i = 0; i < kLgTokensPerWave; ++i)
#pragma unroll
                for (int hb = 0; hb < kLgHeadBlocks; ++hb) C[i][hb] = dots16(A[i][hb], B);
            if (kAhead && kb + 1 < kLgStage / 16) {
                Bn = load32(&kbuf[buf][((kb + 1) * 16 + (lane & 15)) * kLgRowPitch + 32 * g]);
                ksn = kscl[buf][(kb + 1) * 16 + (lane & 15)];
            }
            if (TPW == 2) {
                epilogue(C, ks, rel);
            } else {
                if (kb > 0 || havep) epilogue(Cp, ksp, relp);
#pragma unroll
                for (int hb = 0; hb < kLgHeadBlocks; ++hb) Cp[0][hb] = C[0][hb];
                ksp = ks;
                relp = rel;
            }
        }
        havep = true;
    }
    if (TPW == 1 && havep) epilogue(Cp, ksp, relp);
}

}  // namespace

hipError_t launch_logits(const LogitsParams& p, hipStream_t stream) {
    LogitsParams a = p;
    const int64_t tb = (p.T + kLogitsTokensPerBlock - 1) / kLogitsTokensPerBlock;
    void* args[] = {&a};
    if (p.tokens_per_wave == 1)
        return hipLaunchKernel(reinterpret_cast<const void*>(&mqa_logits_kernel<1>),
                               dim3((unsigned)(tb * p.chunks)), dim3(LgShape<1>::kThreads), args, 0, stream);
    return hipLaunchKernel(reinterpret_cast<const void*>(&mqa_logits_kernel<2>),
                           dim3((unsigned)(tb * p.chunks)), dim3(LgShape<2>::kThreads), args, 0, stream);
}

}  // namespace dsaidx
