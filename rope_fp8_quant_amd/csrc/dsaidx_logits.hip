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
// wavefronts of 1 token.  Keys are staged through LDS 128 at a time (each
// thread brings 32 bytes of one or two key rows), so each 16-key block read
// from L2 feeds 8 tokens x 4 head blocks of MFMAs.  Two tokens per wavefront:
// double-buffered stages, one barrier per stage.  One token per wavefront:
// four wavefronts per SIMD; the workgroup's 256 keys are 16-key blocks
// spread over the whole key range, both stages go to LDS behind one barrier,
// and each wavefront then runs through its blocks on its own, stopping at its
// token's length and issuing each block's MFMAs before the previous block's
// epilogue.  Per
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
// per SIMD for two tokens (168 VGPRs); four for one (128 VGPRs, of which it
// uses about 100; one token reads each key operand just before its MFMAs,
// since reading it a block ahead measured no faster there).
template <int TPW>
struct LgShape {
    static_assert(TPW == 1 || TPW == 2, "one or two tokens per wavefront");
    static constexpr int kWaves = kLogitsTokensPerBlock / TPW;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kKPT = kLgStage / (kThreads / 4);
    static_assert(kKPT * (kThreads / 4) == kLgStage, "stage rows per thread");
    static constexpr int kMinWaves = TPW == 2 ? 3 : 4;
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

// All-ones when ok, else zero: masks a value loaded from a clamped address,
// so that no load sits under a per-lane branch.  (Under a divergent branch the
// compiler must wait for the load before the other side writes the same
// register, which serialises the loads of the set-up.)
__device__ __forceinline__ int lane_mask(bool ok) { return ok ? -1 : 0; }
__device__ __forceinline__ float masked(float v, int m) {
    return __int_as_float(__float_as_int(v) & m);
}

// SLOTS: the keys come from a slot list (else key s is slot s); a template
// parameter rather than a branch, which would make the set-up wait for the
// list's first entries inside it.
template <int TPW, bool SLOTS>
__global__ __launch_bounds__(LgShape<TPW>::kThreads)
__attribute__((amdgpu_waves_per_eu(LgShape<TPW>::kMinWaves)))
void mqa_logits_kernel(LogitsParams p) {
    constexpr int kLgTokensPerWave = TPW;
    constexpr int TPB = kLogitsTokensPerBlock;
    __shared__ __align__(16) uint8_t kbuf[2][kLgStage * kLgRowPitch];
    __shared__ float kscl[2][kLgStage];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4;                      // lane group: bytes [32 g, 32 g + 32)
    // Index arithmetic is 32-bit (the host bounds T, N, the grid and the chunk
    // below 2^31) and every wavefront repeats it, so it is kept short: the
    // SIMD's four wavefronts share one scalar issue slot, and a long set-up
    // holds back the second workgroup on the compute unit.
    //
    // token blocks from the last: under causal lengths the longest rows go
    // first, so the short ones fill in behind them instead of trailing.
    // The 8 XCDs take consecutive workgroups in turn.  Chunk-major order
    // (consecutive workgroups: neighbouring token blocks of one chunk) gives
    // every XCD its share of every chunk whatever the chunk count, which
    // matters when chunks carry unequal work (causal lengths); token-major
    // order (consecutive workgroups: the chunks of one token block) keeps each
    // chunk's keys on one XCD when there are few token blocks and many chunks.
    const uint32_t bx = blockIdx.x;
    const uint32_t qd = (uint32_t)(((uint64_t)bx * p.grid_magic) >> p.grid_shift);
    int tb, ci;    // token block, chunk
    if (p.chunk_major) {
        tb = p.blocks - 1 - (int)(bx - qd * (uint32_t)p.blocks);
        ci = (int)qd;
    } else {
        tb = p.blocks - 1 - (int)qd;
        ci = (int)(bx - qd * (uint32_t)p.chunks);
    }
    const int t_first = tb * TPB;

    // The workgroup's keys.  Two tokens per wavefront: chunk ci's contiguous
    // keys [key0, key0 + chunk).  One token per wavefront (a call of one
    // resident round): the 16 blocks of 16 keys ci, ci + chunks, ci + 2 chunks,
    // ... ci + 15 chunks, so that every workgroup holds keys from the whole
    // range; under ragged lengths each wavefront skips the blocks at or past
    // its own token's length, and no compute unit is left with only the first
    // keys, which every token still needs.  The host takes this shape only
    // when chunks <= 512 and 256 chunks >= N, so those blocks cover every key
    // and N <= 2^17: the key arithmetic stays far inside 32 bits.
    constexpr bool kStrided = TPW == 1;
    const int key0 = kStrided ? 0 : ci * p.chunk;
    // key of row r (0 <= r < kLgStage) of the workgroup's stage st
    auto key_of = [&](int st, int r) -> int {
        if constexpr (kStrided)
            return 16 * (ci + p.chunks * (st * (kLgStage / 16) + (r >> 4))) + (r & 15);
        else
            return key0 + st * kLgStage + r;
    };

    constexpr int KPT = LgShape<TPW>::kKPT;
    const int sk = tid >> 2, sp = tid & 3;
    const int key1 = kStrided || p.N - key0 < p.chunk ? p.N : key0 + p.chunk;

    // Set-up loads.  Each reads a clamped, valid address (the host checks T,
    // N, S >= 1 and 1 <= H <= 64) and is masked where it is used: a load
    // whose result is changed under a branch, even a uniform one, makes the
    // compiler wait for it inside the branch.  Loads retire in issue order, so
    // they go out in the order they are needed: the block's lengths, the slot
    // lists of the first two stages (the key rows depend on them), then the
    // gates and query rows (first needed by the first MFMA).

    // lane l reads the length of token t_first + l % 8
    const int tl = t_first + (lane & (TPB - 1));
    int32_t lraw = 0;
    if (p.lengths) lraw = p.lengths[tl < p.T ? tl : p.T - 1];
    // valid keys of token t_first + i (i wavefront-uniform)
    auto length_of = [&](int i) -> int {
        const int r = __builtin_amdgcn_readlane(lraw, i);
        const int l = !p.lengths ? p.N : min(max(r, 0), p.N);
        return t_first + i < p.T ? l : 0;
    };
    int kend = key1;      // lowered to the longest token's length below
    // keys past every token's length are skipped (the same for the workgroup)
    auto chunk_end = [&]() {
        int kmax = 0;
#pragma unroll
        for (int i = 0; i < TPB; ++i) kmax = max(kmax, length_of(i));
        return min(key1, kmax);
    };
    // slot-list entries of stage st, as read (slot_ok drops the entries at or
    // past kend when the rows are fetched)
    auto slots_at = [&](int st, int32_t (&out)[KPT]) {
        if constexpr (!SLOTS) return;
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const int s = key_of(st, 64 * j + sk);
            out[j] = p.key_slots[min(s, p.N - 1)];
        }
    };

    // Calls of one resident round (one token per wavefront) issue every load
    // before the lengths arrive; larger calls first drop the workgroups with
    // nothing to do (half of them under causal lengths) and load after.
    constexpr bool kEarlyLoads = TPW == 1;
    if constexpr (!kEarlyLoads) {
        kend = chunk_end();
        if (kend <= key_of(0, 0)) return;
    }
    int32_t slot_cur[KPT], slot_next[KPT];
    slots_at(0, slot_cur);
    slots_at(1, slot_next);
    __builtin_amdgcn_sched_barrier(0);   // keep the slot loads ahead of the query rows

    // this wavefront's tokens: gates (zero past H or T), then q rows (A
    // operands).  A lane past H reads row H - 1 and one past T token T - 1:
    // the first meets a zero gate (a finite dot times zero adds nothing, and a
    // NaN code in that row already makes head H - 1's own dot NaN), the second
    // writes nothing, so the rows need no mask (which would make the set-up
    // wait for them before fetching the keys).
    const int t_wave = t_first + wave * kLgTokensPerWave;
    v8i A[kLgTokensPerWave][kLgHeadBlocks];
    float G[kLgTokensPerWave][kLgHeadBlocks][4];
#pragma unroll
    for (int i = 0; i < kLgTokensPerWave; ++i) {
        const int t = t_wave + i;
        const float* wrow = p.w + (int64_t)min(t, p.T - 1) * p.H;
#pragma unroll
        for (int hb = 0; hb < kLgHeadBlocks; ++hb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int hh = hb * 16 + 4 * g + e;
                G[i][hb][e] = masked(wrow[min(hh, p.H - 1)], lane_mask(t < p.T && hh < p.H));
            }
    }
#pragma unroll
    for (int i = 0; i < kLgTokensPerWave; ++i) {
        const uint8_t* qrow = p.q + (int64_t)min(t_wave + i, p.T - 1) * p.H * 128 + 32 * g;
#pragma unroll
        for (int hb = 0; hb < kLgHeadBlocks; ++hb)
            A[i][hb] = load32(qrow + min(hb * 16 + (lane & 15), p.H - 1) * 128);
    }
    if constexpr (kEarlyLoads) {
        // The loads above stay above the exit: no memory access may move
        // across this (empty) statement, so the compiler cannot sink them past
        // the branch into the only path that uses them; and as it redefines
        // the lengths register, their uses (and the wait for them) come after
        // every load of the set-up has been issued.
        asm volatile("" : "+v"(lraw) :: "memory");
        kend = chunk_end();
        if (kend <= key_of(0, 0)) return;
    }

    // stage loader: thread tid brings keys tid / 4 + 64 j (j < KPT) of a
    // stage, bytes [32 (tid % 4), +32) of each as four 8-byte loads, and its
    // scale (stored by the thread with tid % 4 = 0); a key past kend or with a
    // slot outside the cache reads slot 0 and is zeroed when stashed (masking
    // at the fetch would make the wavefront wait for the rows there).  The
    // slot list is read one stage ahead into 32-bit registers.
    auto slot_ok = [&](int s, int32_t raw) {
        return s < kend && (!SLOTS || (uint32_t)raw < p.S);
    };
    struct StageRegs {
        uint2 r[KPT][4];
        float sc[KPT];
        int m[KPT];
    };
    auto fetch = [&](StageRegs& R, int st, const int32_t (&raw)[KPT]) {
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const int s = key_of(st, 64 * j + sk);
            const bool ok = slot_ok(s, raw[j]);
            const uint32_t sl = ok ? (SLOTS ? (uint32_t)raw[j] : (uint32_t)s) : 0u;
            const uint8_t* row;
            const float* scl;
            if (p.page_size) {
                const uint32_t pg = (uint32_t)(((uint64_t)sl * p.page_magic) >> p.page_shift);
                const uint32_t o = sl - pg * (uint32_t)p.page_size;
                const uint8_t* page = p.k_cache + (uint64_t)pg * ((uint32_t)p.page_size * 132u);
                row = page + o * 128u;
                scl = reinterpret_cast<const float*>(page + (uint32_t)p.page_size * 128u) + o;
            } else {
                row = p.k_cache + (uint64_t)sl * (uint64_t)p.k_row_stride;
                scl = p.k_scale + sl;
            }
            R.m[j] = lane_mask(ok);
#pragma unroll
            for (int q = 0; q < 4; ++q) R.r[j][q] = *reinterpret_cast<const uint2*>(row + 32 * sp + 8 * q);
            R.sc[j] = *scl;
        }
    };
    auto stash = [&](const StageRegs& R, int buf) {
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            uint8_t* d = &kbuf[buf][(sk + 64 * j) * kLgRowPitch + 32 * sp];
            const uint32_t m = (uint32_t)R.m[j];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<uint2*>(d + 8 * q) = make_uint2(R.r[j][q].x & m, R.r[j][q].y & m);
            if (sp == 0) kscl[buf][sk + 64 * j] = masked(R.sc[j], R.m[j]);
        }
    };

    // output: after the reduction lanes 0..15 hold token 0's sums and (two
    // tokens) lanes 32..47 token 1's, for the 16 keys of a block (lane % 16);
    // key offsets from here on are relative to key0 (32-bit)
    const int oi = TPW == 2 ? lane >> 5 : 0;
    const bool writer = TPW == 2 ? (lane & 16) == 0 : lane < 16;
    const int otok = t_wave + oi;
    const int olen = oi ? length_of(wave * kLgTokensPerWave + TPW - 1) : length_of(wave * kLgTokensPerWave);
    float* const obase = p.out + (int64_t)min(otok, p.T - 1) * p.out_stride + key0;
    const int wlen = min(olen, kend);       // one token per wavefront: its keys end here
    const int ostop = wlen - key0;
    const int lim = writer && ostop > 0 ? ostop : 0;     // this lane stores keys rel < lim

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

    int buf = 0;
    // One token per wavefront: each block's MFMAs are issued before the
    // previous block's epilogue (its results held over in Cp).  Two tokens
    // run each block's MFMAs and epilogue in turn (their registers leave no
    // room for a second set of results).
    v4f Cp[kLgTokensPerWave][kLgHeadBlocks];
    float ksp = 0.f;
    int relp = 0;
    bool havep = false;
    // heads past H have zero rows and gates and keys past kend zero rows, so
    // they add nothing
    auto block_dots = [&](v4f (&C)[kLgTokensPerWave][kLgHeadBlocks], const v8i& B) {
#pragma unroll
        for (int i = 0; i < kLgTokensPerWave; ++i)
#pragma unroll
            for (int hb = 0; hb < kLgHeadBlocks; ++hb) C[i][hb] = dots16(A[i][hb], B);
    };
    if constexpr (TPW == 2) {
        StageRegs R;
        fetch(R, 0, slot_cur);
#pragma unroll 1
        for (int st = 0; key_of(st, 0) < kend; ++st, buf ^= 1) {
            stash(R, buf);
            __syncthreads();        // the stage is in LDS; every wavefront is done with the other buffer
            if (key_of(st + 1, 0) < kend) {
                fetch(R, st + 1, slot_next);
                slots_at(st + 2, slot_next);
            }
            // each block's key operand and scale are read from LDS one block
            // ahead, so their latency hides behind the epilogue of the block
            // before
            v8i Bn = load32(&kbuf[buf][(lane & 15) * kLgRowPitch + 32 * g]);
            float ksn = kscl[buf][lane & 15];
#pragma unroll
            for (int kb = 0; kb < kLgStage / 16; ++kb) {
                const v8i B = Bn;
                const float ks = ksn;
                v4f C[kLgTokensPerWave][kLgHeadBlocks];
                block_dots(C, B);
                if (kb + 1 < kLgStage / 16) {
                    Bn = load32(&kbuf[buf][((kb + 1) * 16 + (lane & 15)) * kLgRowPitch + 32 * g]);
                    ksn = kscl[buf][(kb + 1) * 16 + (lane & 15)];
                }
                epilogue(C, ks, st * kLgStage + kb * 16 + (lane & 15));
            }
        }
    } else {
        // One resident round: the workgroup's two stages (its chunk of 256
        // keys) are staged together behind one barrier, after which each
        // wavefront runs through its own blocks with no further barrier and
        // stops at its token's length.
        {
            StageRegs R0, R1;
            fetch(R0, 0, slot_cur);
            fetch(R1, 1, slot_next);
            stash(R0, 0);
            stash(R1, 1);
        }
        __syncthreads();
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            if (key_of(st, kLgStage - 16) < wlen) {
#pragma unroll
                for (int kb = 0; kb < kLgStage / 16; ++kb) {
                    const v8i B = load32(&kbuf[st][(kb * 16 + (lane & 15)) * kLgRowPitch + 32 * g]);
                    const float ks = kscl[st][kb * 16 + (lane & 15)];
                    v4f C[kLgTokensPerWave][kLgHeadBlocks];
                    block_dots(C, B);
                    if (kb > 0 || havep) epilogue(Cp, ksp, relp);
#pragma unroll
                    for (int hb = 0; hb < kLgHeadBlocks; ++hb) Cp[0][hb] = C[0][hb];
                    ksp = ks;
                    relp = key_of(st, kb * 16) + (lane & 15);
                }
                havep = true;
            } else if (key_of(st, 0) < wlen) {
                if (havep) epilogue(Cp, ksp, relp);
                havep = false;
#pragma unroll 1
                for (int kb = 0; kb < kLgStage / 16 && key_of(st, kb * 16) < wlen; ++kb) {
                    const v8i B = load32(&kbuf[st][(kb * 16 + (lane & 15)) * kLgRowPitch + 32 * g]);
                    const float ks = kscl[st][kb * 16 + (lane & 15)];
                    v4f C[kLgTokensPerWave][kLgHeadBlocks];
                    block_dots(C, B);
                    epilogue(C, ks, key_of(st, kb * 16) + (lane & 15));
                }
            }
        }
    }
    if (TPW == 1 && havep) epilogue(Cp, ksp, relp);
}

}  // namespace

hipError_t launch_logits(const LogitsParams& p, hipStream_t stream) {
    LogitsParams a = p;
    void* args[] = {&a};
    const dim3 grid((unsigned)p.blocks * (unsigned)p.chunks);
    const bool slots = p.key_slots != nullptr;
    if (p.tokens_per_wave == 1) {
        const void* k = slots ? reinterpret_cast<const void*>(&mqa_logits_kernel<1, true>)
                              : reinterpret_cast<const void*>(&mqa_logits_kernel<1, false>);
        return hipLaunchKernel(k, grid, dim3(LgShape<1>::kThreads), args, 0, stream);
    }
    const void* k = slots ? reinterpret_cast<const void*>(&mqa_logits_kernel<2, true>)
                          : reinterpret_cast<const void*>(&mqa_logits_kernel<2, false>);
    return hipLaunchKernel(k, grid, dim3(LgShape<2>::kThreads), args, 0, stream);
}

}  // namespace dsaidx
