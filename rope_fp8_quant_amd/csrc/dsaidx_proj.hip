// gfx950 kernel of the fused key / head-gate projection with the key
// preparation in its epilogue.
//
// The indexer computes its key and its head gates with one projection of the
// hidden states, the fused wk_weights_proj GEMM ([sglang-fuse] Motivation):
//   out[t, n] = sum_c hidden[t, c] * W[n, c],   n < 128: the key,
//                                              128 <= n < 128 + H: the gates.
// The unfused path writes out as bf16 and the preparation reads it back.  Here
// one dispatch does both: the projection on the matrix cores, then, while the
// workgroup's 128 key rows are still on chip, their LayerNorm, RoPE,
// quantisation and index-K cache store (the same device code as the key rows
// of the preparation kernel), and the gates written as bf16 for the query-side
// call.  The key values are rounded to bf16 first, as the GEMM's output is, so
// the cache holds what the preparation would store from that output.
//
// Mapping.  A workgroup of four wavefronts owns 256 tokens and all 128 + H
// (at most 192) output columns; wavefront w owns tokens 64w .. 64w + 63 as four
// 16-row blocks, with its 4 x 12 accumulator blocks in AGPRs (one wavefront
// per SIMD: 512 registers; 64 rows per wavefront halve the weight operand
// reads from LDS per token against 32).  The contraction runs in stages of
// 64 hidden elements with v_mfma_f32_16x16x32_bf16 (A: 16 tokens x 32, B:
// 32 x 16 columns):
//   - hidden rows go straight from HBM into the A operands (16 bytes per lane,
//     lane l: token l % 16, elements 8 (l / 16) ..), nontemporal: every
//     element is read once; as raw buffer loads from a per-workgroup base,
//     each address is one 32-bit register plus a scalar stage offset;
//   - the stage's weight slice (192 rows x 128 bytes) goes through LDS,
//     double-buffered, one barrier per stage; its rows are 144 bytes apart so
//     that the 16 lanes of a B-operand read hit distinct banks;
//   - each wavefront issues 4 x 12 MFMAs per 32 elements, accumulating in
//     fp32, with each weight operand read from LDS a few operands ahead
//     (the order is pinned with scheduling groups: the compiler otherwise
//     reads each operand just before its MFMAs).
// The first stage starts the accumulators with zero as the MFMAs' C operand:
// zeroing them beforehand gives 192 accumulators one shared zero register, and
// the register allocator then rotates them through spare registers inside
// the loop (about 150 copies per 192 MFMAs).
// Each stage first issues the next stage's weight slice and hidden rows; the
// stage ends with an LDS-only wait and a bare barrier, so the hidden rows stay
// in flight across it.  The weight (0.3 % of the bytes at d = 7168) is re-read
// from L2 by every workgroup.  The hidden rows have one stage to arrive:
// loads retire in issue order, so the wait for the next weight slice at the
// end of a stage is also a wait for the rows issued before it.  Two stages
// would need a second set of weight registers and of hidden rows, which the
// 512 registers of one wavefront per SIMD do not leave.
#include "dsaidx_prep_device.h"

#pragma clang fp contract(off)

namespace dsaidx {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = kProjThreads;
constexpr int kColBlocks = kProjMaxCols / 16;        // 12 blocks of 16 output columns
constexpr int kStageK = kProjStageK;                 // hidden elements per stage (64)
constexpr int kKSteps = kStageK / 32;                // MFMA k steps per stage
constexpr int kWChunks = kStageK / 8;                // 16-byte chunks of a weight row's stage slice
constexpr int kWRowsPerPass = kThreads / kWChunks;   // weight rows staged per pass of the workgroup
constexpr int kWPer = kProjMaxCols / kWRowsPerPass;  // weight chunks staged per thread and stage
static_assert(kWPer * kWRowsPerPass == kProjMaxCols, "weight staging covers the rows");
constexpr int kWPitch = kStageK * 2 + 16;            // LDS bytes per weight row (144)
constexpr int kWStageBytes = kProjMaxCols * kWPitch;   // 27648
constexpr int kKPitch = kRow * 2 + 16;               // LDS bytes per staged key row (272)
constexpr int kGPitch = kProjMaxHeads * 2 + 16;      // LDS bytes per staged gate row (144)
// LDS: the two weight stages during the contraction, then the epilogue's
// staging of the block's key and gate rows (106496 bytes at 256 tokens).
constexpr int kEpilogueBytes = kProjRows * (kKPitch + kGPitch);
constexpr int kSmemBytes = kEpilogueBytes > 2 * kWStageBytes ? kEpilogueBytes : 2 * kWStageBytes;
static_assert(kProjRows == 64 * (kThreads / 64), "64 tokens per wavefront");
static_assert(kThreads / 64 <= kXchgWaves, "rope_generic's exchange buffer covers every wavefront");

// The lane's eight bf16 values of one staged key row (layout order), from LDS.
template <int LAYOUT>
__device__ __forceinline__ uint4 lds_row(const uint8_t* row, int j) {
    if (LAYOUT != kSplit) return *reinterpret_cast<const uint4*>(row + 16 * j);
    const uint2 a = *reinterpret_cast<const uint2*>(row + 8 * j);
    const uint2 b = *reinterpret_cast<const uint2*>(row + 128 + 8 * j);
    return make_uint4(a.x, a.y, b.x, b.y);
}

typedef uint4 ARows[4][kKSteps];   // a wavefront's hidden-row operands of one stage: [row block][k step]

#ifndef DSAIDX_PROJ_AHEAD_B
#define DSAIDX_PROJ_AHEAD_B 4
#endif
constexpr int kAheadB = DSAIDX_PROJ_AHEAD_B;   // weight operands read from LDS ahead of their MFMAs

// Workgroup barrier after this wavefront's LDS writes have completed, with
// its global loads left in flight (a full __syncthreads() also waits for
// those).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// One wavefront per SIMD: each holds 192 accumulators (in AGPRs) and its
// operands in the 512 registers that leaves.
template <int STYLE, int LAYOUT>
__global__ __launch_bounds__(kThreads, 1) void proj_key_prep_kernel(ProjParams a) {
    __shared__ __align__(16) uint8_t smem[kSmemBytes];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15;          // MFMA operand row / column within a block
    const int lq = lane >> 4;          // MFMA operand k group (8 elements)
    const int wc = tid % kWChunks;     // weight staging: 16-byte chunk of a row's stage slice
    const int wr0 = tid / kWChunks;    //   and first row (rows wr0 + kWRowsPerPass j)
    const int64_t T = a.prep.T;
    const int stages = a.d / kStageK;

    for (int64_t blk = blockIdx.x; blk < a.row_blocks; blk += gridDim.x) {
        const int64_t row0 = blk * kProjRows;
        // Operand rows, clamped: a token past T reads row T - 1 and a column
        // past 128 + H reads the last weight row (their results are never
        // stored), so every load below is unconditional and the compiler's
        // waits stay exact.  Byte offsets are 32-bit: the host bounds both
        // row strides by 2^22 elements.
        const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(a.x + row0 * a.x_st), 0, -1, 0x00020000);
        const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(a.w), 0, -1, 0x00020000);
        uint32_t aoff[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t t = row0 + 64 * wave + 16 * i + lr;
            aoff[i] = (uint32_t)(((t < T ? t : T - 1) - row0) * a.x_st * 2) + 16u * lq;
        }
        uint32_t woff[kWPer];
#pragma unroll
        for (int jj = 0; jj < kWPer; ++jj) {
            const int n = wr0 + kWRowsPerPass * jj;
            woff[jj] = (uint32_t)((n < a.n_out ? n : a.n_out - 1) * a.w_st * 2) + 16u * wc;
        }
        f32x4 acc[4][kColBlocks];

        auto fetch_a = [&](int s, ARows& x) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int ks = 0; ks < kKSteps; ++ks)
                    x[i][ks] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                        xrs, aoff[i] + 64 * ks, 2 * kStageK * s, 2));
        };
        auto fetch_w = [&](int s, uint4 (&w)[kWPer]) {
#pragma unroll
            for (int jj = 0; jj < kWPer; ++jj)
                w[jj] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                    wrs, woff[jj], 2 * kStageK * s, 0));
        };
        auto store_w = [&](int buf, const uint4 (&w)[kWPer]) {
            uint8_t* base = smem + buf * kWStageBytes + 16 * wc;
#pragma unroll
            for (int jj = 0; jj < kWPer; ++jj)
                *reinterpret_cast<uint4*>(base + (wr0 + kWRowsPerPass * jj) * kWPitch) = w[jj];
        };
        // Stage s: the weight slice and the hidden rows of stage s + 1 are
        // issued (the weight first), the MFMAs of stage s run on `cur` and
        // weight buffer s & 1, each weight operand read from LDS kAheadB
        // operands before its MFMAs, and the next weight slice goes to the
        // other buffer before the stage's one barrier.  The last stage
        // re-fetches itself instead of branching.
        auto stage = [&](int s, const ARows& cur, ARows& fut, bool first) {
            uint4 wn[kWPer];
            fetch_w(s + 1 < stages ? s + 1 : s, wn);
            fetch_a(s + 1 < stages ? s + 1 : s, fut);
            const uint8_t* wb = smem + (s & 1) * kWStageBytes + lr * kWPitch + 16 * lq;
            auto bread = [&](int o) -> uint4 {       // operand o = kColBlocks ks + cb
                return *reinterpret_cast<const uint4*>(wb + (o % kColBlocks) * 16 * kWPitch +
                                                       64 * (o / kColBlocks));
            };
            constexpr int kOps = kKSteps * kColBlocks;
            uint4 bq[kAheadB];
#pragma unroll
            for (int o = 0; o < kAheadB; ++o) bq[o] = bread(o);
#pragma unroll
            for (int o = 0; o < kOps; ++o) {
                const int ks = o / kColBlocks, cb = o % kColBlocks;
                const bf16x8 b = __builtin_bit_cast(bf16x8, bq[o % kAheadB]);
                if (o + kAheadB < kOps) bq[o % kAheadB] = bread(o + kAheadB);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[i][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, cur[i][ks]), b,
                        first && ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[i][cb], 0, 0, 0);
            }
            // the order above, kept by the scheduler: the stage's global loads,
            // the first kAheadB weight reads, then the four MFMAs of each
            // operand with the next operand's read
            __builtin_amdgcn_sched_group_barrier(0x020, kWPer + 4 * kKSteps, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, kAheadB, 0);
#pragma unroll
            for (int o = kAheadB; o < kOps; ++o) {
                __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 4 * kAheadB, 0);
            store_w((s + 1) & 1, wn);
            lds_barrier();
        };

        ARows A0, A1;
        {
            uint4 w0[kWPer];
            fetch_w(0, w0);
            fetch_a(0, A0);
            store_w(0, w0);
        }
        __syncthreads();
        // two stages per iteration alternate the operand sets; an odd last
        // stage runs after the loop, so that its body has no branches (they
        // would make the compiler's waits conservative)
        stage(0, A0, A1, true);
        int s = 1;
        for (; s + 2 <= stages; s += 2) {
            stage(s, A1, A0, false);
            stage(s + 1, A0, A1, false);
        }
        if (s < stages) stage(s, A1, A0, false);
        __syncthreads();

        // Epilogue 1: the projection's output rounded to bf16 (nearest even),
        // staged in LDS (the stage buffers are free): key rows [256][128] and
        // gate rows [256][H].  Lane l holds column l % 16 of rows 4 (l / 16) ..
        // + 3 of each 16 x 16 block.
        uint8_t* ktile = smem;
        uint8_t* gtile = smem + kProjRows * kKPitch;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int cb = 0; cb < kColBlocks; ++cb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 64 * wave + 16 * i + 4 * lq + e;
                    const int c = 16 * cb + lr;
                    const uint16_t v = (uint16_t)(__float_as_uint(round_bf16(acc[i][cb][e])) >> 16);
                    if (c < kRow)
                        *reinterpret_cast<uint16_t*>(ktile + r * kKPitch + 2 * c) = v;
                    else if (c - kRow < a.H)
                        *reinterpret_cast<uint16_t*>(gtile + r * kGPitch + 2 * (c - kRow)) = v;
                }
        __syncthreads();

        // Epilogue 2: the gates (and, when asked, the bf16 key) to HBM.
        const int rows_here = (int)(T - row0 < kProjRows ? T - row0 : kProjRows);
        for (int idx = tid; idx < rows_here * a.H; idx += kThreads) {
            const int r = idx / a.H;
            const int h = idx - r * a.H;
            a.gates[(row0 + r) * a.g_st + h] = *reinterpret_cast<const uint16_t*>(gtile + r * kGPitch + 2 * h);
        }
        if (a.k_out) {
            for (int idx = tid; idx < rows_here * 16; idx += kThreads) {
                const int r = idx >> 4;
                const int c = idx & 15;
                *reinterpret_cast<uint4*>(a.k_out + (row0 + r) * a.ko_st + 8 * c) =
                    *reinterpret_cast<const uint4*>(ktile + r * kKPitch + 16 * c);
            }
        }

        // Epilogue 3: the key rows, four per wavefront pass, through the
        // preparation's key-row code (LayerNorm, RoPE, quantisation, store).
        const int g = lane >> 4;
        const int j = lane & (kLanesPerRow - 1);
        for (int pass = 0; pass < 16; ++pass) {
            const int r = 64 * wave + 4 * pass + g;
            const int64_t t = row0 + r;
            const bool valid = t < T;
            const uint4 raw = lds_row<LAYOUT>(ktile + r * kKPitch, j);
            int64_t pos = 0, slot = -1;
            if (valid) {
                pos = clamp_position(a.prep.k_pos[t], a.prep.P);
                slot = a.prep.loc[t];
            }
            key_row<STYLE, LAYOUT>(a.prep, valid, raw, pos, slot, lane);
        }
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_proj(const ProjParams& p, int style, unsigned grid, hipStream_t stream) {
    ProjParams copy = p;
    void* args[] = {&copy};
    const void* fn;
    if (p.prep.generic)
        fn = style == 1 ? reinterpret_cast<const void*>(&proj_key_prep_kernel<1, kGeneric>)
                        : reinterpret_cast<const void*>(&proj_key_prep_kernel<0, kGeneric>);
    else if (style == 1)
        fn = reinterpret_cast<const void*>(&proj_key_prep_kernel<1, kSplit>);
    else if (p.prep.R <= 64)
        fn = reinterpret_cast<const void*>(&proj_key_prep_kernel<0, kSplit>);
    else
        fn = reinterpret_cast<const void*>(&proj_key_prep_kernel<0, kContig>);
    return hipLaunchKernel(fn, dim3(grid), dim3(kThreads), args, 0, stream);
}

}  // namespace dsaidx
