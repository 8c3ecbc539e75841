// Private interface between the C-ABI host layer and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsaidx {

constexpr int kRow = 128;           // elements per head vector / key row
constexpr int kLanesPerRow = 16;    // one DPP row of a wavefront per vector
constexpr int kRowsPerWave = 4;     // 64 lanes / 16
// Query heads per wavefront work item: 16 for large batches; 4 when the call
// has at most kSmallBatchHeadRows query rows, where more, shorter work items
// cut the latency of a call that cannot fill the GPU.
constexpr int kHeadsPerItem = 16;
constexpr int kHeadsPerItemSmall = 4;
constexpr int kHeadsPerItemMid = 8;   // large batches of exactly 8 heads: items of 2 tokens x 8 heads
constexpr int64_t kSmallBatchHeadRows = 16384;
constexpr int kTokensPerKItem = 4;  // key rows per wavefront work item
constexpr int32_t kKeyBf16Intermediate = 0x1;  // DSAIDX_K_BF16_INTERMEDIATE
constexpr int32_t kKeyPagedCache = 0x2;        // DSAIDX_K_PAGED_CACHE
constexpr int32_t kKeyBf16Once = 0x4;          // DSAIDX_K_BF16_ROUND_ONCE
constexpr int kPagedScaleBytes = 4;            // fp32 scale per slot in a paged cache

// Everything one dispatch needs.  k_blocks workgroups run key work items and
// the others query work items (which ones: see the kernel); either set may be
// empty.
struct PrepParams {
    // query rows: item = (token, block of heads_per_item heads), or for
    // heads_per_item == kHeadsPerItemMid two tokens x 8 heads
    const uint16_t* q;
    int64_t q_st, q_sh;
    const uint16_t* w;
    int64_t w_st;
    const int64_t* q_pos;
    uint8_t* q_fp8;
    float* w_out;
    float* q_scale;
    float weight_scale;
    int32_t H;
    int32_t heads_per_item;  // kHeadsPerItem, kHeadsPerItemSmall or kHeadsPerItemMid
    int32_t head_blocks;  // ceil(H / heads_per_item); 1 for two-token items
    int32_t k_blocks;
    int32_t k_first;      // host only: fused small call with key workgroups first
    int32_t k_period;     // fused 8-head call of several rounds: one key workgroup in every k_period (0: together)
    uint32_t k_magic;     // workgroup / k_period = (workgroup * k_magic) >> k_shift
    int32_t k_shift;
    int64_t q_items;      // T * head_blocks, or ceil(T / 2) for two-token items (0: no query work)
    // key rows: item = 4 consecutive tokens
    const uint16_t* k;
    int64_t k_st;
    const float* gamma;
    const float* beta;
    const int64_t* k_pos;
    const int64_t* loc;
    uint8_t* k_cache;
    int64_t k_row_stride;  // bytes (planar cache)
    float* k_scale;        // planar cache
    int64_t S;
    int64_t page_size;     // paged cache: slots per page (0 = planar)
    int32_t k_flags;       // DSAIDX_K_* bits
    int64_t k_items;       // ceil(T / 4) (0 when the dispatch has no key work)
    int64_t T;
    float eps;
    // rope table
    int32_t generic;       // host only: element-wise rope path (see the kernel)
    int32_t R;
    const float* cos;
    const float* sin;
    int64_t rs;            // floats between table rows
    int64_t P;             // table rows
};

// Enqueue one dispatch of the preparation kernel for rope style 0 (NeoX) or 1
// (interleaved).
hipError_t launch_prep(const PrepParams& p, int style, unsigned grid, unsigned block,
                       hipStream_t stream);

// Workspace bytes the top-k selection needs for this shape: 0 for rows of up
// to 32768 logits, -1 for a shape too large to launch.
int64_t topk_workspace_bytes(int64_t rows, int64_t cols, int32_t k);

// Enqueue the top-k-per-row selection (one or four dispatches); `workspace`
// holds topk_workspace_bytes(rows, cols, k) bytes.
hipError_t launch_topk(const float* logits, int64_t row_stride, const int32_t* lengths,
                       int64_t rows, int64_t cols, int32_t k, int32_t* out, void* workspace,
                       hipStream_t stream);

// Workspace of the allocation-free top-k entry point: a device array of this
// many bytes in the library's code object, one per GPU (devices 0 ..
// kTopkScratchDevices - 1).  topk_scratch returns its address on `device`,
// which must be the current device on the first call there.
constexpr int64_t kTopkScratchBytes = int64_t(16) << 20;
constexpr int kTopkScratchDevices = 64;
hipError_t topk_scratch(int device, void** ptr);

// Enqueue the stand-alone E4M3FN conversion of in[i] / scale (self-test of
// the device encoder; scale a power of two).
hipError_t launch_fp8_selftest(const float* in, uint8_t* out, int64_t n, float scale,
                               unsigned grid, hipStream_t stream);

// Fused key / head-gate projection with the key preparation in its epilogue
// (one dispatch): out = hidden [T, d] x W[128 + H, d]^T in fp32 on the matrix
// cores, rounded to bf16; columns 0..127 go through the key preparation of
// `prep` (its k / k_st are unused), columns 128.. are written to gates.
constexpr int kProjRows = 256;       // tokens per workgroup
constexpr int kProjThreads = 256;    // 4 wavefronts per workgroup
constexpr int kProjMaxHeads = 64;    // gate columns at most
constexpr int kProjMaxCols = kRow + kProjMaxHeads;
constexpr int kProjStageK = 64;      // d is a multiple of this

struct ProjParams {
    const uint16_t* x;     // hidden bf16 [T, d], token stride x_st (elements)
    int64_t x_st;
    const uint16_t* w;     // weight bf16 [n_out, d], row stride w_st (elements)
    int64_t w_st;
    int32_t d;
    int32_t n_out;         // 128 + H
    int32_t H;
    uint16_t* gates;       // bf16 [T, H], token stride g_st
    int64_t g_st;
    uint16_t* k_out;       // bf16 [T, 128] (token stride ko_st) or null
    int64_t ko_st;
    int64_t row_blocks;    // ceil(T / kProjRows)
    PrepParams prep;       // the key side and the rope table
};

hipError_t launch_proj(const ProjParams& p, int style, unsigned grid, hipStream_t stream);

// Reference HBM stream over `vectors` 16-byte vectors: mode 0 copy, 1 read,
// 2 write (one dispatch).
hipError_t launch_hbm_stream(int mode, const void* src, void* dst, int64_t vectors,
                             uint32_t word, hipStream_t stream);

// Index logits (one dispatch): queries of at most kLogitsMaxHeads heads
// against num_keys keys of the index-K cache.
constexpr int kLogitsMaxHeads = 64;
constexpr int kLogitsTokensPerBlock = 8;     // query tokens per workgroup
constexpr int kLogitsStageKeys = 128;       // keys per LDS stage; chunks are multiples

struct LogitsParams {
    const uint8_t* q;          // [T, H, 128] E4M3 codes
    const float* w;            // [T, H] folded gates
    int32_t T;                 // query tokens, below 2^31
    int32_t H;
    const uint8_t* k_cache;
    int64_t k_row_stride;      // planar: bytes per slot row
    const float* k_scale;      // planar
    uint32_t S;                // slots, capped at 2^31 (every non-negative int32 slot below it is valid)
    int32_t page_size;         // page-interleaved layout: slots per page (0 = planar)
    uint32_t page_magic;       // slot / page_size = (slot * page_magic) >> page_shift
    int32_t page_shift;        //   for every slot below 2^31
    const int32_t* key_slots;  // [N] or null (key s = slot s)
    int32_t N;                 // keys, below 2^31
    const int32_t* lengths;    // [T] or null
    float* out;
    int64_t out_stride;
    int32_t chunk;             // keys per workgroup (at most 2^30)
    int32_t chunks;            // key chunks
    int32_t blocks;            // token blocks, ceil(T / 8): the grid is blocks * chunks (below 2^31)
    uint32_t grid_magic;       // workgroup / (chunk_major ? blocks : chunks) = (wg * grid_magic) >> grid_shift
    int32_t grid_shift;
    int32_t chunk_major;       // workgroup order: chunk-major (1) or token-block-major (0)
    int32_t tokens_per_wave;   // 1: 8-wavefront workgroups, pipelined blocks; 2: 4 wavefronts
};

hipError_t launch_logits(const LogitsParams& p, hipStream_t stream);

}  // namespace dsaidx
