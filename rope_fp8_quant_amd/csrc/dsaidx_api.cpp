// C-ABI host layer of libdsaidx: argument checks, launch shape, status codes.
// The operation and the argument contract are documented in include/dsaidx.h.
#include "dsaidx.h"

#include <cmath>
#include <cstring>

#include "dsaidx_internal.h"

static_assert(dsaidx::kKeyBf16Intermediate == DSAIDX_K_BF16_INTERMEDIATE, "flag bits");
static_assert(dsaidx::kKeyPagedCache == DSAIDX_K_PAGED_CACHE, "flag bits");
static_assert(dsaidx::kKeyBf16Once == DSAIDX_K_BF16_ROUND_ONCE, "flag bits");
static_assert(dsaidx::kTopkScratchBytes == DSAIDX_TOPK_NOALLOC_SCRATCH_BYTES, "scratch size");

namespace {

using dsaidx::PrepParams;

constexpr int64_t kMaxTokens = int64_t(1) << 40;
constexpr int32_t kMaxHeads = 4096;
constexpr unsigned kBlock = 256;          // 4 wavefronts
constexpr unsigned kSmallBlock = 64;      // 1 wavefront (k-only launch shape)
// Launch shape: one workgroup per 4 work items up to this many workgroups
// (beyond it the kernels loop).  A one-shot grid streams measurably faster on
// MI355X than a grid capped near the CU count with long grid-stride loops.
// A dispatch counts its work-items in 32 bits, so workgroups * block size
// stays below 2^32 (max_grid).
#ifndef DSAIDX_MAX_GRID
#define DSAIDX_MAX_GRID (1 << 24)
#endif
constexpr int64_t kMaxGrid = DSAIDX_MAX_GRID;

int64_t max_grid(unsigned block) {
    const int64_t fit = ((int64_t(1) << 32) - 1) / block;
    return fit < kMaxGrid ? fit : kMaxGrid;
}
constexpr int kKeyBlockDivisor = 16;      // fused: key workgroups <= query workgroups / 16
constexpr int64_t kSpreadKeysAbove = 2048; // fused, 8 heads: grids larger than one resident round spread the key workgroups

bool token_count_ok(int64_t t) { return t >= 0 && t <= kMaxTokens; }

bool aligned(const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

dsaidx_status check_rope(const dsaidx_rope* r) {
    if (!r->cos || !r->sin) return DSAIDX_ERR_INVALID_ARGUMENT;
    if (!aligned(r->cos, 4) || !aligned(r->sin, 4)) return DSAIDX_ERR_INVALID_ARGUMENT;
    if (r->rope_dim < 2 || r->rope_dim > dsaidx::kRow || r->rope_dim % 2 != 0)
        return DSAIDX_ERR_INVALID_ARGUMENT;
    if (r->style != DSAIDX_ROPE_NEOX && r->style != DSAIDX_ROPE_INTERLEAVED)
        return DSAIDX_ERR_INVALID_ARGUMENT;
    if (r->row_stride < r->rope_dim / 2) return DSAIDX_ERR_INVALID_ARGUMENT;
    if (r->max_position < 1) return DSAIDX_ERR_INVALID_ARGUMENT;
    return DSAIDX_OK;
}

// The vectorised rope paths need rope_dim a multiple of 16 and 16-byte aligned
// table rows; anything else takes the element-wise path.
bool rope_generic(const dsaidx_rope& r) {
    return !(r.rope_dim % 16 == 0 && r.row_stride % 4 == 0 && aligned(r.cos, 16) &&
             aligned(r.sin, 16));
}

dsaidx_status check_q(const dsaidx_q_args* q) {
    if (q->num_heads < 1 || q->num_heads > kMaxHeads) return DSAIDX_ERR_INVALID_ARGUMENT;
    if (!std::isfinite(q->weight_scale)) return DSAIDX_ERR_INVALID_ARGUMENT;
    if (!q->q || !q->weights || !q->positions || !q->q_fp8 || !q->weights_out)
        return DSAIDX_ERR_INVALID_ARGUMENT;
    if (!aligned(q->q, 16) || !aligned(q->weights, 2) || !aligned(q->positions, 8) ||
        !aligned(q->q_fp8, 8) || !aligned(q->weights_out, 4) ||
        (q->q_scale_out && !aligned(q->q_scale_out, 4)))
        return DSAIDX_ERR_INVALID_ARGUMENT;
    if (q->q_stride_h < dsaidx::kRow || q->q_stride_h % 8 != 0) return DSAIDX_ERR_INVALID_ARGUMENT;
    if (q->q_stride_t % 8 != 0 ||
        q->q_stride_t < (int64_t)(q->num_heads - 1) * q->q_stride_h + dsaidx::kRow)
        return DSAIDX_ERR_INVALID_ARGUMENT;
    if (q->w_stride_t < q->num_heads) return DSAIDX_ERR_INVALID_ARGUMENT;
    return DSAIDX_OK;
}

// The key side; with_row = false skips k and k_stride_t (the projection entry
// computes the key itself).
dsaidx_status check_k(const dsaidx_k_args* k, bool with_row = true) {
    if (!k->ln_gamma || !k->ln_beta || !k->positions || !k->out_cache_loc || !k->k_cache)
        return DSAIDX_ERR_INVALID_ARGUMENT;
    if (!aligned(k->ln_gamma, 16) || !aligned(k->ln_beta, 16) || !aligned(k->positions, 8) ||
        !aligned(k->out_cache_loc, 8) || !aligned(k->k_cache, 8))
        return DSAIDX_ERR_INVALID_ARGUMENT;
    if (with_row && (!k->k || !aligned(k->k, 16) || k->k_stride_t < dsaidx::kRow || k->k_stride_t % 8 != 0))
        return DSAIDX_ERR_INVALID_ARGUMENT;
    if (!(k->ln_eps > 0.0f) || !std::isfinite(k->ln_eps)) return DSAIDX_ERR_INVALID_ARGUMENT;
    if (k->flags & ~(DSAIDX_K_BF16_INTERMEDIATE | DSAIDX_K_PAGED_CACHE | DSAIDX_K_BF16_ROUND_ONCE))
        return DSAIDX_ERR_INVALID_ARGUMENT;
    if ((k->flags & DSAIDX_K_BF16_INTERMEDIATE) && (k->flags & DSAIDX_K_BF16_ROUND_ONCE))
        return DSAIDX_ERR_INVALID_ARGUMENT;
    if (k->num_slots < 1) return DSAIDX_ERR_INVALID_ARGUMENT;
    if (k->flags & DSAIDX_K_PAGED_CACHE) {
        if (k->page_size < 2 || k->page_size > (1 << 20) || k->page_size % 2 != 0 ||
            k->num_slots % k->page_size != 0)
            return DSAIDX_ERR_INVALID_ARGUMENT;
    } else {
        if (!k->k_scale || !aligned(k->k_scale, 4)) return DSAIDX_ERR_INVALID_ARGUMENT;
        if (k->k_cache_row_stride < dsaidx::kRow || k->k_cache_row_stride % 8 != 0)
            return DSAIDX_ERR_INVALID_ARGUMENT;
    }
    return DSAIDX_OK;
}

void fill_rope(PrepParams& p, const dsaidx_rope& r) {
    p.cos = r.cos;
    p.sin = r.sin;
    p.rs = r.row_stride;
    p.P = r.max_position;
    p.R = r.rope_dim;
    p.generic = rope_generic(r) ? 1 : 0;
}

void fill_q(PrepParams& p, const dsaidx_q_args& q) {
    p.q = q.q;
    p.q_st = q.q_stride_t;
    p.q_sh = q.q_stride_h;
    p.w = q.weights;
    p.w_st = q.w_stride_t;
    p.q_pos = q.positions;
    p.q_fp8 = q.q_fp8;
    p.w_out = q.weights_out;
    p.q_scale = q.q_scale_out;
    p.weight_scale = q.weight_scale;
    p.H = q.num_heads;
    // (the element-wise rope path has no two-token items)
    p.heads_per_item = q.num_tokens * q.num_heads <= dsaidx::kSmallBatchHeadRows
                           ? dsaidx::kHeadsPerItemSmall
                           : (q.num_heads == dsaidx::kHeadsPerItemMid && !p.generic
                                  ? dsaidx::kHeadsPerItemMid
                                  : dsaidx::kHeadsPerItem);
    if (p.heads_per_item == dsaidx::kHeadsPerItemMid) {
        // items of two tokens x 8 heads
        p.head_blocks = 1;
        p.q_items = (q.num_tokens + 1) / 2;
    } else {
        p.head_blocks = (q.num_heads + p.heads_per_item - 1) / p.heads_per_item;
        p.q_items = q.num_tokens * p.head_blocks;
    }
    p.T = q.num_tokens;
}

void fill_k(PrepParams& p, const dsaidx_k_args& k) {
    p.k = k.k;
    p.k_st = k.k_stride_t;
    p.gamma = k.ln_gamma;
    p.beta = k.ln_beta;
    p.eps = k.ln_eps;
    p.k_pos = k.positions;
    p.loc = k.out_cache_loc;
    p.k_cache = k.k_cache;
    p.k_row_stride = k.k_cache_row_stride;
    p.k_scale = k.k_scale;
    p.S = k.num_slots;
    p.k_flags = k.flags;
    p.page_size = (k.flags & DSAIDX_K_PAGED_CACHE) ? k.page_size : 0;
    p.k_items = (k.num_tokens + dsaidx::kTokensPerKItem - 1) / dsaidx::kTokensPerKItem;
    p.T = k.num_tokens;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

dsaidx_status to_status(hipError_t err) {
    if (err == hipSuccess) return DSAIDX_OK;
    if (err == hipErrorNoDevice || err == hipErrorInvalidDeviceFunction ||
        err == hipErrorNoBinaryForGpu || err == hipErrorInsufficientDriver)
        return DSAIDX_ERR_UNSUPPORTED;
    return DSAIDX_ERR_HIP;
}

dsaidx_status launch(const PrepParams& p, int style, int64_t grid, unsigned block,
                     dsaidx_stream_t stream) {
    if (grid <= 0) return DSAIDX_OK;
    return to_status(dsaidx::launch_prep(p, style, (unsigned)grid, block,
                                         reinterpret_cast<hipStream_t>(stream)));
}

// Keys per logits workgroup for T queries over N keys: enough workgroups to
// fill the GPU (about 3072, four rounds of the 768 that are resident at three
// per CU; each reads its 8 tokens' queries once), but at least 256 keys each,
// in whole LDS stages.  *chunks receives ceil(N / chunk).
#ifndef DSAIDX_LG_TARGET_WGS
#define DSAIDX_LG_TARGET_WGS 3072
#endif
#ifndef DSAIDX_LG_MIN_CHUNK
#define DSAIDX_LG_MIN_CHUNK 256
#endif
// Workgroups of 8 wavefronts resident at once at two per CU on the 256 CUs.
constexpr int64_t kLogitsOneRound = 512;

int64_t logits_key_chunk(int64_t T, int64_t N, int64_t* chunks) {
    const int64_t blocks = ceil_div(T, dsaidx::kLogitsTokensPerBlock);
    const int64_t most = ceil_div(N, DSAIDX_LG_MIN_CHUNK);
    int64_t want = ceil_div(DSAIDX_LG_TARGET_WGS, blocks);
    if (want > most) want = most;
    if (want < 1) want = 1;
    int64_t chunk = ceil_div(ceil_div(N, want), dsaidx::kLogitsStageKeys) * dsaidx::kLogitsStageKeys;
    if (chunk > (int64_t(1) << 30)) chunk = int64_t(1) << 30;   // key offsets within a chunk are 32-bit
    *chunks = ceil_div(N, chunk);
    return chunk;
}

// Granlund-Montgomery magic number: n / d = (n * magic) >> shift for every
// n below 2^31 (d >= 1).
void page_divisor(int64_t d, uint32_t* magic, int32_t* shift) {
    int l = 0;
    while ((int64_t(1) << l) < d) ++l;
    const int s = 31 + l;
    const unsigned __int128 m = ((unsigned __int128)1 << s) / (unsigned __int128)d + 1;
    *magic = (uint32_t)m;
    *shift = s;
}

int64_t capped_grid(int64_t items, unsigned block) {
    const int64_t need = ceil_div(items, block / 64);
    return need < max_grid(block) ? need : max_grid(block);
}

}  // namespace

extern "C" {

dsaidx_status dsaidx_q_rope_quant_fold(const dsaidx_q_args* q, const dsaidx_rope* rope,
                                       dsaidx_stream_t stream) {
    if (!q || !rope || !token_count_ok(q->num_tokens)) return DSAIDX_ERR_INVALID_ARGUMENT;
    if (q->num_tokens == 0) return DSAIDX_OK;
    dsaidx_status st = check_rope(rope);
    if (st == DSAIDX_OK) st = check_q(q);
    if (st != DSAIDX_OK) return st;
    PrepParams p;
    std::memset(&p, 0, sizeof p);
    fill_rope(p, *rope);
    fill_q(p, *q);
    p.k_blocks = 0;
    return launch(p, rope->style, capped_grid(p.q_items, kBlock), kBlock, stream);
}

dsaidx_status dsaidx_k_norm_rope_quant_store(const dsaidx_k_args* k, const dsaidx_rope* rope,
                                             dsaidx_stream_t stream) {
    if (!k || !rope || !token_count_ok(k->num_tokens)) return DSAIDX_ERR_INVALID_ARGUMENT;
    if (k->num_tokens == 0) return DSAIDX_OK;
    dsaidx_status st = check_rope(rope);
    if (st == DSAIDX_OK) st = check_k(k);
    if (st != DSAIDX_OK) return st;
    PrepParams p;
    std::memset(&p, 0, sizeof p);
    fill_rope(p, *rope);
    fill_k(p, *k);
    const int64_t kb = capped_grid(p.k_items, kBlock);
    p.k_blocks = (int32_t)kb;
    return launch(p, rope->style, kb, kBlock, stream);
}

dsaidx_status dsaidx_k_only_prepare_store(const dsaidx_k_args* k, const dsaidx_rope* rope,
                                          dsaidx_stream_t stream) {
    if (!k || !rope || !token_count_ok(k->num_tokens)) return DSAIDX_ERR_INVALID_ARGUMENT;
    if (k->num_tokens == 0) return DSAIDX_OK;
    dsaidx_status st = check_rope(rope);
    if (st == DSAIDX_OK) st = check_k(k);
    if (st != DSAIDX_OK) return st;
    PrepParams p;
    std::memset(&p, 0, sizeof p);
    fill_rope(p, *rope);
    fill_k(p, *k);
    // One wavefront per workgroup: few tokens spread over as many CUs as
    // possible (the dense decode path runs a handful of tokens).
    const int64_t kb = capped_grid(p.k_items, kSmallBlock);
    p.k_blocks = (int32_t)kb;
    return launch(p, rope->style, kb, kSmallBlock, stream);
}

dsaidx_status dsaidx_qk_fused(const dsaidx_q_args* q, const dsaidx_k_args* k,
                              const dsaidx_rope* rope, dsaidx_stream_t stream) {
    if (!q || !k || !rope || !token_count_ok(q->num_tokens) || q->num_tokens != k->num_tokens)
        return DSAIDX_ERR_INVALID_ARGUMENT;
    if (q->num_tokens == 0) return DSAIDX_OK;
    dsaidx_status st = check_rope(rope);
    if (st == DSAIDX_OK) st = check_q(q);
    if (st == DSAIDX_OK) st = check_k(k);
    if (st != DSAIDX_OK) return st;
    PrepParams p;
    std::memset(&p, 0, sizeof p);
    fill_rope(p, *rope);
    fill_q(p, *q);
    fill_k(p, *k);
    const int64_t qb = capped_grid(p.q_items, kBlock);
    int64_t kb = ceil_div(p.k_items, kBlock / 64);
    // key rows are a small share of the bytes at 16 heads per item (a 16th of
    // the query workgroups suffice); with 8 heads per token they are a sixth,
    // and a small call is latency-bound: no cap there
    const int64_t kcap = p.heads_per_item == dsaidx::kHeadsPerItem
                             ? ceil_div(qb, kKeyBlockDivisor) : capped_grid(p.k_items, kBlock);
    if (kb > kcap) kb = kcap;
    // small calls of 32 tokens or more: key workgroups first (the kernel's kKeysFirst placement)
    p.k_first = (p.heads_per_item == dsaidx::kHeadsPerItemSmall && p.T >= 32) ? 1 : 0;

    p.k_blocks = (int32_t)kb;
    // 8-head calls of more than one resident round (8 workgroups of 256
    // threads per CU): key workgroups spread evenly through the grid, so that
    // their VALU-bound rows overlap the query rows' memory stream (65536
    // tokens: 42.4-42.7 against 43.0-43.1 us with the key workgroups last; at
    // 64 heads, where the key rows are a 24th of the bytes, spreading cost the
    // 8192-token call 3 %)
    if (p.heads_per_item == dsaidx::kHeadsPerItemMid && kb > 0 && qb + kb > kSpreadKeysAbove) {
        p.k_period = (int32_t)((qb + kb) / kb);
        page_divisor(p.k_period, &p.k_magic, &p.k_shift);
    }
    return launch(p, rope->style, qb + kb, kBlock, stream);
}

dsaidx_status dsaidx_proj_k_norm_rope_quant_store(const dsaidx_proj_args* j, const dsaidx_k_args* k,
                                                  const dsaidx_rope* rope, dsaidx_stream_t stream) {
    if (!j || !k || !rope || !token_count_ok(k->num_tokens)) return DSAIDX_ERR_INVALID_ARGUMENT;
    if (k->num_tokens == 0) return DSAIDX_OK;
    dsaidx_status st = check_rope(rope);
    if (st == DSAIDX_OK) st = check_k(k, false);
    if (st != DSAIDX_OK) return st;
    const int64_t d = j->hidden_dim;
    if (d < dsaidx::kProjStageK || d > (int64_t(1) << 20) || d % dsaidx::kProjStageK != 0)
        return DSAIDX_ERR_INVALID_ARGUMENT;
    if (j->num_heads < 1 || j->num_heads > dsaidx::kProjMaxHeads || j->reserved != 0)
        return DSAIDX_ERR_INVALID_ARGUMENT;
    // row strides of at most 2^22 elements keep the kernel's byte offsets
    // within a workgroup's 256 hidden rows, and within the weight, below 2^31
    if (!j->hidden || !aligned(j->hidden, 16) || j->hidden_stride_t < d || j->hidden_stride_t % 8 != 0 ||
        j->hidden_stride_t > (int64_t(1) << 22))
        return DSAIDX_ERR_INVALID_ARGUMENT;
    if (!j->weight || !aligned(j->weight, 16) || j->weight_stride_n < d || j->weight_stride_n % 8 != 0 ||
        j->weight_stride_n > (int64_t(1) << 22))
        return DSAIDX_ERR_INVALID_ARGUMENT;
    if (!j->gates_out || !aligned(j->gates_out, 2) || j->gates_stride_t < j->num_heads)
        return DSAIDX_ERR_INVALID_ARGUMENT;
    if (j->k_out && (!aligned(j->k_out, 16) || j->k_out_stride_t < dsaidx::kRow ||
                     j->k_out_stride_t % 8 != 0))
        return DSAIDX_ERR_INVALID_ARGUMENT;
    dsaidx::ProjParams p;
    std::memset(&p, 0, sizeof p);
    fill_rope(p.prep, *rope);
    fill_k(p.prep, *k);
    p.prep.k = nullptr;
    p.prep.k_st = 0;
    p.x = j->hidden;
    p.x_st = j->hidden_stride_t;
    p.w = j->weight;
    p.w_st = j->weight_stride_n;
    p.d = (int32_t)d;
    p.H = j->num_heads;
    p.n_out = dsaidx::kRow + j->num_heads;
    p.gates = j->gates_out;
    p.g_st = j->gates_stride_t;
    p.k_out = j->k_out;
    p.ko_st = j->k_out_stride_t;
    p.row_blocks = ceil_div(k->num_tokens, dsaidx::kProjRows);
    const int64_t grid = p.row_blocks < max_grid(dsaidx::kProjThreads) ? p.row_blocks
                                                                      : max_grid(dsaidx::kProjThreads);
    return to_status(dsaidx::launch_proj(p, rope->style, (unsigned)grid,
                                         reinterpret_cast<hipStream_t>(stream)));
}

static bool topk_shape_ok(int64_t rows, int64_t cols, int32_t k) {
    return rows >= 0 && rows < (int64_t(1) << 31) && cols >= 0 && cols < (int64_t(1) << 31) &&
           k >= 1 && k <= (1 << 20);
}

int64_t dsaidx_topk_workspace_bytes(int64_t rows, int64_t cols, int32_t k) {
    if (!topk_shape_ok(rows, cols, k)) return -1;
    return dsaidx::topk_workspace_bytes(rows, cols, k);
}

dsaidx_status dsaidx_topk_per_row(const float* logits, int64_t row_stride, const int32_t* lengths,
                                  int64_t rows, int64_t cols, int32_t k, int32_t* out_idx,
                                  void* workspace, int64_t workspace_bytes,
                                  dsaidx_stream_t stream) {
    if (!topk_shape_ok(rows, cols, k)) return DSAIDX_ERR_INVALID_ARGUMENT;
    if (rows == 0) return DSAIDX_OK;
    if (!logits || !out_idx || !aligned(logits, 16) || !aligned(out_idx, 4) ||
        (lengths && !aligned(lengths, 4)))
        return DSAIDX_ERR_INVALID_ARGUMENT;
    if (row_stride < cols || row_stride % 4 != 0) return DSAIDX_ERR_INVALID_ARGUMENT;
    const int64_t need = dsaidx::topk_workspace_bytes(rows, cols, k);
    if (need < 0) return DSAIDX_ERR_INVALID_ARGUMENT;
    if (need > 0 && (!workspace || !aligned(workspace, 16) || workspace_bytes < need))
        return DSAIDX_ERR_INVALID_ARGUMENT;
    return to_status(dsaidx::launch_topk(logits, row_stride, lengths, rows, cols, k, out_idx,
                                         workspace, reinterpret_cast<hipStream_t>(stream)));
}

dsaidx_status dsaidx_topk_per_row_noalloc(const float* logits, int64_t row_stride,
                                          const int32_t* lengths, int64_t rows, int64_t cols,
                                          int32_t k, int32_t* out_idx, dsaidx_stream_t stream) {
    if (!topk_shape_ok(rows, cols, k)) return DSAIDX_ERR_INVALID_ARGUMENT;
    const int64_t need = dsaidx::topk_workspace_bytes(rows, cols, k);
    if (need < 0 || need > dsaidx::kTopkScratchBytes) return DSAIDX_ERR_INVALID_ARGUMENT;
    if (rows == 0) return DSAIDX_OK;
    void* ws = nullptr;
    if (need > 0) {
        int device = -1;
        if (hipGetDevice(&device) != hipSuccess) return DSAIDX_ERR_UNSUPPORTED;
        if (stream) {
            int sdev = -1;
            if (hipStreamGetDevice(reinterpret_cast<hipStream_t>(stream), &sdev) != hipSuccess)
                return DSAIDX_ERR_HIP;
            if (sdev != device) return DSAIDX_ERR_INVALID_ARGUMENT;
        }
        const hipError_t e = dsaidx::topk_scratch(device, &ws);
        if (e != hipSuccess) return to_status(e);
    }
    return dsaidx_topk_per_row(logits, row_stride, lengths, rows, cols, k, out_idx, ws, need,
                               stream);
}

// Division by the page size as a multiply and shift, exact for every
// numerator below 2^31 (Granlund and Montgomery, "Division by invariant
// integers using multiplication", 1994, with N = 31 bits): l = ceil(log2 d),
// shift = 31 + l, magic = floor(2^shift / d) + 1.  Then magic * d - 2^shift
// lies in (0, d] and d <= 2^l = 2^(shift - 31), which is the condition for
// floor(n * magic / 2^shift) = floor(n / d); magic < 2^32 since d > 2^(l - 1).

dsaidx_status dsaidx_mqa_logits(const dsaidx_logits_args* a, dsaidx_stream_t stream) {
    if (!a || a->num_tokens < 0 || a->num_tokens >= (int64_t(1) << 31) || a->num_keys < 0 ||
        a->num_keys >= (int64_t(1) << 31))
        return DSAIDX_ERR_INVALID_ARGUMENT;
    if (a->num_tokens == 0 || a->num_keys == 0) return DSAIDX_OK;
    if (a->num_heads < 1 || a->num_heads > dsaidx::kLogitsMaxHeads) return DSAIDX_ERR_INVALID_ARGUMENT;
    if (!a->q_fp8 || !a->weights || !a->k_cache || !a->logits) return DSAIDX_ERR_INVALID_ARGUMENT;
    if (!aligned(a->q_fp8, 16) || !aligned(a->weights, 4) || !aligned(a->k_cache, 8) ||
        !aligned(a->logits, 4) || (a->key_slots && !aligned(a->key_slots, 4)) ||
        (a->lengths && !aligned(a->lengths, 4)))
        return DSAIDX_ERR_INVALID_ARGUMENT;
    if (a->flags & ~DSAIDX_K_PAGED_CACHE) return DSAIDX_ERR_INVALID_ARGUMENT;
    if (a->num_slots < 1) return DSAIDX_ERR_INVALID_ARGUMENT;
    const bool paged = (a->flags & DSAIDX_K_PAGED_CACHE) != 0;
    if (paged) {
        if (a->page_size < 2 || a->page_size > (1 << 20) || a->page_size % 2 != 0 ||
            a->num_slots % a->page_size != 0)
            return DSAIDX_ERR_INVALID_ARGUMENT;
    } else {
        if (!a->k_scale || !aligned(a->k_scale, 4)) return DSAIDX_ERR_INVALID_ARGUMENT;
        if (a->k_cache_row_stride < dsaidx::kRow || a->k_cache_row_stride % 8 != 0)
            return DSAIDX_ERR_INVALID_ARGUMENT;
    }
    if (!a->key_slots && a->num_keys > a->num_slots) return DSAIDX_ERR_INVALID_ARGUMENT;
    if (a->logits_stride < a->num_keys) return DSAIDX_ERR_INVALID_ARGUMENT;
    const int64_t blocks = ceil_div(a->num_tokens, dsaidx::kLogitsTokensPerBlock);
    int64_t chunks = 0;
    const int64_t chunk = logits_key_chunk(a->num_tokens, a->num_keys, &chunks);
    if (blocks * chunks >= (int64_t(1) << 31)) return DSAIDX_ERR_INVALID_ARGUMENT;
    dsaidx::LogitsParams p;
    std::memset(&p, 0, sizeof p);
    p.q = a->q_fp8;
    p.w = a->weights;
    p.T = (int32_t)a->num_tokens;
    p.H = a->num_heads;
    p.k_cache = a->k_cache;
    p.k_row_stride = paged ? 0 : a->k_cache_row_stride;
    p.k_scale = paged ? nullptr : a->k_scale;
    p.S = (uint32_t)(a->num_slots < (int64_t(1) << 31) ? a->num_slots : (int64_t(1) << 31));
    p.page_size = paged ? (int32_t)a->page_size : 0;
    if (paged) page_divisor(a->page_size, &p.page_magic, &p.page_shift);
    p.key_slots = a->key_slots;
    p.N = (int32_t)a->num_keys;
    p.lengths = a->lengths;
    p.out = a->logits;
    p.out_stride = a->logits_stride;
    p.chunk = (int32_t)chunk;
    p.chunks = (int32_t)chunks;
    p.blocks = (int32_t)blocks;
    p.chunk_major = blocks >= chunks ? 1 : 0;
    // the kernel splits its workgroup index by the magic-number division
    // (Granlund-Montgomery, as for the page size): by the token blocks in
    // chunk-major order, by the chunks in token-block-major order
    page_divisor(p.chunk_major ? blocks : chunks, &p.grid_magic, &p.grid_shift);
    // One token per wavefront when the grid is one resident round (two of its
    // 8-wavefront workgroups per CU): its four wavefronts per SIMD and
    // pipelined blocks shorten a decode call (14.3-14.7 against 15.1-15.5 us
    // for 64 tokens x 16384 keys); larger calls keep two tokens per
    // wavefront, which reads each key operand for twice the MFMAs (285-293
    // against 275-281 us on the causal 8192-token prefill).
    // The one-token kernel takes 16 blocks of 16 keys per workgroup, spread
    // over the key range at a stride of `chunks` blocks: they cover the keys
    // when 256 * chunks >= N (always so in one round, whose chunks hold at
    // most 256 keys).
    p.tokens_per_wave = blocks * chunks <= kLogitsOneRound &&
                        chunks * 2 * dsaidx::kLogitsStageKeys >= a->num_keys ? 1 : 2;
    return to_status(dsaidx::launch_logits(p, reinterpret_cast<hipStream_t>(stream)));
}

dsaidx_status dsaidx_fp8_encode_selftest(const float* in, uint8_t* out, int64_t n,
                                         int32_t scale_exp, dsaidx_stream_t stream) {
    if (n < 0 || !in || !out || !aligned(in, 4) || !aligned(out, 8))
        return DSAIDX_ERR_INVALID_ARGUMENT;
    if (scale_exp < -126 || scale_exp > 127) return DSAIDX_ERR_INVALID_ARGUMENT;
    if (n == 0) return DSAIDX_OK;
    int64_t grid = ceil_div(ceil_div(n, 8), 256);
    if (grid > max_grid(256)) grid = max_grid(256);
    return to_status(dsaidx::launch_fp8_selftest(in, out, n, std::ldexp(1.0f, scale_exp),
                                                 (unsigned)grid,
                                                 reinterpret_cast<hipStream_t>(stream)));
}

dsaidx_status dsaidx_hbm_stream(int32_t mode, const void* src, void* dst, int64_t bytes,
                                uint32_t word, dsaidx_stream_t stream) {
    if (mode != DSAIDX_HBM_COPY && mode != DSAIDX_HBM_READ && mode != DSAIDX_HBM_WRITE)
        return DSAIDX_ERR_INVALID_ARGUMENT;
    if (bytes < 0 || bytes % 16 != 0 || bytes > (int64_t(1) << 38)) return DSAIDX_ERR_INVALID_ARGUMENT;
    if (bytes == 0) return DSAIDX_OK;
    if (!dst || !aligned(dst, 16)) return DSAIDX_ERR_INVALID_ARGUMENT;
    if (mode != DSAIDX_HBM_WRITE && (!src || !aligned(src, 16))) return DSAIDX_ERR_INVALID_ARGUMENT;
    return to_status(dsaidx::launch_hbm_stream(mode, src, dst, bytes / 16, word,
                                               reinterpret_cast<hipStream_t>(stream)));
}

int dsaidx_device_supported(int device) {
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || device < 0 || device >= count) return 0;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess) return 0;
    return std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
}

const char* dsaidx_status_string(dsaidx_status status) {
    switch (status) {
        case DSAIDX_OK: return "DSAIDX_OK";
        case DSAIDX_ERR_INVALID_ARGUMENT: return "DSAIDX_ERR_INVALID_ARGUMENT";
        case DSAIDX_ERR_UNSUPPORTED: return "DSAIDX_ERR_UNSUPPORTED";
        case DSAIDX_ERR_HIP: return "DSAIDX_ERR_HIP";
    }
    return "DSAIDX_UNKNOWN_STATUS";
}

int dsaidx_abi_version(void) { return DSAIDX_ABI_VERSION; }

size_t dsaidx_struct_size(int which) {
    switch (which) {
        case 0: return sizeof(dsaidx_rope);
        case 1: return sizeof(dsaidx_q_args);
        case 2: return sizeof(dsaidx_k_args);
        case 3: return sizeof(dsaidx_logits_args);
        case 4: return sizeof(dsaidx_proj_args);
    }
    return 0;
}

}  // extern "C"
