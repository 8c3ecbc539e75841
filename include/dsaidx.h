/*
 * libdsaidx — DSA-indexer Q/K preparation on MI355X (gfx950).
 *
 * The DeepSeek-Sparse-Attention indexer prepares its query and key before
 * scoring.  Query side, per (token t, head h): RoPE on the rope slice of the
 * 128-wide head vector, quantisation of the vector to FP8 E4M3FN with one
 * power-of-two (ue8m0) scale, and the scale folded into the head-gate weight.
 * Key side, per token: fp32 LayerNorm with fp32 affine parameters, the same
 * RoPE and quantisation, and a scatter of the fp8 row and its scale into the
 * slot-indexed index-K cache at out_cache_loc[t].
 *
 * Sources (page title and section):
 *   [sglang-fuse] sglang PR "[AMD] [GLM5] Fuse the DSA indexer Q/K rope + quant
 *     + K-cache write": Motivation (the operations and their single-launch
 *     fusion), Modifications (the (q_fp8, weights) result sliced to num_tokens,
 *     fp32 norm parameters, separate cos/sin tables, the k-only store path, the
 *     sliced out_cache_loc), Accuracy (ue8m0 scales, one fp32 -> fp8 step),
 *     Profile (one launch instead of four), Checklist (strided inputs, a
 *     replaced rope table, both cache writers).
 *   [vllm-47335] vLLM PR 47335 "[ROCm][Perf] Enable fused indexer-Q RoPE+quant
 *     kernel for DeepSeek/GLM sparse attention": Summary (query RoPE + FP8
 *     quantisation + weight-scale fold in one launch), Kernel-level evidence.
 *
 * Numerics (every entry point, bit for bit the same per row):
 *   x          = fp32(bf16 input)                       (exact)
 *   K only:    mu = fp32(sum x / 128), var = fp32(sum (x - mu)^2 / 128)
 *              with fp64 sums, r = fp32(1 / sqrt(fp64 var + fp64 eps)),
 *              n_i = ((x_i - mu) * r) * gamma_i + beta_i  (each op rounded)
 *   RoPE       pair (a, b) -> (a*c - b*s, b*c + a*s) with c, s = cos/sin of
 *              table row positions[t], column i for pair i < rope_dim/2;
 *              NeoX pairs (i, i + rope_dim/2), interleaved pairs (2i, 2i+1);
 *              elements >= rope_dim pass through.  No fused multiply-add.
 *   scale      e = smallest integer with max(amax, 1e-4) <= 448 * 2^e, where
 *              amax = max |y| over the 128 values (1e-4 is the zero-row guard)
 *   codes      E4M3FN(y * 2^-e), round to nearest even; |y * 2^-e| <= 448 by
 *              construction, so no value saturates
 *   Q extra    weights_out = (fp32(w) * weight_scale) * 2^e; q_scale_out = 2^e
 *   K extra    k_cache[slot][0..127] = codes, k_scale[slot] = 2^e
 *
 * Ownership and execution: every pointer is caller-owned DEVICE memory except
 * the argument structs themselves (host memory, read during the call only).
 * The library allocates nothing, keeps no per-call state and caches no data,
 * so a replaced or rewritten rope table is always honoured.  Work is enqueued
 * asynchronously on `stream` (a hipStream_t; NULL = the null stream of the
 * current device) as exactly one kernel dispatch per call, with no host
 * synchronisation, no device-to-host reads and no memsets, so calls can be
 * captured in a HIP graph.  Calls are reentrant and thread-safe.
 *
 * Errors: all arguments are checked on the host before anything is enqueued;
 * a failed check returns DSAIDX_ERR_INVALID_ARGUMENT and enqueues nothing.
 * num_tokens == 0 (on both sides for the fused call) returns DSAIDX_OK without
 * a launch and without looking at the pointers, since graph split-op slices
 * may be empty and empty tensors may have NULL data pointers.  A launch the HIP runtime rejects returns
 * DSAIDX_ERR_UNSUPPORTED (no gfx950 device / no code object for it) or
 * DSAIDX_ERR_HIP.  Kernel execution errors surface on the stream as usual.
 *
 * Preconditions that are not checked (device data is never read on the host):
 *   - positions[t] in [0, max_position).  A position outside is clamped to the
 *     table for the read, so no access leaves the table; the output of that
 *     token is then unspecified.
 *   - out_cache_loc entries are distinct (repeated slots race).  Entries < 0 or
 *     >= num_slots are skipped: nothing is written for that token.
 *   - inputs are finite with |x| < 2^100; outputs do not overlap inputs or
 *     each other.
 */
#ifndef DSAIDX_H
#define DSAIDX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSAIDX_ABI_VERSION 6
#define DSAIDX_HEAD_DIM 128 /* width of every head vector and K row */

typedef struct ihipStream_t* dsaidx_stream_t; /* the same type as hipStream_t */

typedef enum dsaidx_status {
    DSAIDX_OK = 0,
    DSAIDX_ERR_INVALID_ARGUMENT = 1,
    DSAIDX_ERR_UNSUPPORTED = 2,
    DSAIDX_ERR_HIP = 3
} dsaidx_status;

typedef enum dsaidx_rope_style {
    DSAIDX_ROPE_NEOX = 0,       /* pairs (i, i + rope_dim/2) */
    DSAIDX_ROPE_INTERLEAVED = 1 /* pairs (2i, 2i + 1) */
} dsaidx_rope_style;

/* RoPE tables, read by token position ([sglang-fuse] Modifications: cos and
 * sin are kept as two tables of rope_dim/2 columns).  Row p of the cosine
 * table starts at cos + p * row_stride; likewise sin.  A single combined
 * cos_sin cache of [P, rope_dim] floats is passed as cos = cache,
 * sin = cache + rope_dim/2, row_stride = rope_dim.
 *   cos, sin      fp32, 4-byte aligned
 *   row_stride    floats between rows; >= rope_dim/2
 *   max_position  number of table rows P >= 1
 *   rope_dim      rotated leading dims; even, in [2, 128]
 *   style         dsaidx_rope_style
 * The kernels' vectorised rope paths serve rope_dim a multiple of 16 with
 * 16-byte aligned tables and a row_stride that is a multiple of 4; every
 * other valid table takes an element-wise path with the same results. */
typedef struct dsaidx_rope {
    const float* cos;
    const float* sin;
    int64_t row_stride;
    int64_t max_position;
    int32_t rope_dim;
    int32_t style;
} dsaidx_rope;

/* Query side ([sglang-fuse] Modifications: the (q_fp8, weights) result;
 * [vllm-47335] Summary).  Strides are in elements.
 *   q            bf16 bits [T, H, 128]: (t, h, i) at q[t*q_stride_t + h*q_stride_h + i];
 *                16-byte aligned; q_stride_h >= 128 and q_stride_t >= (H-1)*q_stride_h + 128,
 *                both multiples of 8 (padded head strides are allowed)
 *   weights      bf16 bits head gates [T, H]: (t, h) at weights[t*w_stride_t + h];
 *                w_stride_t >= H (a column slice of a wider GEMM output is allowed)
 *   positions    int64 [T], 8-byte aligned
 *   num_tokens   T >= 0
 *   num_heads    H in [1, 4096]
 *   weight_scale finite constant folded into every gate (1.0 for none)
 *   q_fp8        out: E4M3FN [T, H, 128] contiguous, 8-byte aligned
 *   weights_out  out: fp32 [T, H] contiguous, 4-byte aligned
 *   q_scale_out  out: fp32 [T, H] contiguous (2^e per row), or NULL */
typedef struct dsaidx_q_args {
    const uint16_t* q;
    int64_t q_stride_t;
    int64_t q_stride_h;
    const uint16_t* weights;
    int64_t w_stride_t;
    const int64_t* positions;
    int64_t num_tokens;
    int32_t num_heads;
    float weight_scale;
    uint8_t* q_fp8;
    float* weights_out;
    float* q_scale_out;
} dsaidx_q_args;

/* dsaidx_k_args.flags bits.
 *
 * [sglang-fuse] Accuracy compares the fused K-cache writer (fp32 -> fp8 in one
 * step, the default here) with the unfused one, which rounds to bf16 before
 * quantising; the page does not say at which points.  Two readings:
 *
 * DSAIDX_K_BF16_ROUND_ONCE: the finished fp32 LayerNorm + RoPE value is
 *   rounded to bf16 (nearest, ties to even) once, just before quantisation.
 *   A bf16 rounding moves a value by at most 2^-9 of itself, less than half an
 *   fp8 step, so codes differ from the default writer by at most one step
 *   wherever the two scales agree; the scale drops one step only on a row
 *   whose fp32 max lies just above 448 * 2^e and rounds onto it.  This is
 *   the reading under which the page's observation (identical scales, codes
 *   one step apart, the fused writer closer to fp32) holds by construction.
 *
 * DSAIDX_K_BF16_INTERMEDIATE: the LayerNorm output and the RoPE output are
 *   each rounded to bf16 (the two kernel boundaries of the unfused chain).
 *   The rounding of the rotation's inputs can move a value by more than one
 *   fp8 step where the rotation cancels (a*c close to b*s).
 *
 * At most one of the two bf16 bits may be set.
 *
 * DSAIDX_K_PAGED_CACHE: the page-interleaved index-K cache ([sglang-fuse]
 *   Checklist tests two paged layouts without defining them; this is the
 *   second one).  k_cache holds num_slots / page_size pages of
 *   page_size * 132 bytes: the page_size 128-byte code rows first, then the
 *   page_size fp32 scales.  Slot s lives in page s / page_size at offset
 *   o = s % page_size: codes at page + 128 * o, scale at
 *   page + 128 * page_size + 4 * o.  k_cache_row_stride and k_scale are unused
 *   (k_scale may be NULL). */
#define DSAIDX_K_BF16_INTERMEDIATE 0x1
#define DSAIDX_K_PAGED_CACHE 0x2
#define DSAIDX_K_BF16_ROUND_ONCE 0x4

/* Key side ([sglang-fuse] Motivation and Modifications: fp32 LayerNorm with
 * fp32 params, the index-K cache write at the sliced out_cache_loc).
 *   k                  bf16 bits [T, 128]: row t at k + t*k_stride_t; 16-byte aligned;
 *                      k_stride_t >= 128 and a multiple of 8 (a column slice of a
 *                      wider GEMM output is allowed)
 *   ln_gamma, ln_beta  fp32 [128], 16-byte aligned
 *   ln_eps             > 0, finite
 *   flags              0, or DSAIDX_K_PAGED_CACHE and at most one of
 *                      DSAIDX_K_BF16_INTERMEDIATE, DSAIDX_K_BF16_ROUND_ONCE
 *   positions          int64 [T], 8-byte aligned
 *   out_cache_loc      int64 [T] slot per token, 8-byte aligned
 *   num_tokens         T >= 0
 *   k_cache            in/out: E4M3FN rows; slot s at k_cache + s*k_cache_row_stride,
 *                      codes in its first 128 bytes (planar layout), or the pages of
 *                      DSAIDX_K_PAGED_CACHE; 8-byte aligned
 *   k_cache_row_stride planar: bytes, >= 128 and a multiple of 8
 *   k_scale            planar: in/out fp32 [num_slots], 4-byte aligned
 *   num_slots          S >= 1 (paged: a multiple of page_size)
 *   page_size          paged: slots per page, even, in [2, 2^20]; ignored otherwise */
typedef struct dsaidx_k_args {
    const uint16_t* k;
    int64_t k_stride_t;
    const float* ln_gamma;
    const float* ln_beta;
    float ln_eps;
    int32_t flags;
    const int64_t* positions;
    const int64_t* out_cache_loc;
    int64_t num_tokens;
    uint8_t* k_cache;
    int64_t k_cache_row_stride;
    float* k_scale;
    int64_t num_slots;
    int64_t page_size;
} dsaidx_k_args;

/* Query RoPE + fp8/ue8m0 quantisation + head-gate fold: the fused-Q launch of
 * [vllm-47335] Summary.  One dispatch over the T*H head vectors. */
dsaidx_status dsaidx_q_rope_quant_fold(const dsaidx_q_args* q, const dsaidx_rope* rope,
                                       dsaidx_stream_t stream);

/* Key LayerNorm + RoPE + quantisation + index-K cache store: the key half of
 * the fused-Q tier, where the key path stays a launch of its own
 * ([vllm-47335] Kernel-level evidence).  One dispatch over the T key rows. */
dsaidx_status dsaidx_k_norm_rope_quant_store(const dsaidx_k_args* k, const dsaidx_rope* rope,
                                             dsaidx_stream_t stream);

/* The whole Q and K preparation in ONE dispatch ([sglang-fuse] Motivation and
 * Profile: four launches per layer become one).  q->num_tokens must equal
 * k->num_tokens; Q rows read q->positions and K rows k->positions (normally
 * the same array).  Outputs are byte-identical to dsaidx_q_rope_quant_fold
 * followed by dsaidx_k_norm_rope_quant_store. */
dsaidx_status dsaidx_qk_fused(const dsaidx_q_args* q, const dsaidx_k_args* k,
                              const dsaidx_rope* rope, dsaidx_stream_t stream);

/* K-only prepare-and-store for the dense decode fast path that skips the
 * indexer while the KV length is within index_topk ([sglang-fuse]
 * Modifications and Benchmark).  Same arithmetic and bytes as
 * dsaidx_k_norm_rope_quant_store; a launch shape for few tokens. */
dsaidx_status dsaidx_k_only_prepare_store(const dsaidx_k_args* k, const dsaidx_rope* rope,
                                          dsaidx_stream_t stream);

/* The indexer's key and head-gate projection with the key preparation in its
 * epilogue: the fused wk_weights_proj GEMM of [sglang-fuse] Motivation, whose
 * bf16 output the unfused path writes and the preparation reads back.
 *   out[t, n] = bf16( sum_c hidden[t, c] * weight[n, c] )   (fp32 accumulation)
 *   n < 128:      the key row of token t, prepared exactly as
 *                 dsaidx_k_norm_rope_quant_store prepares a k of these bf16
 *                 values (LayerNorm, RoPE, quantisation, cache store);
 *   128 <= n < 128 + H:  the head gate of head n - 128, written to gates_out
 *                 (the weights input of dsaidx_q_rope_quant_fold).
 * The products are exact in fp32 and the sums are fp32 in an order the
 * library chooses; the bf16 rounding is to nearest even.
 *   hidden         bf16 [T, d]: token t at hidden + t * hidden_stride_t; 16-byte
 *                  aligned; hidden_stride_t >= d, a multiple of 8, at most 2^22
 *   weight         bf16 [128 + H, d] (a Linear layer's [out, in] layout): row n
 *                  at weight + n * weight_stride_n; 16-byte aligned;
 *                  weight_stride_n >= d, a multiple of 8, at most 2^22
 *   hidden_dim     d: a multiple of 64 in [64, 2^20]
 *   num_heads      H in [1, 64]
 *   gates_out      out: bf16 [T, H], token stride gates_stride_t >= H; 2-byte aligned
 *   k_out          out: bf16 [T, 128] (token stride k_out_stride_t >= 128, a
 *                  multiple of 8; 16-byte aligned), or NULL: the projected key as
 *                  the GEMM would write it
 * The key side comes from `k` as for dsaidx_k_norm_rope_quant_store, except
 * that k->k and k->k_stride_t are not used (the key comes from the
 * projection): num_tokens, LayerNorm parameters, positions, out_cache_loc,
 * cache and flags.  One dispatch; T == 0 launches nothing. */
typedef struct dsaidx_proj_args {
    const uint16_t* hidden;
    int64_t hidden_stride_t;
    const uint16_t* weight;
    int64_t weight_stride_n;
    int64_t hidden_dim;
    int32_t num_heads;
    int32_t reserved;   /* 0 */
    uint16_t* gates_out;
    int64_t gates_stride_t;
    uint16_t* k_out;
    int64_t k_out_stride_t;
} dsaidx_proj_args;

dsaidx_status dsaidx_proj_k_norm_rope_quant_store(const dsaidx_proj_args* proj,
                                                  const dsaidx_k_args* k, const dsaidx_rope* rope,
                                                  dsaidx_stream_t stream);

/* Top-k per row: the selection that follows the index logits, each query
 * keeping its index_topk highest-scoring keys ([sglang-fuse] Benchmark:
 * index_topk = 2048; [vllm-47335] Kernel-level evidence: the top-k-per-row
 * decode launch after the paged MQA logits).
 *   logits     fp32 [rows, row_stride] (device), 16-byte aligned; the buffer holds
 *              rows * row_stride floats; row r is valid over [0, len_r) with
 *              len_r = min(max(lengths[r], 0), cols) (lengths NULL: len_r = cols)
 *   row_stride floats between rows, >= cols and a multiple of 4
 *   lengths    int32 [rows] (device) or NULL
 *   rows       >= 0 and < 2^31;  cols in [0, 2^31);  k in [1, 2^20]
 *   out_idx    out: int32 [rows, k] (device), 4-byte aligned.  When len_r > k: the
 *              indices of the k largest valid logits, in no particular order; when
 *              several logits equal the k-th largest, which of them are taken is
 *              not specified (the multiset of selected values is).  When
 *              len_r <= k: 0, 1, ..., len_r - 1, then -1.
 *   workspace  device scratch of at least dsaidx_topk_workspace_bytes(rows, cols, k)
 *              bytes, 16-byte aligned, owned by the caller; its contents on entry
 *              do not matter and are overwritten.  May be NULL when that size is 0.
 *   workspace_bytes  its size.
 * Logits must not be NaN.  One dispatch for rows of up to 32768 logits; four
 * for longer rows (the row spread over workgroups of 4096 logits, with the row's
 * histogram, counters and candidate list in the workspace); no allocation.
 * Calls that share a workspace must be ordered on one stream.  A workspace that
 * is required but NULL, misaligned or too small is DSAIDX_ERR_INVALID_ARGUMENT. */
dsaidx_status dsaidx_topk_per_row(const float* logits, int64_t row_stride, const int32_t* lengths,
                                  int64_t rows, int64_t cols, int32_t k, int32_t* out_idx,
                                  void* workspace, int64_t workspace_bytes,
                                  dsaidx_stream_t stream);

/* Top-k per row for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * arguments and result as dsaidx_topk_per_row, without the workspace: a call
 * that needs one (rows longer than 32768 logits) uses a library-owned device
 * array of DSAIDX_TOPK_NOALLOC_SCRATCH_BYTES (16 MiB) on the current GPU,
 * part of the library's code object (each GPU the library runs on holds its
 * own until the process ends).  The call allocates nothing.
 *   - A call whose dsaidx_topk_workspace_bytes exceeds that size (e.g. more
 *     than 227 rows of 131072 logits) returns DSAIDX_ERR_INVALID_ARGUMENT and
 *     enqueues nothing.
 *   - `stream` must belong to the current device (else
 *     DSAIDX_ERR_INVALID_ARGUMENT).  Devices 0..63 are supported.
 *   - Every call on one GPU shares that GPU's array, which keeps the last
 *     call's contents; the kernels clear what they need, so those contents
 *     do not matter.  Calls that overlap on one GPU (on different streams, or
 *     from several host threads) race on the array: order them on one stream.
 */
#define DSAIDX_TOPK_NOALLOC_SCRATCH_BYTES ((int64_t)16 << 20)
dsaidx_status dsaidx_topk_per_row_noalloc(const float* logits, int64_t row_stride,
                                          const int32_t* lengths, int64_t rows, int64_t cols,
                                          int32_t k, int32_t* out_idx, dsaidx_stream_t stream);

/* Bytes of workspace dsaidx_topk_per_row needs for this shape: 0 when
 * cols <= 32768, else rows * (8224 + 8 * L) with L = max(4096, cols / 16)
 * rounded up to a multiple of 4 (per row: a 2048-bin histogram and counters,
 * and a list of up to L candidate keys and indices; rows whose threshold bin
 * holds more are finished by re-reading the row); -1 for a
 * shape dsaidx_topk_per_row rejects
 * (including rows * ceil(cols / 4096) >= 2^31 when cols > 32768). */
int64_t dsaidx_topk_workspace_bytes(int64_t rows, int64_t cols, int32_t k);

/* Index logits: the step that consumes the prepared query and the index-K
 * cache, between the indexer prep and the top-k (the fp8 paged MQA-logits
 * launch of [vllm-47335] Kernel-level evidence).  The pages name the step but
 * do not write out its arithmetic; the reading taken is the one under which
 * folding each head's query scale into its gate is exact -- a ReLU on each
 * head's dot (it commutes with a positive factor), then a gate-weighted sum
 * over the heads:
 *   logits[t * logits_stride + s] =
 *       kscale(slot) * sum_h weights[t * H + h] * max(0, sum_d q(t, h, d) * k(slot, d))
 * with q(t, h, d) the E4M3FN value of q_fp8[(t * H + h) * 128 + d], k(slot, d)
 * the value of code d of the slot's cache row, kscale(slot) its scale, and
 * slot = key_slots ? key_slots[s] : s.  Products are exact in fp32; the
 * 128-term sums and the head sum are fp32, in an order the library chooses.
 *   q_fp8          E4M3FN codes [T, H, 128], contiguous (the prep call's q_fp8), 16-byte aligned
 *   weights        fp32 [T, H], contiguous (the prep call's weights_out), 4-byte aligned
 *   num_tokens     T in [0, 2^31)
 *   num_heads      H in [1, 64]
 *   flags          0, or DSAIDX_K_PAGED_CACHE for the page-interleaved layout
 *   k_cache, k_cache_row_stride, k_scale, num_slots, page_size
 *                  the index-K cache, read only, as in dsaidx_k_args
 *   key_slots      int32 [num_keys]: the cache slot of each key (a page table's
 *                  flattening), 4-byte aligned; NULL: key s is slot s, and then
 *                  num_keys <= num_slots.  A slot outside [0, num_slots) is
 *                  never addressed (slot 0's row is read in its place and
 *                  discarded) and its logit is 0
 *   num_keys       N in [0, 2^31)
 *   lengths        int32 [T], 4-byte aligned: query t scores keys
 *                  [0, min(max(lengths[t], 0), N)); NULL: all N
 *   logits         out fp32: row t at logits + t * logits_stride, 4-byte aligned;
 *                  entries past a row's length are not written
 *   logits_stride  floats, >= N
 * T == 0 or N == 0 returns DSAIDX_OK with no launch.  One dispatch. */
typedef struct dsaidx_logits_args {
    const uint8_t* q_fp8;
    const float* weights;
    int64_t num_tokens;
    int32_t num_heads;
    int32_t flags;
    const uint8_t* k_cache;
    int64_t k_cache_row_stride;
    const float* k_scale;
    int64_t num_slots;
    int64_t page_size;
    const int32_t* key_slots;
    int64_t num_keys;
    const int32_t* lengths;
    float* logits;
    int64_t logits_stride;
} dsaidx_logits_args;

dsaidx_status dsaidx_mqa_logits(const dsaidx_logits_args* args, dsaidx_stream_t stream);

/* Encode n fp32 values to E4M3FN bytes with the device conversion every
 * kernel above uses, so the conversion can be checked on its own against the
 * format definition: out[i] = E4M3FN(in[i] / 2^scale_exp), rounded to nearest
 * even, the division by the power of two exact -- the same call the kernels
 * make with a row's ue8m0 scale.  in: device fp32 [n], 4-byte aligned, every
 * in[i] / 2^scale_exp in [-448, 448] (values outside are outside the
 * contract); out: device bytes [n], 8-byte aligned; n >= 0; scale_exp in
 * [-126, 127] (2^scale_exp a normal fp32).  One dispatch. */
dsaidx_status dsaidx_fp8_encode_selftest(const float* in, uint8_t* out, int64_t n,
                                         int32_t scale_exp, dsaidx_stream_t stream);

/* Reference HBM streams: a measurement helper, not part of the indexer path.
 * Plain kernels with the preparation kernel's access pattern (16-byte
 * nontemporal loads and stores by every lane, a one-shot grid of 256-thread
 * workgroups) that give the bandwidth a copy, a pure read and a pure write of
 * `bytes` reach on this device, so that a kernel's achieved bandwidth can be
 * set against what its own mix of reads and writes can reach, beside the
 * published peak.
 *   mode   DSAIDX_HBM_COPY: dst[0, bytes) = src[0, bytes)
 *          DSAIDX_HBM_READ: reads src[0, bytes); dst is a sink of at least 16
 *            bytes that is written only if the data fold to `word` (an XOR of
 *            all 32-bit words per thread), so pass a `word` they cannot fold to
 *          DSAIDX_HBM_WRITE: dst[0, bytes) = `word` repeated; src unused
 *   src, dst  device, 16-byte aligned, not overlapping
 *   bytes  >= 0, a multiple of 16, at most 2^38
 * One dispatch (none for bytes == 0). */
#define DSAIDX_HBM_COPY 0
#define DSAIDX_HBM_READ 1
#define DSAIDX_HBM_WRITE 2
dsaidx_status dsaidx_hbm_stream(int32_t mode, const void* src, void* dst, int64_t bytes,
                                uint32_t word, dsaidx_stream_t stream);

/* 1 if `device` is a gfx950 GPU this library has code for, else 0 (also when
 * no GPU or HIP runtime is present).  The counterpart of the import-time
 * kernel probe of [sglang-fuse] Modifications. */
int dsaidx_device_supported(int device);

/* Static, never-NULL description of a status code. */
const char* dsaidx_status_string(dsaidx_status status);

/* DSAIDX_ABI_VERSION of the built library. */
int dsaidx_abi_version(void);

/* sizeof the argument structs as built (0 = dsaidx_rope, 1 = dsaidx_q_args,
 * 2 = dsaidx_k_args, 3 = dsaidx_logits_args, 4 = dsaidx_proj_args; anything
 * else returns 0), for binding checks. */
size_t dsaidx_struct_size(int which);

#ifdef __cplusplus
}
#endif
#endif /* DSAIDX_H */
