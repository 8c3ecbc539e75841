/*
 * CPU oracle for the DSA-indexer Q/K preparation — TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this library.  The product path (libdsaidx and its Python binding)
 * never links, imports or calls it, and shares no code with it.
 *
 * Sources (cited by page title and section):
 *   [sglang-fuse]  sglang pull request "[AMD] [GLM5] Fuse the DSA indexer Q/K
 *                  rope + quant + K-cache write" — sections Motivation,
 *                  Modifications, Accuracy (the paragraph on the two K-cache
 *                  writers), Profile, Checklist.
 *   [vllm-47335]   vLLM pull request 47335 "[ROCm][Perf] Enable fused
 *                  indexer-Q RoPE+quant kernel for DeepSeek/GLM sparse
 *                  attention" — sections Summary, Kernel-level evidence.
 *
 * Arithmetic is IEEE fp32 with every operation rounded on its own (the file is
 * compiled with -ffp-contract=off, so no fused multiply-add), except the
 * LayerNorm sums, which are accumulated in fp64 and rounded to fp32.
 */
#ifndef DSAIDX_ORACLE_H
#define DSAIDX_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Encode one fp32 value as OCP FP8 E4M3FN (bias 7, 3 mantissa bits, no
 * infinities, 0x7F/0xFF = NaN, max finite 448): clamp to [-448, 448], round to
 * nearest, ties to the even code.  The sign is kept (-0 and negative values
 * that round to zero give 0x80). */
uint8_t oracle_fp8_encode(float v);

/* Decode an E4M3FN byte to fp32 (exact). */
float oracle_fp8_decode(uint8_t code);

/* Encode n values (OpenMP over nthreads threads, 0 = library default). */
void oracle_fp8_encode_array(const float* v, uint8_t* out, int64_t n, int nthreads);

/* Power-of-two (ue8m0) scale exponent for a row whose max |value| is amax:
 * the smallest integer e with max(amax, 1e-4) <= 448 * 2^e. */
int oracle_ue8m0_exponent(float amax);

/* Q side.  q is bf16 bits, element (t,h,i) at q[t*q_st + h*q_sh + i];
 * weights bf16 bits at w[t*w_st + h]; cos/sin row p at cos[p*rs ...].
 * Outputs: q_fp8[(t*H + h)*128 + i], w_out[t*H + h], q_scale[t*H + h]
 * (q_scale may be NULL).  Returns 0, or -1 if a position is out of range. */
int oracle_q(const uint16_t* q, int64_t q_st, int64_t q_sh,
             const uint16_t* w, int64_t w_st, const int64_t* pos,
             int64_t T, int H, float weight_scale,
             const float* cos_t, const float* sin_t, int64_t rs, int64_t P,
             int R, int style,
             uint8_t* q_fp8, float* w_out, float* q_scale, int nthreads);

/* Q side, values only: y[(t*H + h)*128 + i] after RoPE, e[t*H + h] the
 * row's scale exponent.  Returns 0, or -1 if a position is out of range. */
int oracle_q_values(const uint16_t* q, int64_t q_st, int64_t q_sh,
                    const int64_t* pos, int64_t T, int H,
                    const float* cos_t, const float* sin_t, int64_t rs, int64_t P,
                    int R, int style, float* y, int32_t* e, int nthreads);

/* K side, values only: for each token t the 128 fp32 values after LayerNorm
 * and RoPE (y[t*128 + i]) and the ue8m0 exponent of the row (e[t]).
 * bf16_mode = 0: fp32 throughout (one fp32 -> fp8 step).
 * bf16_mode = 1: the unfused writer read as rounding to bf16 after LayerNorm
 * and again after RoPE, before quantizing.
 * bf16_mode = 2: the unfused writer read as one bf16 rounding of the finished
 * fp32 LayerNorm + RoPE value, just before quantizing.
 * Returns 0, or -1 on a bad position. */
int oracle_k_values(const uint16_t* k, int64_t k_st,
                    const float* gamma, const float* beta, float eps,
                    const int64_t* pos, int64_t T,
                    const float* cos_t, const float* sin_t, int64_t rs, int64_t P,
                    int R, int style, int bf16_mode,
                    float* y, int32_t* e, int nthreads);

/* K side, full: values as above, then the fp8 row and the fp32 scale 2^e are
 * written to k_cache[slot*row_stride + i] and k_scale[slot] for
 * slot = loc[t] when 0 <= slot < S; nothing else is written. */
int oracle_k(const uint16_t* k, int64_t k_st,
             const float* gamma, const float* beta, float eps,
             const int64_t* pos, const int64_t* loc, int64_t T,
             const float* cos_t, const float* sin_t, int64_t rs, int64_t P,
             int R, int style, int bf16_mode,
             uint8_t* k_cache, int64_t row_stride, float* k_scale, int64_t S,
             int nthreads);

/* K side into the page-interleaved cache: num_slots / page_size pages of
 * page_size * 132 bytes -- the page's page_size 128-byte code rows, then its
 * page_size fp32 scales.  Slot s: page s / page_size, offset s % page_size.
 * Returns 0, -1 on a bad position, -3 if page_size does not divide S. */
int oracle_k_paged(const uint16_t* k, int64_t k_st,
                   const float* gamma, const float* beta, float eps,
                   const int64_t* pos, const int64_t* loc, int64_t T,
                   const float* cos_t, const float* sin_t, int64_t rs, int64_t P,
                   int R, int style, int bf16_mode,
                   uint8_t* cache, int64_t page_size, int64_t S, int nthreads);

/* Number of OpenMP threads a parallel region would use (for reporting). */
int oracle_max_threads(void);

#ifdef __cplusplus
}
#endif
#endif
