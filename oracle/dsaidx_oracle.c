/*
 * CPU oracle for the DSA-indexer Q/K preparation — TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously-correct reference of what the GPU path computes.
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load it; the product library never does, and the two share no code.
 *
 * What is computed (the unfused composition the pages compare the fused kernel
 * against, done in fp32 with one fp32 -> fp8 step):
 *   Q row (t,h): RoPE on the rope slice with cos/sin read at positions[t]
 *     -> per-row fp8 E4M3FN quantisation with a power-of-two (ue8m0) scale
 *     -> the scale folded into the head-gate weight.
 *     [sglang-fuse] Motivation (rope on q and k, fp8 quant of each, head-gate
 *     scale); [vllm-47335] Summary (query RoPE + FP8 quant + weight-scale fold)
 *     and Kernel-level evidence (q -> FP8 ue8m0 quant, weights scale-fold).
 *   K row t: fp32 LayerNorm with fp32 affine params -> RoPE -> the same
 *     quantisation -> fp8 row and scale written to the index-K cache at
 *     out_cache_loc[t].  [sglang-fuse] Motivation (LayerNorm on k, index-K
 *     cache write), Modifications (fp32 norm params; the sliced out_cache_loc).
 *   bf16_mode reproduces the other K-cache writer of [sglang-fuse] Accuracy
 *     (rounds to bf16 before quantising, where the fused one goes fp32 -> fp8
 *     in one step).  Two readings of where it rounds: mode 1 at both kernel
 *     boundaries of the unfused chain (after LayerNorm, after RoPE); mode 2
 *     once, on the finished fp32 LayerNorm + RoPE value, just before the
 *     quantisation.
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes of the repository):
 *   - rope slice = dims [0, R); NeoX pairs (i, i+R/2), interleaved pairs
 *     (2i, 2i+1), both rotated by angle index i < R/2; cos/sin are inputs.
 *   - LayerNorm: biased variance, eps inside the square root, two passes;
 *     sums accumulated in fp64, mean / variance / 1/sqrt rounded to fp32.
 *   - scale exponent e = smallest integer with max(amax, 1e-4) <= 448 * 2^e
 *     (the 1e-4 floor is the zero-row guard); the row is multiplied by 2^-e
 *     before encoding and the stored scale is 2^e.
 *   - folded weight = (fp32(w) * weight_scale) * 2^e, in that order.
 *   - cache slots outside [0, S) are skipped.
 */
#include "dsaidx_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ROW 128           /* elements per head vector / K row */
#define FP8_MAX 448.0     /* largest finite E4M3FN value */
#define AMAX_FLOOR 1e-4f  /* zero-row guard on the row max */

static int nthreads_or_default(int nthreads) {
#ifdef _OPENMP
    return nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

int oracle_max_threads(void) { return nthreads_or_default(0); }

/* bf16 -> fp32 is exact: the bf16 bits are the top half of the fp32 word. */
static float bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* fp32 -> nearest bf16 (ties to even), returned as fp32.  Finite inputs only. */
static float round_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    u &= 0xFFFF0000u;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* ---------------------------------------------------------------- fp8 ---- */

/* OCP FP8 E4M3FN from the format definition: sign bit, 4-bit exponent with
 * bias 7, 3-bit mantissa; exponent field 0 holds subnormals m/8 * 2^-6; the
 * all-ones pattern (exponent 15, mantissa 7) is NaN and there is no infinity,
 * so the largest finite value is 1.75 * 2^8 = 448. */
uint8_t oracle_fp8_encode(float v) {
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    if (isnan(v)) return (uint8_t)(sign | 0x7F);
    double a = fabs((double)v);
    if (a >= FP8_MAX) return (uint8_t)(sign | 0x7E); /* saturate */

    /* Spacing of representable values around a: 2^(E-3) in the binade
     * [2^E, 2^(E+1)) for E >= -6, and 2^-9 in the subnormal range. */
    int E;
    (void)frexp(a, &E); /* a = f * 2^E with f in [0.5, 1) */
    E -= 1;             /* now a in [2^E, 2^(E+1)) */
    double quantum = (a == 0.0 || E < -6) ? ldexp(1.0, -9) : ldexp(1.0, E - 3);
    double q = nearbyint(a / quantum); /* exact division; default mode is ties-to-even */
    double val = q * quantum;          /* nearest representable magnitude */
    if (val == 0.0) return sign;
    if (val > FP8_MAX) val = FP8_MAX;  /* unreachable for a < 448, kept for clarity */

    (void)frexp(val, &E);
    E -= 1;
    if (E < -6) /* subnormal: val = m * 2^-9, m in 1..7 */
        return (uint8_t)(sign | (uint8_t)(val / ldexp(1.0, -9)));
    int mant = (int)(val / ldexp(1.0, E - 3)) - 8; /* val = (8 + mant) * 2^(E-3) */
    return (uint8_t)(sign | ((E + 7) << 3) | mant);
}

float oracle_fp8_decode(uint8_t code) {
    int E = (code >> 3) & 0xF;
    int M = code & 0x7;
    double val;
    if (E == 0xF && M == 0x7) return NAN;
    if (E == 0)
        val = M * ldexp(1.0, -9);
    else
        val = (8 + M) * ldexp(1.0, E - 10); /* (1 + M/8) * 2^(E-7) */
    return (float)((code & 0x80) ? -val : val);
}

void oracle_fp8_encode_array(const float* v, uint8_t* out, int64_t n, int nthreads) {
    int nt = nthreads_or_default(nthreads);
    (void)nt;
#pragma omp parallel for schedule(static) num_threads(nt)
    for (int64_t i = 0; i < n; i++) out[i] = oracle_fp8_encode(v[i]);
}

/* -------------------------------------------------------------- scale ---- */

/* The power-of-two scale is the smallest 2^e that brings the row max into the
 * fp8 range: max(amax, floor) <= 448 * 2^e.  Searched exactly in fp64, where
 * 448 * 2^e is exact for every e that can occur. */
int oracle_ue8m0_exponent(float amax) {
    float ag = (amax > AMAX_FLOOR) ? amax : AMAX_FLOOR;
    double a = (double)ag;
    if (!(a < HUGE_VAL)) return 128; /* infinite input: outside the contract */
    int e;
    (void)frexp(a / FP8_MAX, &e); /* starting guess only */
    while (a > ldexp(FP8_MAX, e)) e++;
    while (a <= ldexp(FP8_MAX, e - 1)) e--;
    return e;
}

/* --------------------------------------------------------------- rope ---- */

/* Rotate the rope slice [0, R) of a 128-vector by the angles of one table row.
 * NeoX style pairs element i with i + R/2; interleaved style pairs 2i with
 * 2i + 1.  Pair i uses c[i], s[i]:  (a, b) -> (a*c - b*s, b*c + a*s), every
 * product and sum rounded to fp32 on its own.  Elements >= R pass through. */
static void rope_row(float* x, const float* c, const float* s, int R, int style) {
    float y[ROW];
    memcpy(y, x, sizeof y);
    int half = R / 2;
    for (int i = 0; i < half; i++) {
        int ia = (style == 0) ? i : 2 * i;
        int ib = (style == 0) ? i + half : 2 * i + 1;
        float a = x[ia], b = x[ib];
        float ac = a * c[i];
        float bs = b * s[i];
        float bc = b * c[i];
        float as = a * s[i];
        y[ia] = ac - bs;
        y[ib] = bc + as;
    }
    memcpy(x, y, sizeof y);
}

/* ------------------------------------------------------------ quantise ---- */

static int row_exponent(const float* y) {
    float amax = 0.0f;
    for (int i = 0; i < ROW; i++) amax = fmaxf(amax, fabsf(y[i]));
    return oracle_ue8m0_exponent(amax);
}

static void encode_row(const float* y, int e, uint8_t* codes) {
    float inv = ldexpf(1.0f, -e); /* exact power of two */
    for (int i = 0; i < ROW; i++) codes[i] = oracle_fp8_encode(y[i] * inv);
}

/* ---------------------------------------------------------- LayerNorm ---- */

/* n_i = ((x_i - mu) * r) * gamma_i + beta_i with mu = sum(x)/128,
 * var = sum((x - mu)^2)/128 (biased, second pass over the fp32 mean) and
 * r = 1/sqrt(var + eps); sums in fp64, mu / var / r rounded to fp32. */
static void layernorm_row(const float* x, const float* g, const float* b, float eps, float* n) {
    double s1 = 0.0;
    for (int i = 0; i < ROW; i++) s1 += (double)x[i];
    float mu = (float)(s1 / ROW);
    double s2 = 0.0;
    for (int i = 0; i < ROW; i++) {
        float d = x[i] - mu;
        s2 += (double)d * (double)d;
    }
    float var = (float)(s2 / ROW);
    float r = (float)(1.0 / sqrt((double)var + (double)eps));
    for (int i = 0; i < ROW; i++) {
        float d = x[i] - mu;
        float dn = d * r;
        float dg = dn * g[i];
        n[i] = dg + b[i];
    }
}

/* ------------------------------------------------------------------ Q ---- */

int oracle_q(const uint16_t* q, int64_t q_st, int64_t q_sh,
             const uint16_t* w, int64_t w_st, const int64_t* pos,
             int64_t T, int H, float weight_scale,
             const float* cos_t, const float* sin_t, int64_t rs, int64_t P,
             int R, int style,
             uint8_t* q_fp8, float* w_out, float* q_scale, int nthreads) {
    int bad = 0;
    int nt = nthreads_or_default(nthreads);
    (void)nt;
#pragma omp parallel for schedule(static) num_threads(nt)
    for (int64_t t = 0; t < T; t++) {
        int64_t p = pos[t];
        if (p < 0 || p >= P) {
#pragma omp atomic write
            bad = 1;
            continue;
        }
        const float* c = cos_t + p * rs;
        const float* s = sin_t + p * rs;
        for (int h = 0; h < H; h++) {
            float x[ROW];
            const uint16_t* src = q + t * q_st + (int64_t)h * q_sh;
            for (int i = 0; i < ROW; i++) x[i] = bf16_to_f32(src[i]);
            rope_row(x, c, s, R, style);
            int e = row_exponent(x);
            encode_row(x, e, q_fp8 + (t * H + h) * ROW);
            float sc = ldexpf(1.0f, e);
            float wv = bf16_to_f32(w[t * w_st + h]);
            float ws = wv * weight_scale;
            w_out[t * H + h] = ws * sc;
            if (q_scale) q_scale[t * H + h] = sc;
        }
    }
    return bad ? -1 : 0;
}

/* Q side, values only: the 128 fp32 values of every row after RoPE
 * (y[(t*H + h)*128 + i]) and the row's scale exponent (e[t*H + h]). */
int oracle_q_values(const uint16_t* q, int64_t q_st, int64_t q_sh,
                    const int64_t* pos, int64_t T, int H,
                    const float* cos_t, const float* sin_t, int64_t rs, int64_t P,
                    int R, int style, float* y, int32_t* e, int nthreads) {
    int bad = 0;
    int nt = nthreads_or_default(nthreads);
    (void)nt;
#pragma omp parallel for schedule(static) num_threads(nt)
    for (int64_t t = 0; t < T; t++) {
        int64_t p = pos[t];
        if (p < 0 || p >= P) {
#pragma omp atomic write
            bad = 1;
            continue;
        }
        for (int h = 0; h < H; h++) {
            float x[ROW];
            const uint16_t* src = q + t * q_st + (int64_t)h * q_sh;
            for (int i = 0; i < ROW; i++) x[i] = bf16_to_f32(src[i]);
            rope_row(x, cos_t + p * rs, sin_t + p * rs, R, style);
            memcpy(y + (t * H + h) * ROW, x, sizeof x);
            e[t * H + h] = row_exponent(x);
        }
    }
    return bad ? -1 : 0;
}

/* ------------------------------------------------------------------ K ---- */

int oracle_k_values(const uint16_t* k, int64_t k_st,
                    const float* gamma, const float* beta, float eps,
                    const int64_t* pos, int64_t T,
                    const float* cos_t, const float* sin_t, int64_t rs, int64_t P,
                    int R, int style, int bf16_mode,
                    float* y, int32_t* e, int nthreads) {
    int bad = 0;
    int nt = nthreads_or_default(nthreads);
    (void)nt;
#pragma omp parallel for schedule(static) num_threads(nt)
    for (int64_t t = 0; t < T; t++) {
        int64_t p = pos[t];
        if (p < 0 || p >= P) {
#pragma omp atomic write
            bad = 1;
            continue;
        }
        float x[ROW], n[ROW];
        for (int i = 0; i < ROW; i++) x[i] = bf16_to_f32(k[t * k_st + i]);
        layernorm_row(x, gamma, beta, eps, n);
        if (bf16_mode == 1) /* the LayerNorm kernel's bf16 output */
            for (int i = 0; i < ROW; i++) n[i] = round_to_bf16(n[i]);
        rope_row(n, cos_t + p * rs, sin_t + p * rs, R, style);
        if (bf16_mode == 1 || bf16_mode == 2) /* bf16 handed to the quantiser */
            for (int i = 0; i < ROW; i++) n[i] = round_to_bf16(n[i]);
        memcpy(y + t * ROW, n, sizeof n);
        e[t] = row_exponent(n);
    }
    return bad ? -1 : 0;
}

int oracle_k(const uint16_t* k, int64_t k_st,
             const float* gamma, const float* beta, float eps,
             const int64_t* pos, const int64_t* loc, int64_t T,
             const float* cos_t, const float* sin_t, int64_t rs, int64_t P,
             int R, int style, int bf16_mode,
             uint8_t* k_cache, int64_t row_stride, float* k_scale, int64_t S,
             int nthreads) {
    if (T <= 0) return 0;
    float* y = (float*)malloc((size_t)T * ROW * sizeof(float));
    int32_t* e = (int32_t*)malloc((size_t)T * sizeof(int32_t));
    if (!y || !e) {
        free(y);
        free(e);
        return -2;
    }
    int rc = oracle_k_values(k, k_st, gamma, beta, eps, pos, T, cos_t, sin_t, rs, P,
                             R, style, bf16_mode, y, e, nthreads);
    if (rc == 0) {
        /* In token order, so the result is defined even for repeated slots. */
        for (int64_t t = 0; t < T; t++) {
            int64_t slot = loc[t];
            if (slot < 0 || slot >= S) continue;
            encode_row(y + t * ROW, e[t], k_cache + slot * row_stride);
            k_scale[slot] = ldexpf(1.0f, e[t]);
        }
    }
    free(y);
    free(e);
    return rc;
}

/* K side into the page-interleaved cache: num_slots / page_size pages of
 * page_size * 132 bytes, each holding its page_size 128-byte code rows and
 * then its page_size fp32 scales.  Slot s is in page s / page_size at offset
 * s % page_size.  Slots outside [0, S) are skipped. */
int oracle_k_paged(const uint16_t* k, int64_t k_st,
                   const float* gamma, const float* beta, float eps,
                   const int64_t* pos, const int64_t* loc, int64_t T,
                   const float* cos_t, const float* sin_t, int64_t rs, int64_t P,
                   int R, int style, int bf16_mode,
                   uint8_t* cache, int64_t page_size, int64_t S, int nthreads) {
    if (T <= 0) return 0;
    if (page_size <= 0 || S % page_size != 0) return -3;
    float* y = (float*)malloc((size_t)T * ROW * sizeof(float));
    int32_t* e = (int32_t*)malloc((size_t)T * sizeof(int32_t));
    if (!y || !e) {
        free(y);
        free(e);
        return -2;
    }
    int rc = oracle_k_values(k, k_st, gamma, beta, eps, pos, T, cos_t, sin_t, rs, P,
                             R, style, bf16_mode, y, e, nthreads);
    if (rc == 0) {
        const int64_t page_bytes = page_size * (ROW + (int64_t)sizeof(float));
        for (int64_t t = 0; t < T; t++) {
            int64_t slot = loc[t];
            if (slot < 0 || slot >= S) continue;
            uint8_t* page = cache + (slot / page_size) * page_bytes;
            int64_t off = slot % page_size;
            encode_row(y + t * ROW, e[t], page + off * ROW);
            float sc = ldexpf(1.0f, e[t]);
            memcpy(page + page_size * ROW + off * (int64_t)sizeof(float), &sc, sizeof sc);
        }
    }
    free(y);
    free(e);
    return rc;
}
