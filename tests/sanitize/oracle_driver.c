/* Runs every oracle entry point under AddressSanitizer and
 * UndefinedBehaviorSanitizer on exactly sized buffers (any read or write past
 * an end is reported), across rope styles and widths, padded strides, both
 * cache layouts, both writer modes and thread counts.  Inputs come from a
 * plain linear congruential generator.  Exit status 0 when every call
 * returns what its contract says. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "dsaidx_oracle.h"

static int g_errors = 0;
#define CHECK(c)                                                                 \
    do {                                                                         \
        if (!(c)) {                                                              \
            fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #c);       \
            ++g_errors;                                                          \
        }                                                                        \
    } while (0)

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) {
    g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(g_state >> 33);
}
static float next_float(void) { return ((float)(next_u32() & 0xFFFFFF) / 16777216.0f - 0.5f) * 8.0f; }
static uint16_t next_bf16(void) {
    float f = next_float();
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

static void* xmalloc(size_t n) {
    void* p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static void fp8_checks(void) {
    for (int c = 0; c < 256; ++c) {
        const float v = oracle_fp8_decode((uint8_t)c);
        if ((c & 0x7F) != 0x7F) CHECK((oracle_fp8_encode(v) & 0x7F) == (c & 0x7F));
    }
    const int64_t n = 4099;
    float* v = xmalloc(n * sizeof(float));
    uint8_t* out = xmalloc(n);
    for (int64_t i = 0; i < n; ++i) v[i] = next_float() * 100.0f;
    oracle_fp8_encode_array(v, out, n, 2);
    for (int64_t i = 0; i < n; ++i) CHECK(out[i] == oracle_fp8_encode(v[i]));
    oracle_fp8_encode_array(v, out, 0, 1);
    free(v);
    free(out);
    CHECK(oracle_ue8m0_exponent(448.0f) == 0);
    CHECK(oracle_ue8m0_exponent(0.0f) == -22);
    CHECK(oracle_max_threads() >= 1);
}

/* One shape through every Q and K entry. */
static void run_shape(int64_t T, int H, int R, int style, int64_t q_pad, int nthreads) {
    const int64_t q_sh = 128 + q_pad, q_st = H * q_sh + 8, w_st = H + 3, k_st = 136;
    const int64_t P = 64, rs = R / 2 + 4, S = 256, row_stride = 136, page = 32;
    const int64_t nq = T ? (T - 1) * q_st + (H - 1) * q_sh + 128 : 0;
    const int64_t nw = T ? (T - 1) * w_st + H : 0;
    const int64_t nk = T ? (T - 1) * k_st + 128 : 0;
    const int64_t ntab = (P - 1) * rs + R / 2;
    uint16_t* q = xmalloc(nq * 2);
    uint16_t* w = xmalloc(nw * 2);
    uint16_t* k = xmalloc(nk * 2);
    float* cos_t = xmalloc(ntab * 4);
    float* sin_t = xmalloc(ntab * 4);
    float* gamma = xmalloc(128 * 4);
    float* beta = xmalloc(128 * 4);
    int64_t* pos = xmalloc(T * 8);
    int64_t* loc = xmalloc(T * 8);
    for (int64_t i = 0; i < nq; ++i) q[i] = next_bf16();
    for (int64_t i = 0; i < nw; ++i) w[i] = next_bf16();
    for (int64_t i = 0; i < nk; ++i) k[i] = next_bf16();
    for (int64_t i = 0; i < ntab; ++i) {
        cos_t[i] = cosf((float)i * 0.01f);
        sin_t[i] = sinf((float)i * 0.01f);
    }
    for (int i = 0; i < 128; ++i) {
        gamma[i] = 1.0f + 0.1f * next_float();
        beta[i] = 0.1f * next_float();
    }
    for (int64_t t = 0; t < T; ++t) {
        pos[t] = next_u32() % P;
        loc[t] = t % 3 == 2 ? -1 : (int64_t)((t * 37 + 5) % S);   /* some skipped slots */
    }
    uint8_t* q_fp8 = xmalloc(T * H * 128);
    float* w_out = xmalloc(T * H * 4);
    float* q_scale = xmalloc(T * H * 4);
    float* y = xmalloc(T * H * 128 * 4 + 4);
    int32_t* e = xmalloc(T * H * 4 + 4);
    CHECK(oracle_q(q, q_st, q_sh, w, w_st, pos, T, H, 0.5f, cos_t, sin_t, rs, P, R, style, q_fp8, w_out,
                   q_scale, nthreads) == 0);
    CHECK(oracle_q(q, q_st, q_sh, w, w_st, pos, T, H, 1.0f, cos_t, sin_t, rs, P, R, style, q_fp8, w_out,
                   NULL, nthreads) == 0);
    CHECK(oracle_q_values(q, q_st, q_sh, pos, T, H, cos_t, sin_t, rs, P, R, style, y, e, nthreads) == 0);
    uint8_t* cache = xmalloc((S - 1) * row_stride + 128);
    float* scale = xmalloc(S * 4);
    uint8_t* paged = xmalloc(S * 132);
    for (int bf16_mode = 0; bf16_mode < 2; ++bf16_mode) {
        CHECK(oracle_k_values(k, k_st, gamma, beta, 1e-6f, pos, T, cos_t, sin_t, rs, P, R, style, bf16_mode,
                              y, e, nthreads) == 0);
        CHECK(oracle_k(k, k_st, gamma, beta, 1e-6f, pos, loc, T, cos_t, sin_t, rs, P, R, style, bf16_mode,
                       cache, row_stride, scale, S, nthreads) == 0);
        CHECK(oracle_k_paged(k, k_st, gamma, beta, 1e-6f, pos, loc, T, cos_t, sin_t, rs, P, R, style,
                             bf16_mode, paged, page, S, nthreads) == 0);
    }
    if (T > 0) {
        CHECK(oracle_k_paged(k, k_st, gamma, beta, 1e-6f, pos, loc, T, cos_t, sin_t, rs, P, R, style, 0,
                             paged, 48, S, nthreads) == -3);
        pos[T - 1] = P;   /* out of the table: reported, nothing read past it */
        CHECK(oracle_q(q, q_st, q_sh, w, w_st, pos, T, H, 1.0f, cos_t, sin_t, rs, P, R, style, q_fp8,
                       w_out, q_scale, nthreads) == -1);
        CHECK(oracle_k(k, k_st, gamma, beta, 1e-6f, pos, loc, T, cos_t, sin_t, rs, P, R, style, 0, cache,
                       row_stride, scale, S, nthreads) == -1);
    }
    free(q); free(w); free(k); free(cos_t); free(sin_t); free(gamma); free(beta); free(pos); free(loc);
    free(q_fp8); free(w_out); free(q_scale); free(y); free(e); free(cache); free(scale); free(paged);
}

int main(void) {
    fp8_checks();
    const int rope_dims[] = {16, 64, 128};
    for (int ri = 0; ri < 3; ++ri)
        for (int style = 0; style < 2; ++style) {
            run_shape(5, 3, rope_dims[ri], style, 8, 2);
            run_shape(1, 1, rope_dims[ri], style, 0, 1);
        }
    run_shape(0, 2, 64, 0, 0, 1);
    if (g_errors) {
        fprintf(stderr, "%d check(s) failed\n", g_errors);
        return 1;
    }
    printf("oracle: all checks passed\n");
    return 0;
}
