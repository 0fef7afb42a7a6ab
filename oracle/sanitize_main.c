/*
 * sanitize_main.c -- test infrastructure: drives every function of the fp64 oracle
 * (xo.c) on small shapes that reach its edges (one row, one token, empty and full
 * caches, clamped accepted counts, ties in the greedy argmax) so that a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer sees every loop bound and index the
 * oracle computes.  Each call's result is also checked against a property it must have.
 * Exit status 0: no sanitizer report and every property held.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void xo_gemm(const uint16_t* x, const uint16_t* w, double* y, int M, int N, int K);
void xo_gdn(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* a, const float* b,
            const float* S0, int B, int T, int Hk, int Hv, int dk, int dv, double* o, double* S_all, double* S_T);
void xo_rollback(const uint16_t* k, const uint16_t* v, const float* a, const float* b, const float* S0,
                 const int32_t* kv_len, const int32_t* n_keep, int B, int T, int Hk, int Hv, int dk, int dv,
                 double* S_n, int32_t* kv_out);
void xo_attn(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new, const uint16_t* k_cache,
             const uint16_t* v_cache, const int32_t* kv_len, int B, int T, int Hq, int Hkv, int d, int Lmax,
             double scale, double* o);
void xo_attn_row(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new, const uint16_t* k_cache,
                 const uint16_t* v_cache, const int32_t* kv_len, int B, int T, int Hq, int Hkv, int d, int Lmax,
                 double scale, int bb, int r, int h, double* out);
void xo_greedy(const double* logits, const int32_t* draft, int B, int T, int N, int32_t* ids, int32_t* n_keep);
void xo_logprob(const double* logits, const int32_t* ids, int B, int T, int N, double* lp);

static uint32_t state = 12345u;
static double unif(void) { state = state * 1664525u + 1013904223u; return ((state >> 8) & 0xFFFFFF) / 16777216.0; }
static uint16_t bf16(double x) {                 /* nearest-even bf16 bits of (float)x */
    float f = (float)x;
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
static uint16_t* bf_array(size_t n, double s) {
    uint16_t* p = malloc(n * sizeof(uint16_t));
    for (size_t i = 0; i < n; ++i) p[i] = bf16((2.0 * unif() - 1.0) * s);
    return p;
}
static float* f_array(size_t n, double lo, double hi) {
    float* p = malloc(n * sizeof(float));
    for (size_t i = 0; i < n; ++i) p[i] = (float)(lo + (hi - lo) * unif());
    return p;
}
static int fails = 0;
#define CHECK(c) do { if (!(c)) { fprintf(stderr, "property failed: %s (line %d)\n", #c, __LINE__); ++fails; } } while (0)

static void gemm(void) {
    const int M = 3, N = 5, K = 7;
    uint16_t* x = bf_array((size_t)M * K, 1.0);
    uint16_t* w = bf_array((size_t)N * K, 1.0);
    double* y = malloc(sizeof(double) * M * N);
    xo_gemm(x, w, y, M, N, K);
    for (int i = 0; i < M * N; ++i) CHECK(isfinite(y[i]));
    free(x); free(w); free(y);
}

static void gdn(int B, int T, int Hk, int Hv, int dk, int dv) {
    const size_t nk = (size_t)B * T * Hk * dk, nv = (size_t)B * T * Hv * dv, na = (size_t)B * T * Hv;
    const size_t ns = (size_t)B * Hv * dk * dv;
    uint16_t *q = bf_array(nk, 0.3), *k = bf_array(nk, 0.3), *v = bf_array(nv, 1.0);
    float *a = f_array(na, 0.3, 0.95), *bb = f_array(na, 0.0, 1.0), *S0 = f_array(ns, -0.1, 0.1);
    double* o = malloc(sizeof(double) * nv);
    double* S_all = malloc(sizeof(double) * ns * (size_t)(T + 1));
    double* S_T = malloc(sizeof(double) * ns);
    xo_gdn(q, k, v, a, bb, S0, B, T, Hk, Hv, dk, dv, o, S_all, S_T);
    const size_t st = ns / B;                          /* one request's state */
    for (int i = 0; i < B; ++i)
        for (size_t e = 0; e < st; ++e) {
            CHECK(S_all[((size_t)i * (T + 1) + T) * st + e] == S_T[(size_t)i * st + e]);
            CHECK(S_all[((size_t)i * (T + 1)) * st + e] == (double)S0[(size_t)i * st + e]);
        }
    /* rollback to every clamped count, and a count past T */
    int32_t* kv = malloc(sizeof(int32_t) * B);
    int32_t* nkeep = malloc(sizeof(int32_t) * B);
    int32_t* kv_out = malloc(sizeof(int32_t) * B);
    double* Sn = malloc(sizeof(double) * ns);
    for (int n = -1; n <= T + 1; ++n) {
        for (int i = 0; i < B; ++i) { kv[i] = 10 + i; nkeep[i] = n + i; }
        xo_rollback(k, v, a, bb, S0, kv, nkeep, B, T, Hk, Hv, dk, dv, Sn, kv_out);
        for (int i = 0; i < B; ++i) {
            CHECK(kv_out[i] == 10 + i + n + i);        /* the length moves by n_keep as given */
            const int nn = n + i < 0 ? 0 : (n + i > T ? T : n + i);   /* the state clamps it */
            for (size_t e = 0; e < st; ++e)
                CHECK(Sn[(size_t)i * st + e] == S_all[((size_t)i * (T + 1) + nn) * st + e]);
        }
    }
    free(q); free(k); free(v); free(a); free(bb); free(S0); free(o); free(S_all); free(S_T);
    free(kv); free(nkeep); free(kv_out); free(Sn);
}

static void attn(int B, int T, int Hq, int Hkv, int d, const int32_t* L0, int Lmax) {
    const size_t nq = (size_t)B * T * Hq * d, nn = (size_t)B * T * Hkv * d, nc = (size_t)B * Hkv * Lmax * d;
    uint16_t *q = bf_array(nq, 1.0), *kn = bf_array(nn, 1.0), *vn = bf_array(nn, 1.0);
    uint16_t *kc = bf_array(nc, 1.0), *vc = bf_array(nc, 1.0);
    double* o = malloc(sizeof(double) * nq);
    double* row = malloc(sizeof(double) * d);
    const double scale = 1.0 / sqrt((double)d);
    xo_attn(q, kn, vn, kc, vc, L0, B, T, Hq, Hkv, d, Lmax, scale, o);
    for (int bb = 0; bb < B; ++bb)
        for (int r = 0; r < T; ++r)
            for (int h = 0; h < Hq; ++h) {
                xo_attn_row(q, kn, vn, kc, vc, L0, B, T, Hq, Hkv, d, Lmax, scale, bb, r, h, row);
                for (int j = 0; j < d; ++j) CHECK(row[j] == o[(((size_t)bb * T + r) * Hq + h) * d + j]);
            }
    free(q); free(kn); free(vn); free(kc); free(vc); free(o); free(row);
}

static void head(void) {
    const int B = 2, T = 3, N = 6;
    double logits[2 * 3 * 6];
    for (int i = 0; i < B * T * N; ++i) logits[i] = (double)((i * 7) % 5);   /* ties in every row */
    int32_t draft[6] = {0, 4, 1, 3, 2, 0}, ids[6], nk[2];
    double lp[6];
    xo_greedy(logits, draft, B, T, N, ids, nk);
    for (int i = 0; i < B * T; ++i) CHECK(ids[i] >= 0 && ids[i] < N);
    for (int i = 0; i < B; ++i) CHECK(nk[i] >= 1 && nk[i] <= T);
    xo_logprob(logits, ids, B, T, N, lp);
    for (int i = 0; i < B * T; ++i) CHECK(lp[i] <= 0.0 && isfinite(lp[i]));
}

int main(void) {
    gemm();
    gdn(1, 1, 1, 1, 4, 4);
    gdn(2, 5, 2, 4, 8, 4);
    gdn(1, 16, 1, 3, 16, 8);
    {
        const int32_t L0a[1] = {0};
        attn(1, 1, 2, 1, 8, L0a, 1);                 /* empty cache, capacity exactly L0 + T */
        const int32_t L0b[2] = {3, 9};
        attn(2, 4, 4, 2, 8, L0b, 13);                /* ragged lengths, one request at capacity */
    }
    head();
    if (fails) { fprintf(stderr, "%d properties failed\n", fails); return 1; }
    printf("oracle sanitizer run: ok\n");
    return 0;
}
