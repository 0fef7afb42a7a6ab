/*
 * xo.c -- plain, slow fp64 CPU oracle for the speculative-decoding verify step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark may.  It shares no code, header, table or helper with the HIP
 * path: it reads the same raw inputs (bf16 bit patterns, fp32 values, int32
 * lengths) and computes, in double precision, the plain definitions below.
 *
 * Sources.  "Post" is the author's r/LocalLLaMA post on bit-exact speculative
 * decoding of Qwen3.8-27B on one RTX PRO 6000 (feedman.me mirror); "card" is
 * the recipe card "Qwen3.8-27B Bit-Exact Spec-Decode 1x RTX PRO 6000 SGLang".
 *  - Post, the paragraph on the two verify changes: verify advances the GDN
 *    (gated delta net) recurrence with the decode arithmetic, whose state is
 *    fp32 (post, launch command: the mamba SSM dtype flag).  The pages print
 *    no equation; the rule used throughout is the gated delta rule
 *        S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,  o_t = S_t q_t.
 *  - Same paragraph: verify attention is computed as one decode row per draft
 *    position, so row r of a T-row verify over a cache of L0 positions sees
 *    positions 0..L0+r, the same positions the decode step there would see;
 *    plain softmax(scale * q.K^T) V.
 *  - Post, the DeepGEMM paragraph, and card, runtime env (the M <= 16 small-M
 *    gate): the bf16 projection GEMMs y = x W^T, weights stored one output
 *    row per line with K contiguous.
 *  - Post, first paragraph and decode table: greedy decoding at temperature
 *    zero, compared on token ids.
 *
 * Every loop is written in the order of the definition; there is no blocking,
 * fusion or reordering.  OpenMP only splits independent output units
 * (request/head, row, output element) across threads; the arithmetic inside a
 * unit does not depend on the thread count.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* A bf16 value is the top half of an IEEE fp32 bit pattern. */
static double xo_bf16(uint16_t h) {
    union { uint32_t u; float f; } c;
    c.u = ((uint32_t)h) << 16;
    return (double)c.f;
}

int xo_version(void) { return 1; }

/* ------------------------------------------------------------------------ */
/* Projection GEMM: y[m][n] = sum_{k=0}^{K-1} x[m][k] * w[n][k], k ascending. */
/* x: bf16 [M][K], w: bf16 [N][K], y: fp64 [M][N].                            */
/* ------------------------------------------------------------------------ */
void xo_gemm(const uint16_t* x, const uint16_t* w, double* y, int M, int N, int K) {
    long mn = (long)M * (long)N;
#pragma omp parallel for schedule(static)
    for (long e = 0; e < mn; ++e) {
        long m = e / N, n = e % N;
        const uint16_t* xr = x + m * (long)K;
        const uint16_t* wr = w + n * (long)K;
        double s = 0.0;
        for (int k = 0; k < K; ++k) s += xo_bf16(xr[k]) * xo_bf16(wr[k]);
        y[e] = s;
    }
}

/* ------------------------------------------------------------------------ */
/* Gated delta rule, one request and one value head, T tokens.               */
/*                                                                          */
/* The state is the d_v x d_k matrix S (value index j, key index i).  In     */
/* memory (input state S0 and every saved state) it is stored key-major:     */
/* element (j, i) at offset i*dv + j, i.e. layout [dk][dv].                  */
/*                                                                          */
/* Per token t, with decay a, beta b, key k, value v, query q:               */
/*   P   = S (I - b k k^T)          (P[j][i] = S[j][i] - b (sum_l S[j][l]k[l]) k[i]) */
/*   S  <- a P + b v k^T                                                     */
/*   o_t = S q                                                               */
/* i.e. the matrix product with (I - b k k^T) expanded row by row.           */
/* ------------------------------------------------------------------------ */
static void xo_gdn_head(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        const float* a, const float* b, const float* S0,
                        int T, int Hk, int Hv, int dk, int dv, int h,
                        double* o,        /* [T][Hv][dv] slice base or NULL     */
                        double* S_save,   /* [T+1][Hv][dk][dv] base or NULL     */
                        double* S_fin)    /* [Hv][dk][dv] base or NULL          */
{
    int g = h / (Hv / Hk);                 /* key head that serves value head h */
    double* S = (double*)malloc(sizeof(double) * (size_t)dv * dk);   /* S[j*dk+i] */
    double* Sk = (double*)malloc(sizeof(double) * (size_t)dv);
    double* kt = (double*)malloc(sizeof(double) * (size_t)dk);
    double* qt = (double*)malloc(sizeof(double) * (size_t)dk);
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j)
            S[(size_t)j * dk + i] = (double)S0[((size_t)h * dk + i) * dv + j];
    if (S_save) {
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                S_save[((size_t)h * dk + i) * dv + j] = S[(size_t)j * dk + i];
    }
    for (int t = 0; t < T; ++t) {
        const uint16_t* kr = k + ((size_t)t * Hk + g) * dk;
        const uint16_t* qr = q + ((size_t)t * Hk + g) * dk;
        const uint16_t* vr = v + ((size_t)t * Hv + h) * dv;
        double at = (double)a[(size_t)t * Hv + h];
        double bt = (double)b[(size_t)t * Hv + h];
        for (int i = 0; i < dk; ++i) { kt[i] = xo_bf16(kr[i]); qt[i] = xo_bf16(qr[i]); }
        /* S k (uses the previous state) */
        for (int j = 0; j < dv; ++j) {
            double s = 0.0;
            for (int i = 0; i < dk; ++i) s += S[(size_t)j * dk + i] * kt[i];
            Sk[j] = s;
        }
        /* S <- a (S - b (S k) k^T) + b v k^T */
        for (int j = 0; j < dv; ++j) {
            double vj = xo_bf16(vr[j]);
            for (int i = 0; i < dk; ++i) {
                double p = S[(size_t)j * dk + i] - bt * Sk[j] * kt[i];
                S[(size_t)j * dk + i] = at * p + bt * vj * kt[i];
            }
        }
        /* o_t = S_t q_t */
        if (o) {
            for (int j = 0; j < dv; ++j) {
                double s = 0.0;
                for (int i = 0; i < dk; ++i) s += S[(size_t)j * dk + i] * qt[i];
                o[((size_t)t * Hv + h) * dv + j] = s;
            }
        }
        if (S_save) {
            double* dst = S_save + (size_t)(t + 1) * Hv * dk * dv;
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j)
                    dst[((size_t)h * dk + i) * dv + j] = S[(size_t)j * dk + i];
        }
    }
    if (S_fin) {
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                S_fin[((size_t)h * dk + i) * dv + j] = S[(size_t)j * dk + i];
    }
    free(S); free(Sk); free(kt); free(qt);
}

/*
 * xo_gdn: B requests, T tokens each.
 *   q, k : bf16 [B][T][Hk][dk]     v : bf16 [B][T][Hv][dv]
 *   a, b : fp32 [B][T][Hv]         S0: fp32 [B][Hv][dk][dv]
 *   o    : fp64 [B][T][Hv][dv] or NULL
 *   S_all: fp64 [B][T+1][Hv][dk][dv] or NULL (S_all[b][0] = S0[b], S_all[b][t] = S_t)
 *   S_T  : fp64 [B][Hv][dk][dv] or NULL
 */
void xo_gdn(const uint16_t* q, const uint16_t* k, const uint16_t* v,
            const float* a, const float* b, const float* S0,
            int B, int T, int Hk, int Hv, int dk, int dv,
            double* o, double* S_all, double* S_T)
{
    long units = (long)B * Hv;
#pragma omp parallel for schedule(dynamic, 1)
    for (long u = 0; u < units; ++u) {
        int bb = (int)(u / Hv), h = (int)(u % Hv);
        size_t st = (size_t)Hv * dk * dv;
        xo_gdn_head(q + (size_t)bb * T * Hk * dk, k + (size_t)bb * T * Hk * dk,
                    v + (size_t)bb * T * Hv * dv, a + (size_t)bb * T * Hv,
                    b + (size_t)bb * T * Hv, S0 + (size_t)bb * st,
                    T, Hk, Hv, dk, dv, h,
                    o ? o + (size_t)bb * T * Hv * dv : NULL,
                    S_all ? S_all + (size_t)bb * (T + 1) * st : NULL,
                    S_T ? S_T + (size_t)bb * st : NULL);
    }
}

/*
 * Rollback to the accepted prefix: the state after the first n_keep[b] rows,
 * i.e. the recurrence above run over rows 0..n-1 only (n = 0 gives S0 back),
 * and the new cache length kv_len[b] + n_keep[b].
 *   k, v, a, b and S0 as for xo_gdn (q is not needed for the state).
 *   S_n   : fp64 [B][Hv][dk][dv]    kv_out: int32 [B]
 */
void xo_rollback(const uint16_t* k, const uint16_t* v, const float* a, const float* b,
                 const float* S0, const int32_t* kv_len, const int32_t* n_keep,
                 int B, int T, int Hk, int Hv, int dk, int dv,
                 double* S_n, int32_t* kv_out)
{
    long units = (long)B * Hv;
    for (int bb = 0; bb < B; ++bb) kv_out[bb] = kv_len[bb] + n_keep[bb];
#pragma omp parallel for schedule(dynamic, 1)
    for (long u = 0; u < units; ++u) {
        int bb = (int)(u / Hv), h = (int)(u % Hv);
        int n = n_keep[bb];
        if (n < 0) n = 0;
        if (n > T) n = T;
        size_t st = (size_t)Hv * dk * dv;
        /* q only feeds o, which is not requested here; pass k in its place. */
        xo_gdn_head(k + (size_t)bb * T * Hk * dk, k + (size_t)bb * T * Hk * dk,
                    v + (size_t)bb * T * Hv * dv, a + (size_t)bb * T * Hv,
                    b + (size_t)bb * T * Hv, S0 + (size_t)bb * st,
                    n, Hk, Hv, dk, dv, h, NULL, NULL, S_n + (size_t)bb * st);
    }
}

/* ------------------------------------------------------------------------ */
/* Attention, one decode row per draft position.                            */
/*                                                                          */
/* Request b held L0 = kv_len[b] cached positions before the verify; the T   */
/* new key/value rows take positions L0..L0+T-1.  Row r (query q[b][r][h])   */
/* sees positions 0..L0+r inclusive; key/value j comes from the cache for    */
/* j < L0 and from the new rows for j >= L0.  Query head h reads KV head     */
/* h / (Hq/Hkv).  o = sum_j softmax_j(scale * q.k_j) v_j with the maximum    */
/* subtracted before exponentiating.                                         */
/* ------------------------------------------------------------------------ */
static void xo_attn_row_impl(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                             const uint16_t* k_cache, const uint16_t* v_cache,
                             const int32_t* kv_len, int T, int Hq, int Hkv, int d,
                             int Lmax, double scale, int bb, int r, int h, double* out)
{
    int g = h / (Hq / Hkv);
    long L0 = kv_len[bb];
    long len = L0 + r + 1;
    const uint16_t* qr = q + (((size_t)bb * T + r) * Hq + h) * d;
    double* s = (double*)malloc(sizeof(double) * (size_t)len);
    double* qd = (double*)malloc(sizeof(double) * (size_t)d);
    for (int e = 0; e < d; ++e) qd[e] = xo_bf16(qr[e]);
    double mx = -INFINITY;
    for (long j = 0; j < len; ++j) {
        const uint16_t* kr = (j < L0)
            ? k_cache + (((size_t)bb * Hkv + g) * Lmax + j) * d
            : k_new + (((size_t)bb * T + (j - L0)) * Hkv + g) * d;
        double dot = 0.0;
        for (int e = 0; e < d; ++e) dot += qd[e] * xo_bf16(kr[e]);
        s[j] = scale * dot;
        if (s[j] > mx) mx = s[j];
    }
    double den = 0.0;
    for (long j = 0; j < len; ++j) { s[j] = exp(s[j] - mx); den += s[j]; }
    for (int e = 0; e < d; ++e) out[e] = 0.0;
    for (long j = 0; j < len; ++j) {
        const uint16_t* vr = (j < L0)
            ? v_cache + (((size_t)bb * Hkv + g) * Lmax + j) * d
            : v_new + (((size_t)bb * T + (j - L0)) * Hkv + g) * d;
        for (int e = 0; e < d; ++e) out[e] += s[j] * xo_bf16(vr[e]);
    }
    for (int e = 0; e < d; ++e) out[e] /= den;
    free(s); free(qd);
}

/* One row (b, r, h); out: fp64 [d]. */
void xo_attn_row(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                 const uint16_t* k_cache, const uint16_t* v_cache, const int32_t* kv_len,
                 int B, int T, int Hq, int Hkv, int d, int Lmax, double scale,
                 int bb, int r, int h, double* out)
{
    (void)B;
    xo_attn_row_impl(q, k_new, v_new, k_cache, v_cache, kv_len, T, Hq, Hkv, d, Lmax,
                     scale, bb, r, h, out);
}

/* All rows; o: fp64 [B][T][Hq][d]. */
void xo_attn(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
             const uint16_t* k_cache, const uint16_t* v_cache, const int32_t* kv_len,
             int B, int T, int Hq, int Hkv, int d, int Lmax, double scale, double* o)
{
    long rows = (long)B * T * Hq;
#pragma omp parallel for schedule(dynamic, 1)
    for (long u = 0; u < rows; ++u) {
        int bb = (int)(u / ((long)T * Hq));
        int r = (int)((u / Hq) % T);
        int h = (int)(u % Hq);
        xo_attn_row_impl(q, k_new, v_new, k_cache, v_cache, kv_len, T, Hq, Hkv, d, Lmax,
                         scale, bb, r, h, o + (size_t)u * d);
    }
}

/* ------------------------------------------------------------------------ */
/* Greedy acceptance at temperature 0.                                       */
/* ids[b][t] = argmax_n logits[b][t][n] (lowest index among equal maxima).    */
/* Row t of a verify consumed input token draft[b][t] (draft[b][0] is the    */
/* root, the last accepted token); draft t+1 is accepted when it equals       */
/* ids[b][t] and every earlier draft was accepted.  n_keep[b] = 1 + the       */
/* number of accepted drafts = the number of verify rows that stay.          */
/* ------------------------------------------------------------------------ */
void xo_greedy(const double* logits, const int32_t* draft, int B, int T, int N,
               int32_t* ids, int32_t* n_keep)
{
    for (int bb = 0; bb < B; ++bb) {
        for (int t = 0; t < T; ++t) {
            const double* row = logits + ((size_t)bb * T + t) * N;
            int best = 0;
            for (int n = 1; n < N; ++n)
                if (row[n] > row[best]) best = n;
            ids[(size_t)bb * T + t] = best;
        }
        int acc = 0;
        while (acc + 1 < T && draft[(size_t)bb * T + acc + 1] == ids[(size_t)bb * T + acc]) ++acc;
        n_keep[bb] = acc + 1;
    }
}

/* ------------------------------------------------------------------------ */
/* Log-probability of a chosen token (post, first paragraph: the outputs    */
/* compared were token ids and their logprobs).  With z the row's logits:   */
/*   lp[b][t] = log softmax(z)[id] = z[id] - max(z) - log sum_n exp(z[n] - max(z)) */
/* fp64, n ascending.                                                        */
/* ------------------------------------------------------------------------ */
void xo_logprob(const double* logits, const int32_t* ids, int B, int T, int N, double* lp)
{
    for (long r = 0; r < (long)B * T; ++r) {
        const double* row = logits + r * N;
        double m = row[0];
        for (int n = 1; n < N; ++n)
            if (row[n] > m) m = row[n];
        double s = 0.0;
        for (int n = 0; n < N; ++n) s += exp(row[n] - m);
        lp[r] = (row[ids[r]] - m) - log(s);
    }
}
