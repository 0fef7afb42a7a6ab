// xv_attn.hip -- attention verify rows: one decode row per draft position.
//
// The post's second verify change: verify attention runs as decode rows, one
// per draft position.  Row r of request b (cache length L0 before the verify)
// is exactly the decode row at position L0 + r: it sees positions 0..L0+r, and
// every number it produces depends only on its own query, its length and the
// key/value bytes at those positions -- never on T, on the other rows, on the
// batch, on Lmax or on the workspace size.
//
// Two kernels on the caller's stream:
//  1. xv_attn_partial_kernel, grid (chunk, KV head, request).  A chunk is
//     XV_ATTN_C positions at an absolute boundary.  The workgroup loads the
//     chunk's keys and values into LDS 64 positions at a time (new rows come
//     from k_new/v_new and are also appended to the cache by the one
//     workgroup whose chunk holds them), and computes, for every (query head of
//     the group, row) pair with a visible position in the chunk:
//         s_j = scale * (q . k_j)            (bf16 MFMA, fp32 accumulate)
//         m_c = max_j s_j over visible j     (exact)
//         p_j = exp(s_j - m_c), 0 for masked j
//         l_c = sum_j p_j                    (fixed order: in-lane ascending,
//                                             then lane butterfly 16, 32)
//         acc_c = sum_j p_j v_j              (MFMA with p split into bf16 hi + lo)
//     One wave owns 16 pairs; scores are computed transposed (S^T = K Q^T) so
//     that each lane already holds the probabilities of its pair in the order
//     the P.V MFMA consumes them, with no round trip through LDS.
//  2. xv_attn_combine_kernel, grid (query head, row, request): with
//     M = max_c m_c, beta_c = exp(m_c - M), L = sum_c l_c beta_c and
//     A = sum_c acc_c beta_c in ascending chunk order; o = A / L, stored as
//     bf16 (nearest even) and optionally fp32.
// Masked positions are excluded by index, never by value, and positions at or
// past L0 + T are never read (their LDS slots are zero-filled).
#include "xv_common.h"
#include <math.h>

namespace {

constexpr int XV_ATTN_C = 256;      // chunk length (positions), fixed for every call
constexpr int XV_ATTN_SUB = 64;     // positions per LDS sub-block
constexpr int XV_ATTN_WAVES = 8;    // 16 pairs per wave -> up to 128 (head, row) pairs
constexpr int XV_ATTN_MAX_NC = 8192;

template <int D>
__global__ __launch_bounds__(XV_ATTN_WAVES * 64)
void xv_attn_partial_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_new,
                            const uint16_t* __restrict__ v_new, uint16_t* __restrict__ k_cache,
                            uint16_t* __restrict__ v_cache, const int32_t* __restrict__ kv_len,
                            float* __restrict__ ws_acc, float* __restrict__ ws_ml,
                            int T, int Hq, int Hkv, int Lmax, int NC, float scale)
{
    constexpr int KS = D / 32;                  // MFMA k-steps over the head dim
    constexpr int DB = D / 16;                  // 16-wide blocks of output dims
    constexpr int NCB = XV_ATTN_C / 16;         // 16-position score blocks per chunk
    constexpr int NSB = XV_ATTN_C / XV_ATTN_SUB;
    constexpr int KPAD = D + 8;                 // LDS row pitch (bf16) of K
    constexpr int VPAD = XV_ATTN_SUB + 8;       // LDS row pitch (bf16) of V^T
    __shared__ __attribute__((aligned(16))) uint16_t Ks[XV_ATTN_SUB * KPAD];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VPAD];

    const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int Hg = Hq / Hkv;
    const int P = Hg * T;
    int L0 = kv_len[b];
    L0 = L0 < 0 ? 0 : (L0 > Lmax - T ? Lmax - T : L0);
    const int Lend = L0 + T;
    const int c0 = c * XV_ATTN_C;
    if (c0 >= Lend) return;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const bool tile_on = wave * 16 < P;
    const int pair = wave * 16 + lr;            // the pair whose scores this lane holds
    const bool pair_ok = pair < P;
    const int pr = pair_ok ? pair / Hg : 0;
    const int ph = g * Hg + (pair_ok ? pair % Hg : 0);
    const int plen = L0 + pr + 1;

    const size_t kvbase = ((size_t)b * Hkv + g) * Lmax;
    const xv_u32x4 zero = {0u, 0u, 0u, 0u};

    xv_u32x4 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qf[ks] = pair_ok ? xv_load16(q + (((size_t)b * T + pr) * Hq + ph) * D + ks * 32 + lg * 8) : zero;

    // ---- phase 1: scores S^T[pos][pair] for the whole chunk ----
    xv_f32x4 sc[NCB];
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb) {
        const int p0 = c0 + sb * XV_ATTN_SUB;
        if (p0 >= Lend) {                       // uniform: nothing visible from here on
#pragma unroll
            for (int cbl = 0; cbl < 4; ++cbl) sc[sb * 4 + cbl] = xv_f32x4{0.f, 0.f, 0.f, 0.f};
            continue;
        }
        __syncthreads();
        for (int idx = threadIdx.x; idx < XV_ATTN_SUB * (D / 8); idx += blockDim.x) {
            const int i = idx / (D / 8), cc = idx % (D / 8);
            const int pos = p0 + i;
            xv_u32x4 val = zero;
            if (pos < L0) {
                val = xv_load16(k_cache + (kvbase + pos) * D + cc * 8);
            } else if (pos < Lend) {
                val = xv_load16(k_new + (((size_t)b * T + (pos - L0)) * Hkv + g) * D + cc * 8);
                xv_store16(k_cache + (kvbase + pos) * D + cc * 8, val);
            }
            xv_store16(&Ks[i * KPAD + cc * 8], val);
        }
        __syncthreads();
        if (tile_on) {
#pragma unroll
            for (int cbl = 0; cbl < 4; ++cbl) {
                xv_f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    acc = xv_mfma16x16x32(xv_load16(&Ks[(cbl * 16 + lr) * KPAD + ks * 32 + lg * 8]),
                                          qf[ks], acc);
                sc[sb * 4 + cbl] = acc;
            }
        }
    }

    // ---- phase 2: chunk max, probabilities, chunk sum (per pair, fixed order) ----
    float m = -INFINITY;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int pos = c0 + cb * 16 + 4 * lg + i;
            const float sv = sc[cb][i] * scale;
            sc[cb][i] = sv;
            if (pair_ok && pos < plen) m = fmaxf(m, sv);
        }
    m = fmaxf(m, __shfl_xor(m, 16));
    m = fmaxf(m, __shfl_xor(m, 32));
    float l = 0.f;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int pos = c0 + cb * 16 + 4 * lg + i;
            const float pv = (pair_ok && pos < plen) ? expf(sc[cb][i] - m) : 0.f;
            sc[cb][i] = pv;
            l = l + pv;
        }
    l = l + __shfl_xor(l, 16);
    l = l + __shfl_xor(l, 32);

    // ---- phase 3: acc = P V over every sub-block of the chunk ----
    xv_f32x4 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = xv_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb) {
        const int p0 = c0 + sb * XV_ATTN_SUB;
        __syncthreads();
        // V rows [p0, p0 + 64) transposed into Vt[d][pos]; 8 positions x 8 dims per item
        for (int idx = threadIdx.x; idx < (XV_ATTN_SUB / 8) * (D / 8); idx += blockDim.x) {
            const int pg = idx / (D / 8), dg = idx % (D / 8);
            xv_u32x4 rows[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int pos = p0 + pg * 8 + e;
                rows[e] = zero;
                if (pos < L0) {
                    rows[e] = xv_load16(v_cache + (kvbase + pos) * D + dg * 8);
                } else if (pos < Lend) {
                    rows[e] = xv_load16(v_new + (((size_t)b * T + (pos - L0)) * Hkv + g) * D + dg * 8);
                    xv_store16(v_cache + (kvbase + pos) * D + dg * 8, rows[e]);
                }
            }
#pragma unroll
            for (int dd = 0; dd < 8; ++dd) {
                xv_u32x4 outv;
#pragma unroll
                for (int w2 = 0; w2 < 4; ++w2) {
                    const uint32_t lo = rows[2 * w2][dd >> 1], hi = rows[2 * w2 + 1][dd >> 1];
                    outv[w2] = (dd & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u))
                                        : ((lo & 0xFFFFu) | (hi << 16));
                }
                xv_store16(&Vt[(dg * 8 + dd) * VPAD + pg * 8], outv);
            }
        }
        __syncthreads();
        if (tile_on) {
#pragma unroll
            for (int kk = 0; kk < XV_ATTN_SUB / 32; ++kk) {
                // k-slot e of lane group lg <-> local position kk*32 + 4*lg + e (e < 4)
                //                                       or kk*32 + 16 + 4*lg + (e - 4)
                const xv_f32x4 pa = sc[sb * 4 + kk * 2];
                const xv_f32x4 pb = sc[sb * 4 + kk * 2 + 1];
                float pe[8] = {pa[0], pa[1], pa[2], pa[3], pb[0], pb[1], pb[2], pb[3]};
                xv_u32x4 phi, plo;
#pragma unroll
                for (int w2 = 0; w2 < 4; ++w2) {
                    const uint16_t h0 = xv_f32_to_bf16(pe[2 * w2]);
                    const uint16_t h1 = xv_f32_to_bf16(pe[2 * w2 + 1]);
                    const uint16_t l0 = xv_f32_to_bf16(pe[2 * w2] - xv_bf16_to_f32(h0));
                    const uint16_t l1 = xv_f32_to_bf16(pe[2 * w2 + 1] - xv_bf16_to_f32(h1));
                    phi[w2] = (uint32_t)h0 | ((uint32_t)h1 << 16);
                    plo[w2] = (uint32_t)l0 | ((uint32_t)l1 << 16);
                }
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const uint16_t* vr = &Vt[(db * 16 + lr) * VPAD + kk * 32];
                    const uint2 va = *reinterpret_cast<const uint2*>(vr + 4 * lg);
                    const uint2 vb = *reinterpret_cast<const uint2*>(vr + 16 + 4 * lg);
                    const xv_u32x4 vf = {va.x, va.y, vb.x, vb.y};
                    oacc[db] = xv_mfma16x16x32(phi, vf, oacc[db]);
                    oacc[db] = xv_mfma16x16x32(plo, vf, oacc[db]);
                }
            }
        }
    }

    // ---- phase 4: write the chunk partials of pairs that see this chunk ----
    if (!tile_on) return;
    if (lg == 0 && pair_ok && plen > c0) {
        const size_t idx = (((size_t)b * T + pr) * Hq + ph) * NC + c;
        ws_ml[idx * 2 + 0] = m;
        ws_ml[idx * 2 + 1] = l;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int pair2 = wave * 16 + 4 * lg + i;
        if (pair2 >= P) continue;
        const int r2 = pair2 / Hg;
        if (L0 + r2 + 1 <= c0) continue;
        const int h2 = g * Hg + pair2 % Hg;
        float* dst = ws_acc + ((((size_t)b * T + r2) * Hq + h2) * NC + c) * D + lr;
#pragma unroll
        for (int db = 0; db < DB; ++db) dst[db * 16] = oacc[db][i];
    }
}

template <int D>
__global__ __launch_bounds__(D)
void xv_attn_combine_kernel(const float* __restrict__ ws_acc, const float* __restrict__ ws_ml,
                            const int32_t* __restrict__ kv_len, uint16_t* __restrict__ o,
                            float* __restrict__ o32, int T, int Hq, int Lmax, int NC)
{
    extern __shared__ float sh[];               // [NC] beta, [NC] l*beta, [D] max scratch
    float* sbeta = sh;
    float* slw = sh + NC;
    float* sred = sh + 2 * NC;
    const int h = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x;
    int L0 = kv_len[b];
    L0 = L0 < 0 ? 0 : (L0 > Lmax - T ? Lmax - T : L0);
    const int len = L0 + r + 1;
    const int nc = (len + XV_ATTN_C - 1) / XV_ATTN_C;
    const size_t base = (((size_t)b * T + r) * Hq + h) * NC;

    float mloc = -INFINITY;
    for (int cc = tid; cc < nc; cc += D) mloc = fmaxf(mloc, ws_ml[(base + cc) * 2]);
    sred[tid] = mloc;
    __syncthreads();
    if (tid == 0) {
        float mm = sred[0];
        for (int i = 1; i < D; ++i) mm = fmaxf(mm, sred[i]);
        sred[0] = mm;
    }
    __syncthreads();
    const float M = sred[0];
    for (int cc = tid; cc < nc; cc += D) {
        const float be = expf(ws_ml[(base + cc) * 2] - M);
        sbeta[cc] = be;
        slw[cc] = ws_ml[(base + cc) * 2 + 1] * be;
    }
    __syncthreads();
    float L = 0.f, A = 0.f;
    const float* ap = ws_acc + base * D + tid;
#pragma unroll 8
    for (int cc = 0; cc < nc; ++cc) {
        L = L + slw[cc];
        A = __builtin_fmaf(ap[(size_t)cc * D], sbeta[cc], A);
    }
    const float ov = A / L;
    const size_t oi = (((size_t)b * T + r) * Hq + h) * D + tid;
    o[oi] = xv_f32_to_bf16(ov);
    if (o32) o32[oi] = ov;
}

template <int D>
int xv_attn_launch(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                   uint16_t* k_cache, uint16_t* v_cache, const int32_t* kv_len,
                   uint16_t* o, float* o32, float* ws_acc, float* ws_ml,
                   int B, int T, int Hq, int Hkv, int Lmax, int NC, float scale, hipStream_t st)
{
    (void)hipGetLastError();
    hipLaunchKernelGGL(xv_attn_partial_kernel<D>, dim3(NC, Hkv, B), dim3(XV_ATTN_WAVES * 64), 0, st,
                       q, k_new, v_new, k_cache, v_cache, kv_len, ws_acc, ws_ml,
                       T, Hq, Hkv, Lmax, NC, scale);
    int s = xv_launch_status();
    if (s != XV_OK) return s;
    const size_t shmem = sizeof(float) * (2 * (size_t)NC + D);
    hipLaunchKernelGGL(xv_attn_combine_kernel<D>, dim3(Hq, T, B), dim3(D), shmem, st,
                       ws_acc, ws_ml, kv_len, o, o32, T, Hq, Lmax, NC);
    return xv_launch_status();
}

size_t xv_attn_ws(int B, int T, int Hq, int d, int Lmax, size_t* acc_bytes) {
    const size_t NC = (size_t)((Lmax + XV_ATTN_C - 1) / XV_ATTN_C);
    const size_t pairs = (size_t)B * T * Hq * NC;
    const size_t a = pairs * (size_t)d * sizeof(float);
    if (acc_bytes) *acc_bytes = a;
    return a + pairs * 2 * sizeof(float);
}

}  // namespace

extern "C" int xv_attn_chunk_tokens(void) { return XV_ATTN_C; }

extern "C" size_t xv_attn_workspace_bytes(int B, int T, int Hq, int d, int Lmax) {
    if (B <= 0 || T <= 0 || Hq <= 0 || d <= 0 || Lmax <= 0) return 0;
    return xv_attn_ws(B, T, Hq, d, Lmax, nullptr);
}

extern "C" int xv_attn_verify_rows(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                                   uint16_t* k_cache, uint16_t* v_cache, const int32_t* kv_len,
                                   uint16_t* o, float* o32, void* workspace, size_t workspace_bytes,
                                   int B, int T, int Hq, int Hkv, int d, int Lmax, float scale,
                                   void* stream)
{
    XV_REQUIRE(B >= 0 && T >= 1 && T <= 16 && Hkv >= 1 && Hq >= 1 && Hq % Hkv == 0, XV_ERR_SHAPE);
    XV_REQUIRE((Hq / Hkv) * T <= 16 * XV_ATTN_WAVES, XV_ERR_SHAPE);
    XV_REQUIRE(d == 64 || d == 128 || d == 256, XV_ERR_SHAPE);
    XV_REQUIRE(Lmax >= T && (Lmax + XV_ATTN_C - 1) / XV_ATTN_C <= XV_ATTN_MAX_NC, XV_ERR_SHAPE);
    XV_REQUIRE(scale == scale, XV_ERR_SHAPE);
    if (B == 0) return XV_OK;
    XV_REQUIRE(q && k_new && v_new && k_cache && v_cache && kv_len && o && workspace, XV_ERR_NULL);
    XV_REQUIRE(xv_aligned16(q) && xv_aligned16(k_new) && xv_aligned16(v_new) &&
               xv_aligned16(k_cache) && xv_aligned16(v_cache) && xv_aligned(kv_len, 4) &&
               xv_aligned(o, 2) && xv_aligned(o32, 4) && xv_aligned16(workspace), XV_ERR_ALIGN);
    size_t acc_bytes = 0;
    const size_t need = xv_attn_ws(B, T, Hq, d, Lmax, &acc_bytes);
    XV_REQUIRE(workspace_bytes >= need, XV_ERR_WORKSPACE);
    const int NC = (Lmax + XV_ATTN_C - 1) / XV_ATTN_C;
    float* ws_acc = reinterpret_cast<float*>(workspace);
    float* ws_ml = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + acc_bytes);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    switch (d) {
        case 64:  return xv_attn_launch<64>(q, k_new, v_new, k_cache, v_cache, kv_len, o, o32, ws_acc,
                                            ws_ml, B, T, Hq, Hkv, Lmax, NC, scale, st);
        case 128: return xv_attn_launch<128>(q, k_new, v_new, k_cache, v_cache, kv_len, o, o32, ws_acc,
                                             ws_ml, B, T, Hq, Hkv, Lmax, NC, scale, st);
        default:  return xv_attn_launch<256>(q, k_new, v_new, k_cache, v_cache, kv_len, o, o32, ws_acc,
                                             ws_ml, B, T, Hq, Hkv, Lmax, NC, scale, st);
    }
}
