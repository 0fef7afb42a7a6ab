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
//         s_j = (q . k_j) * (scale * log2 e) (bf16 MFMA, fp32 accumulate; log2 units)
//         m_c = max_j s_j over visible j     (exact)
//         p_j = 2^(s_j - m_c), 0 for masked j
//         l_c = sum_j p_j                    (fixed order: in-lane ascending,
//                                             then lane butterfly 16, 32)
//         acc_c = sum_j p_j v_j              (MFMA with p split into bf16 hi + lo)
//     Scores are computed transposed (S^T = K Q^T) so that each lane already
//     holds the probabilities of its pair in the order the P.V MFMA consumes
//     them.  A wave owns 16 pairs (one tile); when there are fewer tiles than
//     waves, the tiles' P.V output dims are split over the spare waves (each
//     output column is still one MFMA chain over the same k-slots).
//  2. xv_attn_combine_kernel, grid (query head, row, request): with
//     M = max_c m_c, beta_c = 2^(m_c - M), L = sum_c l_c beta_c and
//     A = sum_c acc_c beta_c in ascending chunk order; o = A / L, stored as
//     bf16 (nearest even) and optionally fp32.
// Masked positions are excluded by index, never by value, and positions at or
// past L0 + T are never read (their LDS slots are zero-filled).
#include "xv_common.h"
#include <math.h>

namespace {

constexpr int XV_ATTN_C = 256;      // chunk length (positions), fixed for every call
constexpr int XV_ATTN_WAVES = 8;    // 16 pairs per wave -> up to 128 (head, row) pairs
constexpr int XV_ATTN_MAX_NC = 8192;

// LDS layouts (16-byte granules, XOR-swizzled so that both the cooperative
// stores and the MFMA fragment reads spread over the banks):
//   K  : [pos][d]  granule (pos, c = d/8)   at pos * (D/8) + (c ^ (pos & 7))
//   V^T: [d][pos]  granule (d, c = pos/8)   at d * (C/8) + (c ^ ((d ^ (d >> 3)) & 7))
template <int D>
__device__ __forceinline__ int xv_k_granule(int pos, int c) { return pos * (D / 8) + (c ^ (pos & 7)); }
__device__ __forceinline__ int xv_vt_granule(int d, int c) {
    return d * (XV_ATTN_C / 8) + (c ^ ((d ^ (d >> 3)) & 7));
}

template <int D>
__global__ __launch_bounds__(XV_ATTN_WAVES * 64)
void xv_attn_partial_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_new,
                            const uint16_t* __restrict__ v_new, uint16_t* __restrict__ k_cache,
                            uint16_t* __restrict__ v_cache, const int32_t* __restrict__ kv_len,
                            float* __restrict__ ws_acc, float* __restrict__ ws_ml,
                            int T, int Hq, int Hkv, int Lmax, int NC, float scale_log2)
{
    constexpr int C = XV_ATTN_C;
    constexpr int NT = XV_ATTN_WAVES * 64;
    constexpr int KS = D / 32;                  // MFMA k-steps over the head dim
    constexpr int DB = D / 16;                  // 16-wide blocks of output dims
    constexpr int NCB = C / 16;                 // 16-position score blocks per chunk
    constexpr int KG = C * (D / 8) / NT;        // K granules per thread
    constexpr int VTILES = (C / 8) * (D / 8);   // 8 x 8 V tiles per chunk
    constexpr int VT = (VTILES + NT - 1) / NT;  // V tiles per thread (last may be partial)
    __shared__ __attribute__((aligned(16))) xv_u32x4 lds[C * D / 8];

    const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int Hg = Hq / Hkv;
    const int P = Hg * T;
    int L0 = kv_len[b];
    L0 = L0 < 0 ? 0 : (L0 > Lmax - T ? Lmax - T : L0);
    const int Lend = L0 + T;
    const int c0 = c * C;
    if (c0 >= Lend) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    // waves -> (pair tile, slice of the output dims)
    const int ntiles = (P + 15) / 16;
    const int dsplit = 1;                       // one wave owns a tile's whole output
    const int tile = wave / dsplit, dq = wave % dsplit;
    const int dbw = DB / dsplit;                // output-dim blocks of this wave
    const bool tile_on = tile < ntiles;
    const int pair = tile * 16 + lr;            // the pair whose scores this lane holds
    const bool pair_ok = pair < P;
    const int pr = pair_ok ? pair / Hg : 0;
    const int ph = g * Hg + (pair_ok ? pair % Hg : 0);
    const int plen = L0 + pr + 1;
    const bool full = c0 + C <= L0 + 1;         // every position visible to every row

    const size_t kvbase = ((size_t)b * Hkv + g) * Lmax;
    const xv_u32x4 zero = {0u, 0u, 0u, 0u};

    // ---- issue every load of the chunk at once: K granules, V 8x8 tiles, Q ----
    // Loads are straight-line: a position in [L0, L0 + T) reads the new row, one
    // before L0 the cache, one past L0 + T re-reads cache position 0 (never used,
    // zeroed below).  The new rows are appended to the cache afterwards.
    auto src_row = [&](const uint16_t* cache, const uint16_t* fresh, int pos) -> const uint16_t* {
        if (pos < L0) return cache + (kvbase + pos) * D;
        if (pos < Lend) return fresh + (((size_t)b * T + (pos - L0)) * Hkv + g) * D;
        return cache + kvbase * D;
    };
    xv_u32x4 kreg[KG];
#pragma unroll
    for (int i = 0; i < KG; ++i) {
        const int idx = tid + i * NT;
        const int pos = c0 + idx / (D / 8), cc = idx % (D / 8);
        kreg[i] = xv_load16(src_row(k_cache, k_new, pos) + cc * 8);
    }
    xv_u32x4 vreg[VT][8];
#pragma unroll
    for (int i = 0; i < VT; ++i) {
        const int tile = (tid + i * NT) < VTILES ? tid + i * NT : VTILES - 1;
        const int pg = tile / (D / 8), dg = tile % (D / 8);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            vreg[i][e] = xv_load16(src_row(v_cache, v_new, c0 + pg * 8 + e) + dg * 8);
    }
    xv_u32x4 qf[KS];
    {
        const uint16_t* qp = q + (((size_t)b * T + pr) * Hq + ph) * D + lg * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[ks] = xv_load16(qp + ks * 32);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[ks] = pair_ok ? qf[ks] : zero;
    }
#pragma unroll
    for (int i = 0; i < KG; ++i) {                       // zero past L0 + T; append new rows
        const int idx = tid + i * NT;
        const int pos = c0 + idx / (D / 8), cc = idx % (D / 8);
        if (pos >= Lend) kreg[i] = zero;
        else if (pos >= L0) xv_store16(k_cache + (kvbase + pos) * D + cc * 8, kreg[i]);
    }
#pragma unroll
    for (int i = 0; i < VT; ++i) {
        const int tile = tid + i * NT;
        const int pg = tile / (D / 8), dg = tile % (D / 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int pos = c0 + pg * 8 + e;
            if (pos >= Lend || tile >= VTILES) vreg[i][e] = zero;
            else if (pos >= L0) xv_store16(v_cache + (kvbase + pos) * D + dg * 8, vreg[i][e]);
        }
    }

    // ---- K into LDS; scores S^T[pos][pair] for the whole chunk ----
#pragma unroll
    for (int i = 0; i < KG; ++i) {
        const int idx = tid + i * NT;
        lds[xv_k_granule<D>(idx / (D / 8), idx % (D / 8))] = kreg[i];
    }
    __syncthreads();
    xv_f32x4 sc[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) sc[cb] = xv_f32x4{0.f, 0.f, 0.f, 0.f};
    if (tile_on) {
        // per score block: one MFMA chain over ks ascending; the 16 chains are interleaved
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
                sc[cb] = xv_mfma16x16x32(lds[xv_k_granule<D>(cb * 16 + lr, ks * 4 + lg)], qf[ks], sc[cb]);
    }

    // ---- chunk max, probabilities, chunk sum (per pair, fixed order) ----
    float m = -INFINITY;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float sv = sc[cb][i] * scale_log2;
            sc[cb][i] = sv;
            if (full || c0 + cb * 16 + 4 * lg + i < plen) m = fmaxf(m, sv);
        }
    m = fmaxf(m, __shfl_xor(m, 16));
    m = fmaxf(m, __shfl_xor(m, 32));
    if (!pair_ok) m = 0.f;                      // lanes of padding pairs: keep finite
    float l = 0.f;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool vis = full || c0 + cb * 16 + 4 * lg + i < plen;
            const float pv = vis ? __builtin_amdgcn_exp2f(sc[cb][i] - m) : 0.f;
            sc[cb][i] = pv;
            l = l + pv;
        }
    l = l + __shfl_xor(l, 16);
    l = l + __shfl_xor(l, 32);

    // ---- V^T into LDS (8 x 8 register transposes), then acc = P V ----
    __syncthreads();                            // every wave is done reading K
#pragma unroll
    for (int i = 0; i < VT; ++i) {
        const int tile = tid + i * NT;
        if (tile < VTILES) {
            const int pg = tile / (D / 8), dg = tile % (D / 8);
#pragma unroll
            for (int dd = 0; dd < 8; ++dd) {
                xv_u32x4 outv;
#pragma unroll
                for (int w2 = 0; w2 < 4; ++w2) {
                    const uint32_t lo = vreg[i][2 * w2][dd >> 1], hi = vreg[i][2 * w2 + 1][dd >> 1];
                    outv[w2] = (dd & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u))
                                        : ((lo & 0xFFFFu) | (hi << 16));
                }
                lds[xv_vt_granule(dg * 8 + dd, pg)] = outv;
            }
        }
    }
    __syncthreads();
    xv_f32x4 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = xv_f32x4{0.f, 0.f, 0.f, 0.f};
    if (tile_on) {
        const char* ldsb = reinterpret_cast<const char*>(lds);
        const int half = (lg & 1) * 8;          // byte offset inside a 16-byte granule
#pragma unroll
        for (int kk = 0; kk < C / 32; ++kk) {
            // k-slot e of lane group lg <-> chunk position kk*32 + 4*lg + e (e < 4)
            //                                    or kk*32 + 16 + 4*lg + (e - 4)
            const xv_f32x4 pa = sc[kk * 2];
            const xv_f32x4 pb = sc[kk * 2 + 1];
            const float pe[8] = {pa[0], pa[1], pa[2], pa[3], pb[0], pb[1], pb[2], pb[3]};
            xv_u32x4 phi, plo;
#pragma unroll
            for (int w2 = 0; w2 < 4; ++w2) {
                const uint32_t h = xv_pack_bf16x2(pe[2 * w2], pe[2 * w2 + 1]);
                phi[w2] = h;
                plo[w2] = xv_pack_bf16x2(pe[2 * w2] - xv_bf16_lo(h), pe[2 * w2 + 1] - xv_bf16_hi(h));
            }
            const int ca = kk * 4 + (lg >> 1);      // granule of positions kk*32 + 4*lg ..
            // per output block: hi then lo; blocks of a group of 4 are interleaved
#pragma unroll
            for (int db0 = 0; db0 < DB; db0 += 4) {
                if (db0 / dbw != dq) continue;      // uniform per wave
                xv_u32x4 vf[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int d = (db0 + u) * 16 + lr;
                    const char* rowp = ldsb + (size_t)d * (C * 2) + half;
                    const int sw = (d ^ (d >> 3)) & 7;
                    const uint2 va = *reinterpret_cast<const uint2*>(rowp + ((ca ^ sw) << 4));
                    const uint2 vb = *reinterpret_cast<const uint2*>(rowp + (((ca + 2) ^ sw) << 4));
                    vf[u] = xv_u32x4{va.x, va.y, vb.x, vb.y};
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) oacc[db0 + u] = xv_mfma16x16x32(phi, vf[u], oacc[db0 + u]);
#pragma unroll
                for (int u = 0; u < 4; ++u) oacc[db0 + u] = xv_mfma16x16x32(plo, vf[u], oacc[db0 + u]);
            }
        }
    }

    // ---- write the chunk partials of pairs that see this chunk ----
    if (!tile_on) return;
    if (dq == 0 && lg == 0 && pair_ok && plen > c0) {
        const size_t idx = (((size_t)b * T + pr) * Hq + ph) * NC + c;
        ws_ml[idx * 2 + 0] = m;
        ws_ml[idx * 2 + 1] = l;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int pair2 = tile * 16 + 4 * lg + i;
        if (pair2 >= P) continue;
        const int r2 = pair2 / Hg;
        if (L0 + r2 + 1 <= c0) continue;
        const int h2 = g * Hg + pair2 % Hg;
        float* dst = ws_acc + ((((size_t)b * T + r2) * Hq + h2) * NC + c) * D + lr;
#pragma unroll
        for (int db = 0; db < DB; ++db)
            if (db / dbw == dq) dst[db * 16] = oacc[db][i];
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
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, off));
    if ((tid & 63) == 0) sred[tid >> 6] = mloc;
    __syncthreads();
    if (tid == 0) {
        float mm = sred[0];
        for (int i = 1; i < D / 64; ++i) mm = fmaxf(mm, sred[i]);
        sred[0] = mm;
    }
    __syncthreads();
    const float M = sred[0];
    for (int cc = tid; cc < nc; cc += D) {
        const float be = __builtin_amdgcn_exp2f(ws_ml[(base + cc) * 2] - M);
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
    // scores are kept in log2 units: s * log2(e), so that 2^(s' - m') = e^(s - m)
    const float scale_log2 = (float)((double)scale * 1.4426950408889634);
    hipLaunchKernelGGL(xv_attn_partial_kernel<D>, dim3(NC, Hkv, B), dim3(XV_ATTN_WAVES * 64), 0, st,
                       q, k_new, v_new, k_cache, v_cache, kv_len, ws_acc, ws_ml,
                       T, Hq, Hkv, Lmax, NC, scale_log2);
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
