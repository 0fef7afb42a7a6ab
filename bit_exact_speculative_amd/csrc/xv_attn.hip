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
//  1. A partial kernel over chunks of XV_ATTN_C positions at absolute
//     boundaries.  For each (query head, row) pair with a visible position in
//     the chunk it computes
//         s_j = (q . k_j) * (scale * log2 e) (bf16 MFMA, fp32 accumulate; log2 units)
//         m_c = max_j s_j over visible j     (exact)
//         p_j = 2^(s_j - m_c), 0 for masked j
//         l_c = sum_j p_j                    (fixed order: in-lane over positions
//                                             16 cb + 4 g + i ascending, then
//                                             lane butterfly 16, 32)
//         acc_c = sum_j p_j v_j              (MFMA with p split into bf16 hi + lo;
//                                             per 16 output dims one chain over
//                                             the chunk's k-slots, ascending)
//     Scores are computed transposed (S^T = K Q^T) so that each lane holds its
//     pair's probabilities in the order the P.V MFMA consumes them.  New rows
//     come from k_new/v_new and are appended to the cache by one workgroup.
//     Three kernels form exactly these numbers with different work splits:
//     xv_attn_partial_wide_kernel (workgroup per chunk, KV head and request,
//     wave per 16-pair tile), xv_attn_partial_tile_kernel (workgroup per
//     16-pair tile as well, the waves splitting its positions and output dims)
//     and xv_attn_stream_kernel (persistent workgroups streaming the chunk
//     groups of one KV head and request, for long contexts); the host picks by
//     grid size only, so a pair's bits never depend on it.
//  2. xv_attn_combine_kernel, grid (query head, row, request): the row's chunk
//     partials folded in two levels (xv_fold_factors): the chunks of each group
//     of XV_ATTN_G = 8 in ascending order with a running maximum, then the group
//     partials in ascending order the same way; o = A / L, stored as bf16
//     (nearest even) and optionally fp32.  The streaming kernel folds each
//     group's chunks itself and hands the combine group partials; the prefill
//     mode of the same kernel folds both levels for its rows.  Every form uses
//     the same operations in the same order.
// Masked positions are excluded by index, never by value, and positions at or
// past L0 + T are never read (their LDS slots are zero-filled).
#include "xv_common.h"
#include "xv_gdn_impl.h"
#include <math.h>
#include <mutex>

namespace {

constexpr int XV_ATTN_C = 256;      // chunk length (positions), fixed for every call
constexpr int XV_ATTN_WAVES = 8;    // waves of a partial-kernel workgroup
constexpr int XV_ATTN_MAX_NC = 4608;   // chunks of the capacity (1,179,648 positions), at most
constexpr int XV_ATTN_G = 8;           // chunks per group of the two-level fold (2048 positions)
constexpr int XV_ATTN_WIDE_MIN = 128; // (chunk, KV head, request) workgroups from which the wide kernel runs (also
                                      // when the per-tile split would take more than one round)
constexpr int XV_ATTN_STREAM_MIN = 1024; // ... and from which the persistent streaming kernel runs (about 4 chunks per CU)
constexpr int XV_COMBINE_U = 24;    // chunks per block of combine loads kept in flight
static_assert(XV_COMBINE_U % 4 == 0, "the long-row combine reads its per-chunk factors four at a time");
constexpr int XV_COMBINE_PRE = 8;   // chunks a short row's combine loads before its maximum
// arrival counters at the start of the workspace: the per-tile split folds its rows in the same
// launch when its (request, KV head, tile) groups are at most this many, else a combine follows
constexpr int XV_ATTN_COUNTERS = 1024;
constexpr size_t XV_ATTN_COUNTER_BYTES = XV_ATTN_COUNTERS * sizeof(int);
// GDN + attention in one launch while their workgroups are at most these multiples
// of the CU count (GDN with one, or else two, column groups per workgroup)
constexpr double XV_FUSE_ONE_COL = 1.0;
constexpr double XV_FUSE_TWO_COL = 1.0;
// the combine's per-chunk LDS arrays are padded to whole pairs of load blocks
__host__ __device__ constexpr int xv_combine_pad(int nc) { return (nc + 2 * XV_COMBINE_U - 1) / (2 * XV_COMBINE_U) * (2 * XV_COMBINE_U); }
// the long-row combine's LDS (three per-chunk arrays, three per-group arrays and a scan
// array of 256) stays within the 64 KB of dynamic LDS a launch gets without an attribute
static_assert(sizeof(float) * (3 * xv_combine_pad(XV_ATTN_MAX_NC) + 3 * xv_combine_pad(XV_ATTN_MAX_NC) / XV_ATTN_G + 256)
              <= 65536, "combine LDS");
static_assert((2 * XV_COMBINE_U) % XV_ATTN_G == 0, "a block of combine loads holds whole groups");

// LDS layouts (16-byte granules, XOR-swizzled so that both the cooperative
// stores and the MFMA fragment reads spread over the banks):
//   K  : [pos][d]  granule (pos, c = d/8)   at pos * (D/8) + (c ^ (pos & KX)), KX = 15 (7 at
//        d = 64): a score MFMA's K fragment (16 positions x 4 granules) then covers sixteen
//        16-byte bank groups, where pos & 7 left eight
//   V^T: [d][pos]  granule (d, c = pos/8)   at d * (C/8) + (c ^ ((d ^ (d >> 3)) & 7))
template <int D>
__device__ __forceinline__ int xv_k_granule(int pos, int c) {
    constexpr int KX = D / 8 > 16 ? 15 : D / 8 - 1;
    return pos * (D / 8) + (c ^ (pos & KX));
}
__device__ __forceinline__ int xv_vt_granule(int d, int c) {
    return d * (XV_ATTN_C / 8) + (c ^ ((d ^ (d >> 3)) & 7));
}

// One chunk of one request's KV head, staged through registers: every load is
// issued at once and is straight-line: a position in [L0, L0 + T) reads the new
// row, one before L0 the cache, one past L0 + T re-reads cache position 0 (never
// used, zeroed before it reaches LDS).  The new rows are appended to the cache
// after the loads.
template <int D, int NT, int DS = 1>
struct XvChunk {
    static constexpr int C = XV_ATTN_C;
    static constexpr int DV = D / DS;                  // value dims this workgroup stages
    static constexpr int KG = C * (D / 8) / NT;        // K granules per thread
    static constexpr int VTILES = (C / 8) * (DV / 8);  // 8 x 8 V tiles per chunk
    static constexpr int VT = (VTILES + NT - 1) / NT;  // V tiles per thread (last may be partial)
    xv_u32x4 kreg[KG];
    xv_u32x4 vreg[VT][8];
    int dg0 = 0;                                       // first 8-dim value group staged

    __device__ __forceinline__ void load(const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
                                         const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
                                         size_t kvbase, size_t newbase, int newstride, int L0, int Lend, int c0, int tid) {
        auto src = [&](const uint16_t* cache, const uint16_t* fresh, int pos) -> const uint16_t* {
            if (pos < L0) return cache + (kvbase + pos) * D;
            if (pos < Lend) return fresh + newbase + (size_t)(pos - L0) * newstride;
            return cache + kvbase * D;
        };
#pragma unroll
        for (int i = 0; i < KG; ++i) {
            const int idx = tid + i * NT;
            kreg[i] = xv_load16(src(k_cache, k_new, c0 + idx / (D / 8)) + (idx % (D / 8)) * 8);
        }
#pragma unroll
        for (int i = 0; i < VT; ++i) {
            const int vt = (tid + i * NT) < VTILES ? tid + i * NT : VTILES - 1;
            const int pg = vt / (DV / 8), dg = dg0 + vt % (DV / 8);
#pragma unroll
            for (int e = 0; e < 8; ++e) vreg[i][e] = xv_load16(src(v_cache, v_new, c0 + pg * 8 + e) + dg * 8);
        }
    }
    // zero the positions past L0 + T; append the new K rows (append_k) and the staged
    // dims of the new V rows (append_v)
    __device__ __forceinline__ void settle(uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache,
                                           size_t kvbase, int L0, int Lend, int c0, int tid,
                                           bool append_k, bool append_v) {
        const xv_u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < KG; ++i) {
            const int idx = tid + i * NT;
            const int pos = c0 + idx / (D / 8);
            if (pos >= Lend) kreg[i] = zero;
            else if (append_k && pos >= L0) xv_store16(k_cache + (kvbase + pos) * D + (idx % (D / 8)) * 8, kreg[i]);
        }
#pragma unroll
        for (int i = 0; i < VT; ++i) {
            const int vt = tid + i * NT;
            const int pg = vt / (DV / 8), dg = dg0 + vt % (DV / 8);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int pos = c0 + pg * 8 + e;
                if (pos >= Lend || vt >= VTILES) vreg[i][e] = zero;
                else if (append_v && pos >= L0) xv_store16(v_cache + (kvbase + pos) * D + dg * 8, vreg[i][e]);
            }
        }
    }
    __device__ __forceinline__ void k_to_lds(xv_u32x4* lds, int tid) const {
#pragma unroll
        for (int i = 0; i < KG; ++i) {
            const int idx = tid + i * NT;
            lds[xv_k_granule<D>(idx / (D / 8), idx % (D / 8))] = kreg[i];
        }
    }
    // V^T of the staged dims into LDS (rows d - 8*dg0) through 8 x 8 register transposes
    __device__ __forceinline__ void vt_to_lds(xv_u32x4* lds, int tid) const {
#pragma unroll
        for (int i = 0; i < VT; ++i) {
            const int vt = tid + i * NT;
            if (vt < VTILES) {
                const int pg = vt / (DV / 8), dg = vt % (DV / 8);
#pragma unroll
                for (int dd = 0; dd < 8; ++dd) {
                    xv_u32x4 outv;
#pragma unroll
                    for (int w2 = 0; w2 < 4; ++w2) {
                        const uint32_t lo = vreg[i][2 * w2][dd >> 1], hi = vreg[i][2 * w2 + 1][dd >> 1];
                        outv[w2] = (dd & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
                    }
                    lds[xv_vt_granule(dg * 8 + dd, pg)] = outv;
                }
            }
        }
    }
};

// The fold of partials (m, l, acc) in ascending order, with the running maximum M (-inf
// before the first):
//     M' = max(M, m),  a = 2^(M - M'),  b = 2^(m - M')
//     L  = fma(L, a, l b),  A = fma(A, a, acc b),  M = M'
// The first partial gives a = 0, b = 1: A = acc, L = l exactly.  A row's output is folded
// in two levels: the chunk partials of each group of XV_ATTN_G consecutive chunks (chunks
// 8 g .. 8 g + 7 that the row sees) are folded into a group partial (M_g, L_g, A_g), and the
// group partials, in ascending group order, into (M, L, A); o = A / L.  A row with at most
// one group gets exactly the fold of its chunks.  Whoever forms a level (the streaming
// kernel in registers, the combine from chunk or group partials, the prefill kernel) uses
// these operations in this order, so the bits never depend on who did.
__device__ __forceinline__ void xv_fold_factors(float& M, float m, float& a, float& b) {
    const float Mn = fmaxf(M, m);
    a = __builtin_amdgcn_exp2f(M - Mn);
    b = __builtin_amdgcn_exp2f(m - Mn);
    M = Mn;
}

// The P.V MFMA operands for k-slot group kk (chunk positions kk*32 ..): k-slot e
// of lane group lg is position kk*32 + 4*lg + e (e < 4) or kk*32 + 16 + 4*lg + (e - 4),
// which is where the transposed score MFMA left the lane's probabilities.
// A: the 8 probabilities as bf16 hi + lo (p = hi + lo to 16 bits).
__device__ __forceinline__ void xv_p_split(const xv_f32x4& pa, const xv_f32x4& pb, xv_u32x4& phi, xv_u32x4& plo) {
    const float pe[8] = {pa[0], pa[1], pa[2], pa[3], pb[0], pb[1], pb[2], pb[3]};
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) {
        const uint32_t h = xv_pack_bf16x2(pe[2 * w2], pe[2 * w2 + 1]);
        phi[w2] = h;
        plo[w2] = xv_pack_bf16x2(pe[2 * w2] - xv_bf16_lo(h), pe[2 * w2 + 1] - xv_bf16_hi(h));
    }
}
// B: V^T rows d = db*16 + lr at those positions.
__device__ __forceinline__ xv_u32x4 xv_vt_frag(const xv_u32x4* lds, int db, int kk, int lr, int lg) {
    const char* ldsb = reinterpret_cast<const char*>(lds);
    const int d = db * 16 + lr;
    const char* rowp = ldsb + (size_t)d * (XV_ATTN_C * 2) + (lg & 1) * 8;
    const int sw = (d ^ (d >> 3)) & 7;
    const int ca = kk * 4 + (lg >> 1);
    const uint2 va = *reinterpret_cast<const uint2*>(rowp + ((ca ^ sw) << 4));
    const uint2 vb = *reinterpret_cast<const uint2*>(rowp + (((ca + 2) ^ sw) << 4));
    return xv_u32x4{va.x, va.y, vb.x, vb.y};
}

// Store a wave's P.V output blocks db0 .. db0 + NB - 1 of pairs tile*16 + 4*lg + i.
// Partials are written with non-temporal (streaming) vector stores, and the long-row combine
// reads them the same way: each is read once, by the next kernel, and not keeping them in the
// caches leaves fewer dirty lines to be written back during the projections that follow
// (long context: 0.264 -> 0.261 ms per step).  AGENT: device-coherent stores instead, for a
// combine by another workgroup of the same launch (the per-tile split).
__device__ __forceinline__ void xv_store_agent(float* p, float v) {
    __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 xv_load2_agent(const float* p) {
    const uint64_t u = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    return make_float2(__uint_as_float((uint32_t)u), __uint_as_float((uint32_t)(u >> 32)));
}
template <int D, int NB, bool AGENT = false>
__device__ __forceinline__ void xv_store_acc(float* __restrict__ ws_acc, const xv_f32x4 (&oacc)[NB], int db0,
                                             int tile, int lr, int lg, int P, int Hg, int g, int b, int T,
                                             int Hq, int NC, int c, int L0, int c0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int pair = tile * 16 + 4 * lg + i;
        if (pair >= P) continue;
        const int r = pair / Hg;
        if (L0 + r + 1 <= c0) continue;             // the row sees nothing of this chunk
        const int h = g * Hg + pair % Hg;
        float* dst = ws_acc + ((((size_t)b * T + r) * Hq + h) * NC + c) * D + lr;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            if (AGENT) xv_store_agent(&dst[(db0 + j) * 16], oacc[j][i]);
            else __builtin_nontemporal_store(oacc[j][i], &dst[(db0 + j) * 16]);
        }
    }
}

// Many workgroups (large batch or long context): one workgroup per (chunk, KV
// head, request) serves every pair of the group, one 16-pair tile per wave: each
// wave computes all of its tile's scores and all output dims.
template <int D>
__global__ __launch_bounds__(XV_ATTN_WAVES * 64)
void xv_attn_partial_wide_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_new,
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
    const int tile = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const bool tile_on = tile < (P + 15) / 16;
    const int pair = tile * 16 + lr;            // the pair whose scores this lane holds
    const bool pair_ok = pair < P;
    const int pr = pair_ok ? pair / Hg : 0;
    const int ph = g * Hg + (pair_ok ? pair % Hg : 0);
    const int plen = L0 + pr + 1;
    const bool full = c0 + C <= L0 + 1;         // every position visible to every row
    const size_t kvbase = ((size_t)b * Hkv + g) * Lmax;
    const xv_u32x4 zero = {0u, 0u, 0u, 0u};

    XvChunk<D, NT> ch;
    ch.load(k_cache, v_cache, k_new, v_new, kvbase, ((size_t)b * T * Hkv + g) * D, Hkv * D, L0, Lend, c0, tid);
    xv_u32x4 qf[KS];
    {
        const uint16_t* qp = q + (((size_t)b * T + pr) * Hq + ph) * D + lg * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[ks] = xv_load16(qp + ks * 32);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[ks] = pair_ok ? qf[ks] : zero;
    }
    ch.settle(k_cache, v_cache, kvbase, L0, Lend, c0, tid, true, true);

    // ---- K into LDS; scores S^T[pos][pair] for the whole chunk ----
    ch.k_to_lds(lds, tid);
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

    // ---- V^T into LDS, then acc = P V: per output block one chain over k-slots, hi then lo ----
    __syncthreads();                            // every wave is done reading K
    ch.vt_to_lds(lds, tid);
    __syncthreads();
    if (!tile_on) return;
    xv_f32x4 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = xv_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < C / 32; ++kk) {
        xv_u32x4 phi, plo;
        xv_p_split(sc[kk * 2], sc[kk * 2 + 1], phi, plo);
        // blocks of a group of 4 are interleaved so dependent MFMAs never issue back to back
#pragma unroll
        for (int db0 = 0; db0 < DB; db0 += 4) {
            xv_u32x4 vf[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) vf[u] = xv_vt_frag(lds, db0 + u, kk, lr, lg);
#pragma unroll
            for (int u = 0; u < 4; ++u) oacc[db0 + u] = xv_mfma16x16x32(phi, vf[u], oacc[db0 + u]);
#pragma unroll
            for (int u = 0; u < 4; ++u) oacc[db0 + u] = xv_mfma16x16x32(plo, vf[u], oacc[db0 + u]);
        }
    }

    // ---- the chunk partials of pairs that see this chunk ----
    if (lg == 0 && pair_ok && plen > c0) {
        const size_t idx = (((size_t)b * T + pr) * Hq + ph) * NC + c;
        __builtin_nontemporal_store(m, &ws_ml[idx * 2 + 0]);
        __builtin_nontemporal_store(l, &ws_ml[idx * 2 + 1]);
    }
    xv_store_acc<D, DB>(ws_acc, oacc, 0, tile, lr, lg, P, Hg, g, b, T, Hq, NC, c, L0, c0);
}

// Streaming partial kernel, two modes over one body.
//  * Verify (PF = false, long contexts): persistent workgroups stream the chunk groups of
//    one (KV head, request), group x, x + WPG, x + 2 WPG, ... for workgroup x, the chunks
//    of a group in ascending order, and write one partial per group (the group's chunks
//    folded in registers).  A request whose groups would leave most of its WPG workgroups
//    idle (2 x groups <= WPG: a short row in a large cache) is streamed by chunks instead,
//    one chunk partial each (a group of one chunk is the chunk's partial, bit for bit);
//    xv_stream_grouped() is that choice, and the combine makes it again from the same
//    inputs.
//  * Prefill (PF = true): one workgroup per (request, KV head, block
//    of 64 (row, head) pairs) walks every chunk its last row sees, in ascending order, and
//    folds both levels in registers into the rows' outputs (no workspace).
// A chunk goes through LDS as four 64-position sub-blocks of K, then four of V^T; each
// sub-block is a "unit" loaded into registers two units before it is staged (the next
// chunk's K units while the current chunk's V is consumed), and staged into one of two LDS
// slots while the unit before it is consumed from the other (one barrier per unit), so HBM
// loads, LDS staging and the MFMA work overlap.  Up to 4 tiles of 16 pairs; waves t and t + 4
// share tile t: wave t forms the score blocks of the chunk's first half, wave t + 4 those
// of the second, the chunk max meets through LDS, the fp32 probabilities go through LDS one
// sub-block at a time (three slots), the chunk sum is one chain per lane that wave t runs
// over the first half and wave t + 4 continues, and each wave forms half of the tile's P.V
// output dims.  Every chain and ordered sum of a chunk is the wide kernel's, and the folds
// are the combine's operations in its order (xv_fold_factors), so every bit is the same as
// the per-chunk kernels followed by the combine.
constexpr int XV_ATTN_SB = 64;              // positions per streamed sub-block
constexpr int XV_ATTN_UNITS = 2;            // units in flight
constexpr int XV_ATTN_SPAIRS = 64;          // (row, head) pairs per workgroup: 4 tiles of 16

template <int D>
struct XvUnit {
    static constexpr int NT = XV_ATTN_WAVES * 64;
    static constexpr int KG = XV_ATTN_SB * (D / 8) / NT;           // K granules per thread
    static constexpr int VT4 = (XV_ATTN_SB / 4) * (D / 8);         // 4 x 8 V tiles per sub-block
    static_assert(KG >= 1 && KG <= 4 && VT4 <= NT, "unit split");
    xv_u32x4 r[4];                                                  // K: KG granules; V: one 4 x 8 tile
};

// whether the streaming kernel folds request b's chunks in groups of XV_ATTN_G (else it
// writes chunk partials): nchunks, the chunks the request's last row sees; wpg, the
// streaming grid's workgroups per (KV head, request)
__host__ __device__ inline bool xv_stream_grouped(int nchunks, int wpg) {
    return 2 * ((nchunks + XV_ATTN_G - 1) / XV_ATTN_G) > wpg;
}

struct XvStreamArgs {
    const uint16_t* q;          // [B][R][Hq][D]
    const uint16_t* k_new;      // verify: the rows to append, [B][R][Hkv][D]
    const uint16_t* v_new;
    uint16_t* k_cache;          // [B][Hkv][Lmax][D]
    uint16_t* v_cache;
    const int32_t* kv_len;      // [B]: cached length before the R rows
    float* ws_acc;              // verify: group partials [B][R][Hq][NG][D]
    float* ws_ml;               // verify: [B][R][Hq][NG][2] (max, sum)
    uint16_t* o;                // prefill: outputs [B][R][Hq][D]
    float* o32;
    int R;                      // rows per request (verify T, prefill P)
    int Hq, Hkv, Lmax;
    int NC, NG;                 // verify: chunks and groups of the capacity (the partials' strides)
    int NRB;                    // prefill: pair blocks per (request, KV head)
    float scale_log2;
};

template <int D, bool PF>
__global__ __launch_bounds__(XV_ATTN_WAVES * 64)
void xv_attn_stream_kernel(const XvStreamArgs A)
{
    constexpr int C = XV_ATTN_C;
    constexpr int G = XV_ATTN_G;
    constexpr int SB = XV_ATTN_SB;
    constexpr int NSB = C / SB;                 // sub-blocks per chunk
    constexpr int NT = XV_ATTN_WAVES * 64;
    constexpr int KS = D / 32;
    constexpr int DB = D / 16;
    constexpr int NCB = C / 16;
    constexpr int NU = XV_ATTN_UNITS;
    constexpr int CBS = SB / 16;                // score blocks per sub-block
    constexpr int CBH = NCB / 2;                // score blocks per wave
    constexpr int DBH = DB / 2;                 // output blocks per wave (half of the head dim)
    constexpr int PS = SB + 4;                  // probability row pitch of a sub-block slot (floats)
    constexpr int KG = XvUnit<D>::KG;
    constexpr int VT4 = XvUnit<D>::VT4;
    static_assert(NSB == 4 && 8 % NU == 0 && XV_ATTN_WAVES == 8, "four units per chunk half, unit k in buffer k % NU, two waves per tile");
    constexpr int QP = D + 8;                   // query row pitch in LDS (bf16)
    // two slots, each a K sub-block [pos][d] or a V^T sub-block [d][pos] (swizzled): unit u of a
    // chunk (K sub-blocks 0..3, then V^T sub-blocks 0..3) is staged into slot u % 2 while unit
    // u - 1 is consumed from the other
    __shared__ __attribute__((aligned(16))) xv_u32x4 skv[2][SB * D / 8];
    // the probabilities of one sub-block per slot, [tile][pair][pos]: sub-block v in slot v % 3
    __shared__ __attribute__((aligned(16))) float sp[3][4 * 16 * PS];
    __shared__ __attribute__((aligned(16))) uint16_t sq[4 * 16 * QP];   // the 4 tiles' queries
    __shared__ float smax[XV_ATTN_WAVES][16];
    __shared__ float sl[4][64];                 // a tile's chunk-sum chains, wave t -> t + 4 -> t

    const int Hg = A.Hq / A.Hkv;
    const int Ptot = Hg * A.R;
    int g, b, pair0;
    if constexpr (PF) {                         // the blocks of the last rows (most chunks) first
        const int bid = (int)blockIdx.x;
        pair0 = (A.NRB - 1 - bid % A.NRB) * XV_ATTN_SPAIRS;
        g = (bid / A.NRB) % A.Hkv;
        b = bid / (A.NRB * A.Hkv);
    } else {
        pair0 = 0;
        g = blockIdx.y;
        b = blockIdx.z;
    }
    int L0 = A.kv_len[b];
    L0 = L0 < 0 ? 0 : (L0 > A.Lmax - A.R ? A.Lmax - A.R : L0);
    const int Lend = L0 + A.R;
    const int npair = Ptot - pair0 < XV_ATTN_SPAIRS ? Ptot - pair0 : XV_ATTN_SPAIRS;
    const int first_len = L0 + pair0 / Hg + 1;                  // every pair sees the positions below
    const int nchunks = (L0 + (pair0 + npair - 1) / Hg + 1 + C - 1) / C;   // chunks the last row sees
    // this workgroup's chunks, in order: verify, the chunks of its groups (gs = log2 of the
    // group size: 3, or 0 for chunk partials); prefill, all of them, in groups of G
    int x = 0, WPG = 1, nitems, gs = 3, NI = 0;
    if constexpr (PF) {
        nitems = nchunks;
    } else {
        x = (int)blockIdx.x;
        WPG = (int)gridDim.x;
        gs = xv_stream_grouped(nchunks, WPG) ? 3 : 0;
        NI = gs ? A.NG : A.NC;
        const int ge = 1 << gs;
        const int ngr = (nchunks + ge - 1) >> gs;
        if (x >= ngr) return;                   // uniform
        const int ngw = (ngr - 1 - x) / WPG + 1;
        const int lastg = x + (ngw - 1) * WPG;
        nitems = ((ngw - 1) << gs) + (nchunks - (lastg << gs) < ge ? nchunks - (lastg << gs) : ge);
    }
    static_assert(G == 8, "group size 1 << 3");
    auto chunk_of = [&](int it) __attribute__((always_inline)) -> int {
        if constexpr (PF) return it;
        else return ((x + (it >> gs) * WPG) << gs) + (it & ((1 << gs) - 1));
    };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int tile = wave & 3;
    const int dh = wave >> 2;                   // which half of the score blocks and of the dims
    const int lr = lane & 15, lg = lane >> 4;
    const bool tile_on = tile * 16 < npair;
    const int tlast = pair0 + (tile * 16 + 15 < npair ? tile * 16 + 15 : npair - 1);
    const int tlen = L0 + tlast / Hg + 1;       // the tile's last row: it sees a chunk when that row does
    const int pl = tile * 16 + lr;              // this lane's score pair
    const bool pair_ok = pl < npair;
    const int gp = pair0 + (pair_ok ? pl : 0);
    const int pr = gp / Hg;
    const int ph = g * Hg + gp % Hg;
    const int plen = L0 + pr + 1;
    // this lane's output pairs tile*16 + 4 lg + i
    int orow[4], ohead[4];
    bool ook[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int ol = tile * 16 + 4 * lg + i;
        ook[i] = ol < npair;
        const int og = pair0 + (ook[i] ? ol : 0);
        orow[i] = og / Hg;
        ohead[i] = g * Hg + og % Hg;
    }
    const size_t kvbase = ((size_t)b * A.Hkv + g) * A.Lmax;
    const size_t newbase = ((size_t)b * A.R * A.Hkv + g) * D;
    const int newstride = A.Hkv * D;
    const xv_u32x4 zero = {0u, 0u, 0u, 0u};

    // verify: positions before L0 from the cache, the new rows from k_new / v_new; prefill:
    // every visible position from the cache (its rows were appended first).  Past L0 + R:
    // cache position 0 (never used, zeroed before it reaches LDS).
    auto src = [&](const uint16_t* cache, const uint16_t* fresh, int pos) __attribute__((always_inline)) -> const uint16_t* {
        if constexpr (PF) {
            (void)fresh;
            return cache + (kvbase + (pos < Lend ? pos : 0)) * D;
        } else {
            if (pos < L0) return cache + (kvbase + pos) * D;
            if (pos < Lend) return fresh + newbase + (size_t)(pos - L0) * newstride;
            return cache + kvbase * D;
        }
    };
    // this thread's granules of a unit, as element offsets from the unit's first cache row:
    // K granule i is position idx / (D/8), dims (idx % (D/8)) * 8 (idx = tid + i NT); V: a 4 x 8
    // tile, positions pg4 * 4 .. + 3, dims dg * 8 ..
    int koff[KG];
#pragma unroll
    for (int i = 0; i < KG; ++i) {
        const int idx = tid + i * NT;
        koff[i] = (idx / (D / 8)) * D + (idx % (D / 8)) * 8;
    }
    const int vtc = tid < VT4 ? tid : VT4 - 1;
    const int voff = (vtc / (D / 8)) * 4 * D + (vtc % (D / 8)) * 8;
    // a unit whose 64 positions all precede the new rows (verify) or the end of the rows
    // (prefill) is read straight from the cache: one base for the workgroup, no per-position
    // choice, no zeroing, no append
    const int plain_end = PF ? Lend : L0;
    // unit u of item it: u < 4 is K sub-block u, u >= 4 is V sub-block u - 4
    auto load_unit = [&](XvUnit<D>& U, int it, int u) __attribute__((always_inline)) {
        const int p0 = chunk_of(it) * C + (u & 3) * SB;
        if (p0 + SB <= plain_end) {             // uniform
            const uint16_t* base = (u < 4 ? A.k_cache : A.v_cache) + (kvbase + p0) * D;
            if (u < 4) {
#pragma unroll
                for (int i = 0; i < KG; ++i) U.r[i] = PF ? xv_load16(base + koff[i]) : xv_load16_nt(base + koff[i]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    U.r[e] = PF ? xv_load16(base + voff + e * D) : xv_load16_nt(base + voff + e * D);
            }
            return;
        }
        if (u < 4) {
#pragma unroll
            for (int i = 0; i < KG; ++i) {
                const int idx = tid + i * NT;
                U.r[i] = xv_load16(src(A.k_cache, A.k_new, p0 + idx / (D / 8)) + (idx % (D / 8)) * 8);
            }
        } else {
            const int vt = tid < VT4 ? tid : VT4 - 1;
            const int pg4 = vt / (D / 8), dg = vt % (D / 8);
#pragma unroll
            for (int e = 0; e < 4; ++e) U.r[e] = xv_load16(src(A.v_cache, A.v_new, p0 + pg4 * 4 + e) + dg * 8);
        }
    };
    // into LDS: positions past L0 + R zeroed; verify appends the new rows to the cache
    auto store_unit = [&](XvUnit<D>& U, int it, int u, xv_u32x4* slot) __attribute__((always_inline)) {
        const int p0 = chunk_of(it) * C + (u & 3) * SB;
        const bool plain = p0 + SB <= plain_end;     // uniform
        if (u < 4) {
#pragma unroll
            for (int i = 0; i < KG; ++i) {
                const int idx = tid + i * NT;
                const int lp = idx / (D / 8), cc = idx % (D / 8);
                const int pos = p0 + lp;
                if (!plain) {
                    if (pos >= Lend) U.r[i] = zero;
                    else if (!PF && pos >= L0) xv_store16(A.k_cache + (kvbase + pos) * D + cc * 8, U.r[i]);
                }
                slot[xv_k_granule<D>(lp, cc)] = U.r[i];
            }
        } else if (tid < VT4) {
            // a 4 (positions) x 8 (dims) tile -> for each of its 8 dims, 4 positions of V^T (8 bytes)
            const int pg4 = tid / (D / 8), dg = tid % (D / 8);
            if (!plain) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int pos = p0 + pg4 * 4 + e;
                    if (pos >= Lend) U.r[e] = zero;
                    else if (!PF && pos >= L0) xv_store16(A.v_cache + (kvbase + pos) * D + dg * 8, U.r[e]);
                }
            }
            char* vb = reinterpret_cast<char*>(slot);
#pragma unroll
            for (int dd = 0; dd < 8; ++dd) {
                const uint32_t a0 = U.r[0][dd >> 1], a1 = U.r[1][dd >> 1];
                const uint32_t a2 = U.r[2][dd >> 1], a3 = U.r[3][dd >> 1];
                uint2 outv;
                outv.x = (dd & 1) ? ((a0 >> 16) | (a1 & 0xFFFF0000u)) : ((a0 & 0xFFFFu) | (a1 << 16));
                outv.y = (dd & 1) ? ((a2 >> 16) | (a3 & 0xFFFF0000u)) : ((a2 & 0xFFFFu) | (a3 << 16));
                const int d = dg * 8 + dd;
                const int gi = d * (SB / 8) + ((pg4 >> 1) ^ ((d ^ (d >> 3)) & 7));
                *reinterpret_cast<uint2*>(vb + gi * 16 + (pg4 & 1) * 8) = outv;
            }
        }
    };

    // the 4 tiles' queries into LDS (rows of pairs past the block are zero); visible after the first barrier
    {
        constexpr int QG = (4 * 16 * (D / 8) + NT - 1) / NT;
#pragma unroll
        for (int i = 0; i < QG; ++i) {
            const int e = tid + i * NT;
            if (e < 4 * 16 * (D / 8)) {
                const int p2 = e / (D / 8), cc = e % (D / 8);
                const int gq = pair0 + (p2 < npair ? p2 : 0);
                const xv_u32x4 v = xv_load16(A.q + (((size_t)b * A.R + gq / Hg) * A.Hq + g * Hg + gq % Hg) * D + cc * 8);
                *reinterpret_cast<xv_u32x4*>(sq + p2 * QP + cc * 8) = p2 < npair ? v : zero;
            }
        }
    }
    const uint16_t* const qrow = sq + (tile * 16 + lr) * QP + lg * 8;
    XvUnit<D> ub[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) load_unit(ub[u], 0, u);

    // the fold of the current group (and, prefill, of the groups so far): per score pair
    // (lane lr) the running maximum and sum, per output pair 4 lg + i the P.V sums
    float Mg = -INFINITY, Lg = 0.f, Mt = -INFINITY, Lt = 0.f;
    xv_f32x4 Ag[DBH], At[PF ? DBH : 1];
#pragma unroll
    for (int j = 0; j < DBH; ++j) Ag[j] = xv_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < (PF ? DBH : 1); ++j) At[j] = xv_f32x4{0.f, 0.f, 0.f, 0.f};

    // unit k of item it (k >= 8: unit k - 8 of the next item; past the last item the same unit
    // of this item again, a cache hit, so that every load is unconditional; never consumed)
    auto load_ahead = [&](XvUnit<D>& U, int it, int k) __attribute__((always_inline)) {
        if (k < 8) load_unit(U, it, k);
        else load_unit(U, it + 1 < nitems ? it + 1 : it, k - 8);
    };
    store_unit(ub[0], 0, 0, skv[0]);
    load_ahead(ub[0], 0, NU);
    __syncthreads();

    for (int it = 0; it < nitems; ++it) {
        const int c = chunk_of(it);
        const int c0 = c * C;
        const bool full = c0 + C <= first_len;
        const bool more = it + 1 < nitems;
        const bool tsee = tile_on && c0 < tlen;     // uniform per wave
        const int cb0 = dh * CBH;                   // this wave's half of the score blocks
        xv_f32x4 sc[CBH];
#pragma unroll
        for (int j = 0; j < CBH; ++j) sc[j] = xv_f32x4{0.f, 0.f, 0.f, 0.f};
        xv_f32x4 oacc[DBH];
#pragma unroll
        for (int j = 0; j < DBH; ++j) oacc[j] = xv_f32x4{0.f, 0.f, 0.f, 0.f};
        float m = 0.f, l = 0.f;
        // the probabilities of score blocks j (of this wave's half) into their sub-block's slot
        auto put_p = [&](int j) __attribute__((always_inline)) {
            const int cb = cb0 + j, sv = cb / CBS;
            float* const tp = sp[sv % 3] + tile * 16 * PS;
            *reinterpret_cast<xv_f32x4*>(tp + lr * PS + (cb % CBS) * 16 + 4 * lg) = sc[j];
        };

        // step u consumes unit u (slot u % 2) while unit u + 1 goes into the other slot, freed by
        // the barrier that ended step u - 1, and unit u + 1 + NU is loaded into its registers
#pragma unroll
        for (int u = 0; u < 2 * NSB; ++u) {
            if (u + 1 < 2 * NSB) {
                store_unit(ub[(u + 1) % NU], it, u + 1, skv[(u + 1) & 1]);
                load_ahead(ub[(u + 1) % NU], it, u + 1 + NU);
            } else {                                // the next item's first unit
                store_unit(ub[0], more ? it + 1 : it, 0, skv[0]);
                load_ahead(ub[0], more ? it + 1 : it, NU);
            }
            if (u < NSB) {
                // ---- this wave's half of the score blocks, one K sub-block at a time ----
                const xv_u32x4* const sk = skv[u & 1];
                if (tsee && (u * CBS) / CBH == dh) {        // uniform per wave
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {       // per score block one chain over ks
                        const xv_u32x4 qk = *reinterpret_cast<const xv_u32x4*>(qrow + ks * 32);
                        xv_u32x4 kf[CBS];
#pragma unroll
                        for (int j = 0; j < CBS; ++j) kf[j] = sk[xv_k_granule<D>(j * 16 + lr, ks * 4 + lg)];
#pragma unroll
                        for (int j = 0; j < CBS; ++j)
                            sc[(u * CBS) % CBH + j] = xv_mfma16x16x32(kf[j], qk, sc[(u * CBS) % CBH + j]);
                    }
                }
                if (u == NSB - 1) {                 // the chunk's scores complete: this wave's max
                    float mw = -INFINITY;
#pragma unroll
                    for (int j = 0; j < CBH; ++j)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float sv = sc[j][i] * A.scale_log2;
                            sc[j][i] = sv;
                            if (full || c0 + (cb0 + j) * 16 + 4 * lg + i < plen) mw = fmaxf(mw, sv);
                        }
                    mw = fmaxf(mw, __shfl_xor(mw, 16));
                    mw = fmaxf(mw, __shfl_xor(mw, 32));
                    if (lg == 0) smax[wave][lr] = mw;
                }
            } else {
                const int v = u - NSB;              // V^T sub-block v
                if (v == 0) {
                    // ---- chunk max over both waves (exact), probabilities; the chunk sum in the
                    // wide kernel's order: each lane's chain over score blocks 0 .. 15 (wave t
                    // runs 0 .. 7 and hands it to wave t + 4), then the two cross-lane levels ----
                    m = fmaxf(smax[tile][lr], smax[tile + 4][lr]);
                    if (!pair_ok) m = 0.f;
                    if (tsee) {
#pragma unroll
                        for (int j = 0; j < CBH; ++j)
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const bool vis = full || c0 + (cb0 + j) * 16 + 4 * lg + i < plen;
                                sc[j][i] = vis ? __builtin_amdgcn_exp2f(sc[j][i] - m) : 0.f;
                            }
                        if (dh == 0) {
#pragma unroll
                            for (int j = 0; j < CBH; ++j)
#pragma unroll
                                for (int i = 0; i < 4; ++i) l = l + sc[j][i];
                            sl[tile][lane] = l;
                        }
                        // sub-blocks 0 and 1 (waves 0-3) and 2 (waves 4-7); sub-block 3 after step 4
#pragma unroll
                        for (int j = 0; j < CBH; ++j)
                            if (dh == 0 || j < CBS) put_p(j);
                    }
                    __syncthreads();                // those probabilities and the chains visible
                    if (tsee && dh == 1) {
                        l = sl[tile][lane];
#pragma unroll
                        for (int j = 0; j < CBH; ++j)
#pragma unroll
                            for (int i = 0; i < 4; ++i) l = l + sc[j][i];
                        l = l + __shfl_xor(l, 16);
                        l = l + __shfl_xor(l, 32);
                        sl[tile][lane] = l;         // back to wave t, read after this step
                    }
                }
                if (v == 1 && tsee && dh == 1) {    // sub-block 3 into slot 0, which step 4 freed
#pragma unroll
                    for (int j = CBS; j < CBH; ++j) put_p(j);
                }
                // ---- acc = P V over this sub-block's two k-slot groups; this wave's half of the dims ----
                if (tsee) {
                    const char* const svt = reinterpret_cast<const char*>(skv[u & 1]);
                    const float* const tp = sp[v % 3] + tile * 16 * PS;
#pragma unroll
                    for (int k2 = 0; k2 < SB / 32; ++k2) {
                        xv_u32x4 phi, plo;
                        xv_p_split(*reinterpret_cast<const xv_f32x4*>(tp + lr * PS + k2 * 32 + 4 * lg),
                                   *reinterpret_cast<const xv_f32x4*>(tp + lr * PS + k2 * 32 + 16 + 4 * lg), phi, plo);
                        const int ca = k2 * 4 + (lg >> 1);
#pragma unroll
                        for (int j0 = 0; j0 < DBH; j0 += 4) {
                            constexpr int GW = DBH < 4 ? DBH : 4;
                            xv_u32x4 vf[GW];
#pragma unroll
                            for (int w4 = 0; w4 < GW; ++w4) {
                                const int d = (dh * DBH + j0 + w4) * 16 + lr;
                                const char* rowp = svt + (size_t)d * (SB * 2) + (lg & 1) * 8;
                                const int sw = (d ^ (d >> 3)) & 7;
                                const uint2 va = *reinterpret_cast<const uint2*>(rowp + ((ca ^ sw) << 4));
                                const uint2 vb = *reinterpret_cast<const uint2*>(rowp + (((ca + 2) ^ sw) << 4));
                                vf[w4] = xv_u32x4{va.x, va.y, vb.x, vb.y};
                            }
#pragma unroll
                            for (int w4 = 0; w4 < GW; ++w4) oacc[j0 + w4] = xv_mfma16x16x32(phi, vf[w4], oacc[j0 + w4]);
#pragma unroll
                            for (int w4 = 0; w4 < GW; ++w4) oacc[j0 + w4] = xv_mfma16x16x32(plo, vf[w4], oacc[j0 + w4]);
                        }
                    }
                }
            }
            __syncthreads();                        // unit u consumed, unit u + 1 staged
        }
        if (tsee && dh == 0) l = sl[tile][lane];    // the chunk sum from wave t + 4

        // ---- the chunk folded into its group, for the pairs that see it ----
        if (tsee) {
            float Mn = Mg, fa, fb;
            xv_fold_factors(Mn, m, fa, fb);
            const bool sees = pair_ok && plen > c0;
            if (sees) {
                Mg = Mn;
                Lg = __builtin_fmaf(Lg, fa, l * fb);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float ai = __shfl(fa, 4 * lg + i), bi = __shfl(fb, 4 * lg + i);
                const bool si = ook[i] && L0 + orow[i] + 1 > c0;
#pragma unroll
                for (int j = 0; j < DBH; ++j)
                    Ag[j][i] = si ? __builtin_fmaf(Ag[j][i], ai, oacc[j][i] * bi) : Ag[j][i];
            }
        }

        // ---- a group complete: verify writes its partial, prefill folds it into the total ----
        if ((c & ((1 << gs) - 1)) == (1 << gs) - 1 || !more) {
            const int gi = c >> gs;
            const int gc0 = (gi << gs) * C;
            if constexpr (!PF) {
                if (tile_on) {
                    if (lg == 0 && dh == 0 && pair_ok && plen > gc0) {
                        const size_t idx = (((size_t)b * A.R + pr) * A.Hq + ph) * NI + gi;
                        __builtin_nontemporal_store(Mg, &A.ws_ml[idx * 2 + 0]);
                        __builtin_nontemporal_store(Lg, &A.ws_ml[idx * 2 + 1]);
                    }
                    xv_store_acc<D, DBH>(A.ws_acc, Ag, dh * DBH, tile, lr, lg, Ptot, Hg, g, b, A.R, A.Hq, NI, gi, L0, gc0);
                }
            } else {
                if (tile_on) {
                    float Mn = Mt, fa, fb;
                    xv_fold_factors(Mn, Mg, fa, fb);
                    if (pair_ok && plen > gc0) {
                        Mt = Mn;
                        Lt = __builtin_fmaf(Lt, fa, Lg * fb);
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float ai = __shfl(fa, 4 * lg + i), bi = __shfl(fb, 4 * lg + i);
                        const bool si = ook[i] && L0 + orow[i] + 1 > gc0;
#pragma unroll
                        for (int j = 0; j < DBH; ++j)
                            At[j][i] = si ? __builtin_fmaf(At[j][i], ai, Ag[j][i] * bi) : At[j][i];
                    }
                }
            }
            Mg = -INFINITY;
            Lg = 0.f;
#pragma unroll
            for (int j = 0; j < DBH; ++j) Ag[j] = xv_f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }

    if constexpr (PF) {                         // o = A / L: this wave's half of the dims
        if (!tile_on) return;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float Li = __shfl(Lt, 4 * lg + i);
            if (!ook[i]) continue;
            const size_t ob = (((size_t)b * A.R + orow[i]) * A.Hq + ohead[i]) * D + lr;
#pragma unroll
            for (int j = 0; j < DBH; ++j) {
                const float ov = At[j][i] / Li;
                A.o[ob + (dh * DBH + j) * 16] = xv_f32_to_bf16(ov);
                if (A.o32) A.o32[ob + (dh * DBH + j) * 16] = ov;
            }
        }
    }
}

// Few workgroups (small batch, short context): one workgroup per (request, KV
// head, chunk, 16-pair tile, 1/DS of the value dims), so that the chunk's work is
// spread over more CUs.  The tile's queries are staged once in LDS; the waves
// split the tile's score blocks (every d-part workgroup forms all scores), the
// probabilities go through LDS, and each wave forms the output dims of its
// slice.  Every chain and ordered sum is the one the wide kernel forms, so the
// two give the same bits.
struct XvTileArgs {
    const uint16_t* q; const uint16_t* k_new; const uint16_t* v_new;
    uint16_t* k_cache; uint16_t* v_cache; const int32_t* kv_len;
    float* ws_acc; float* ws_ml;
    int T, Hq, Hkv, Lmax, NC, NTILE, items, per_xcd;
    int NCG;                    // chunks in the grid (NC, or fewer under a length bound); NC is the stride
    float scale_log2;
    uint16_t* o; float* o32;    // the rows' outputs (the in-launch combine)
    int* counters;              // arrival counters, one per (request, KV head, tile); zero between calls
};

template <int D>
struct XvTileSmem {
    static constexpr int PP = XV_ATTN_C + 4;    // probability row pitch (floats)
    static constexpr int QP = D + 8;            // query row pitch in LDS (bf16)
    xv_u32x4 lds[XV_ATTN_C * D / 8];
    float sp[16 * PP];
    uint16_t sq[16 * QP];
    float smax[XV_ATTN_WAVES][16];
    int last;
};

// The rows of one tile's pairs, the dims of one d-part, folded from their chunk partials
// exactly as xv_attn_combine_kernel folds them without DEEP (each group's chunks, then the
// groups, o = A / L), by the last of that (tile, d-part)'s chunk workgroups to finish.  The
// partials cross workgroups (and XCDs) through device-scope accesses only: relaxed
// agent-scope stores, completed (vmcnt 0) before the workgroup's barrier and its counter
// increment, and loads issued only by the workgroup that saw the final count; no cache
// write-back is needed.  Thread t: pair t / 32 of the tile, dims 2 (t % 32) + 64 e and the
// next of the d-part (each load instruction reads 256 contiguous bytes of a pair's
// partial).  GU: chunks whose loads are issued together (8, a whole group, or 4 when the
// tile's rows see at most 4 chunks; the chunks past a row are skipped either way).
template <int D, int DS, int GU>
__device__ __forceinline__ void xv_tile_combine(const XvTileArgs& A, int b, int g, int tile, int dpart, int L0)
{
    constexpr int C = XV_ATTN_C;
    constexpr int G = XV_ATTN_G;
    constexpr int E = D / DS / 64;              // dim pairs per thread
    static_assert(E >= 1 && GU <= G, "layout");
    const int tid = threadIdx.x;
    const int Hq = A.Hq, Hg = Hq / A.Hkv, T = A.T, NC = A.NC;
    const int pair = tile * 16 + (tid >> 5);
    if (pair >= Hg * T) return;                 // uniform per half wave
    const int pr = pair / Hg, ph = g * Hg + pair % Hg;
    const int nc = (L0 + pr + 1 + C - 1) / C;   // the row's chunks
    const int ng = (nc + G - 1) / G;
    const size_t base = (((size_t)b * T + pr) * Hq + ph) * NC;
    const int d0 = dpart * (D / DS) + 2 * (tid & 31);
    float M = -INFINITY, L = 0.f;
    float Ao[2 * E];
#pragma unroll
    for (int e = 0; e < 2 * E; ++e) Ao[e] = 0.f;
    for (int gi = 0; gi < ng; ++gi) {
        // the group's loads issued together; chunks past the row re-read the group's first
        float2 ml[GU], pa[GU][E];
#pragma unroll
        for (int u = 0; u < GU; ++u) {
            const int cc = gi * G + u < nc ? gi * G + u : gi * G;
            ml[u] = xv_load2_agent(A.ws_ml + (base + cc) * 2);
#pragma unroll
            for (int e = 0; e < E; ++e) pa[u][e] = xv_load2_agent(A.ws_acc + (base + cc) * D + d0 + 64 * e);
        }
        float Mg = -INFINITY, Lg = 0.f;
        float Ag[2 * E];
#pragma unroll
        for (int e = 0; e < 2 * E; ++e) Ag[e] = 0.f;
#pragma unroll
        for (int u = 0; u < GU; ++u) {
            if (gi * G + u < nc) {
                float fa, fb;
                xv_fold_factors(Mg, ml[u].x, fa, fb);
                Lg = __builtin_fmaf(Lg, fa, ml[u].y * fb);
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    Ag[2 * e] = __builtin_fmaf(Ag[2 * e], fa, pa[u][e].x * fb);
                    Ag[2 * e + 1] = __builtin_fmaf(Ag[2 * e + 1], fa, pa[u][e].y * fb);
                }
            }
        }
        float fa, fb;
        xv_fold_factors(M, Mg, fa, fb);
        L = __builtin_fmaf(L, fa, Lg * fb);
#pragma unroll
        for (int e = 0; e < 2 * E; ++e) Ao[e] = __builtin_fmaf(Ao[e], fa, Ag[e] * fb);
    }
    const size_t ob = (((size_t)b * T + pr) * Hq + ph) * D + d0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const float o0 = Ao[2 * e] / L, o1 = Ao[2 * e + 1] / L;
        *reinterpret_cast<uint32_t*>(A.o + ob + 64 * e) =
            (uint32_t)xv_f32_to_bf16(o0) | ((uint32_t)xv_f32_to_bf16(o1) << 16);
        if (A.o32) *reinterpret_cast<float2*>(A.o32 + ob + 64 * e) = make_float2(o0, o1);
    }
}

// workgroup bid of the tile grid (its items are laid out for the XCD round robin)
template <int D, int DS>
__device__ __forceinline__ void xv_attn_tile_body(const XvTileArgs A, int bid, XvTileSmem<D>& S)
{
    const uint16_t* __restrict__ q = A.q;
    const uint16_t* __restrict__ k_new = A.k_new;
    const uint16_t* __restrict__ v_new = A.v_new;
    uint16_t* __restrict__ k_cache = A.k_cache;
    uint16_t* __restrict__ v_cache = A.v_cache;
    const int32_t* __restrict__ kv_len = A.kv_len;
    float* __restrict__ ws_acc = A.ws_acc;
    float* __restrict__ ws_ml = A.ws_ml;
    const int T = A.T, Hq = A.Hq, Hkv = A.Hkv, Lmax = A.Lmax, NC = A.NC, NTILE = A.NTILE, NCG = A.NCG;
    const int items = A.items, per_xcd = A.per_xcd;
    const float scale_log2 = A.scale_log2;
    constexpr int C = XV_ATTN_C;
    constexpr int NW = XV_ATTN_WAVES;
    constexpr int NT = NW * 64;
    constexpr int KS = D / 32;
    constexpr int DB = D / 16;
    constexpr int DBP = DB / DS;                // output blocks of this d-part
    constexpr int NCB = C / 16;
    constexpr int CBW = NCB / NW;               // score blocks per wave
    constexpr int DBW = DBP >= NW ? DBP / NW : 1; // output blocks per wave (waves past DBP idle)
    constexpr int PP = C + 4;                   // probability row pitch (floats)
    constexpr int QP = D + 8;                   // query row pitch in LDS (bf16)
    constexpr int QG = (16 * (D / 8) + NT - 1) / NT;   // query granules per thread
    static_assert(NCB % NW == 0 && DB % DS == 0, "work must split evenly");
    xv_u32x4* lds = S.lds;
    float* sp = S.sp;
    uint16_t* sq = S.sq;
    float (*smax)[16] = S.smax;

    // work item: consecutive items (the tiles and d-parts of one chunk) share an XCD's L2
    const int u = (bid % 8) * per_xcd + bid / 8;
    if (u >= items) return;
    const int dpart = u % DS;
    const int tile = (u / DS) % NTILE;
    const int c = (u / (DS * NTILE)) % NCG;
    const int g = (u / (DS * NTILE * NCG)) % Hkv;
    const int b = u / (DS * NTILE * NCG * Hkv);
    const int Hg = Hq / Hkv;
    const int P = Hg * T;
    int L0 = kv_len[b];
    L0 = L0 < 0 ? 0 : (L0 > Lmax - T ? Lmax - T : L0);
    const int Lend = L0 + T;
    const int c0 = c * C;
    if (c0 >= Lend) return;                     // uniform over the workgroup

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int pair = tile * 16 + lr;            // the pair whose scores this lane holds
    const bool pair_ok = pair < P;
    const int pr = pair_ok ? pair / Hg : 0;
    const int ph = g * Hg + (pair_ok ? pair % Hg : 0);
    const int plen = L0 + pr + 1;
    const bool full = c0 + C <= L0 + 1;         // every position visible to every row
    const size_t kvbase = ((size_t)b * Hkv + g) * Lmax;
    const xv_u32x4 zero = {0u, 0u, 0u, 0u};

    XvChunk<D, NT, DS> ch;
    ch.dg0 = dpart * (D / 8 / DS);
    ch.load(k_cache, v_cache, k_new, v_new, kvbase, ((size_t)b * T * Hkv + g) * D, Hkv * D, L0, Lend, c0, tid);
    xv_u32x4 qreg[QG];                          // the tile's 16 query rows, one granule each
#pragma unroll
    for (int i = 0; i < QG; ++i) {
        int e = tid + i * NT;
        e = e < 16 * (D / 8) ? e : 0;
        const int p2 = tile * 16 + e / (D / 8);
        const int p2c = p2 < P ? p2 : 0;
        qreg[i] = xv_load16(q + (((size_t)b * T + p2c / Hg) * Hq + g * Hg + p2c % Hg) * D + (e % (D / 8)) * 8);
    }
    ch.settle(k_cache, v_cache, kvbase, L0, Lend, c0, tid, tile == 0 && dpart == 0, tile == 0);
#pragma unroll
    for (int i = 0; i < QG; ++i) {
        const int e = tid + i * NT;
        if (e < 16 * (D / 8)) {
            const int p2 = tile * 16 + e / (D / 8);
            *reinterpret_cast<xv_u32x4*>(sq + (e / (D / 8)) * QP + (e % (D / 8)) * 8) = p2 < P ? qreg[i] : zero;
        }
    }

    // ---- K into LDS; this wave's score blocks S^T[pos][pair] ----
    ch.k_to_lds(lds, tid);
    __syncthreads();
    xv_u32x4 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const xv_u32x4*>(sq + lr * QP + ks * 32 + lg * 8);
    const int cb0 = wave * CBW;
    xv_f32x4 sc[CBW];
#pragma unroll
    for (int j = 0; j < CBW; ++j) sc[j] = xv_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int j = 0; j < CBW; ++j)
            sc[j] = xv_mfma16x16x32(lds[xv_k_granule<D>((cb0 + j) * 16 + lr, ks * 4 + lg)], qf[ks], sc[j]);

    // ---- chunk max over every wave's blocks (exact), probabilities into LDS ----
    float mw = -INFINITY;
#pragma unroll
    for (int j = 0; j < CBW; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float sv = sc[j][i] * scale_log2;
            sc[j][i] = sv;
            if (full || c0 + (cb0 + j) * 16 + 4 * lg + i < plen) mw = fmaxf(mw, sv);
        }
    mw = fmaxf(mw, __shfl_xor(mw, 16));
    mw = fmaxf(mw, __shfl_xor(mw, 32));
    if (lg == 0) smax[wave][lr] = mw;
    __syncthreads();                            // also: every wave is done reading K
    float m = smax[0][lr];
#pragma unroll
    for (int w = 1; w < NW; ++w) m = fmaxf(m, smax[w][lr]);
    if (!pair_ok) m = 0.f;                      // lanes of padding pairs: keep finite
#pragma unroll
    for (int j = 0; j < CBW; ++j) {
        xv_f32x4 pv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool vis = full || c0 + (cb0 + j) * 16 + 4 * lg + i < plen;
            pv[i] = vis ? __builtin_amdgcn_exp2f(sc[j][i] - m) : 0.f;
        }
        *reinterpret_cast<xv_f32x4*>(sp + lr * PP + (cb0 + j) * 16 + 4 * lg) = pv;
    }
    ch.vt_to_lds(lds, tid);
    __syncthreads();

    // ---- chunk sum l (wave 0), in the wide kernel's order; every d-part forms the same (m, l)
    // and stores it (the same bits to the same place), so that each d-part's fold needs only
    // its own workgroups ----
    if (wave == 0) {
        float l = 0.f;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const xv_f32x4 pv = *reinterpret_cast<const xv_f32x4*>(sp + lr * PP + cb * 16 + 4 * lg);
#pragma unroll
            for (int i = 0; i < 4; ++i) l = l + pv[i];
        }
        l = l + __shfl_xor(l, 16);
        l = l + __shfl_xor(l, 32);
        if (lg == 0 && pair_ok && plen > c0) {
            const size_t idx = (((size_t)b * T + pr) * Hq + ph) * NC + c;
            xv_store_agent(&ws_ml[idx * 2 + 0], m);
            xv_store_agent(&ws_ml[idx * 2 + 1], l);
        }
    }

    // ---- acc = P V for this wave's output blocks ----
    const int dbl0 = wave * DBW;                // first block, local to the d-part
    if (dbl0 < DBP) {                           // uniform per wave
        xv_f32x4 oacc[DBW];
#pragma unroll
        for (int j = 0; j < DBW; ++j) oacc[j] = xv_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < C / 32; ++kk) {
            xv_u32x4 phi, plo;
            xv_p_split(*reinterpret_cast<const xv_f32x4*>(sp + lr * PP + kk * 32 + 4 * lg),
                       *reinterpret_cast<const xv_f32x4*>(sp + lr * PP + kk * 32 + 16 + 4 * lg), phi, plo);
            xv_u32x4 vf[DBW];
#pragma unroll
            for (int j = 0; j < DBW; ++j) vf[j] = xv_vt_frag(lds, dbl0 + j, kk, lr, lg);
#pragma unroll
            for (int j = 0; j < DBW; ++j) oacc[j] = xv_mfma16x16x32(phi, vf[j], oacc[j]);
#pragma unroll
            for (int j = 0; j < DBW; ++j) oacc[j] = xv_mfma16x16x32(plo, vf[j], oacc[j]);
        }
        xv_store_acc<D, DBW, true>(ws_acc, oacc, dpart * DBP + dbl0, tile, lr, lg, P, Hg, g, b, T, Hq, NC, c,
                                   L0, c0);
    }

    // ---- the combine of the tile's pairs, by the last of its chunk workgroups to finish ----
    if (!A.counters) return;                    // too many tiles: a combine launch follows
    __builtin_amdgcn_s_waitcnt(0x0F70);         // vmcnt(0): this thread's partial stores have completed
    __syncthreads();
    const int ncb = (Lend + C - 1) / C < NCG ? (Lend + C - 1) / C : NCG;   // chunk workgroups of the d-part
    int* cnt = A.counters + (((size_t)b * Hkv + g) * NTILE + tile) * DS + dpart;
    if (tid == 0) S.last = atomicAdd(cnt, 1) == ncb - 1;
    __syncthreads();
    if (!S.last) return;                        // uniform over the workgroup
    if (ncb <= 4) xv_tile_combine<D, DS, 4>(A, b, g, tile, dpart, L0);   // uniform
    else xv_tile_combine<D, DS, XV_ATTN_G>(A, b, g, tile, dpart, L0);
    if (tid == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D, int DS>
__global__ __launch_bounds__(XV_ATTN_WAVES * 64)
void xv_attn_partial_tile_kernel(XvTileArgs A)
{
    __shared__ __attribute__((aligned(16))) XvTileSmem<D> sm;
    xv_attn_tile_body<D, DS>(A, (int)blockIdx.x, sm);
}

// One workgroup per (query head, row, request), one thread per output dim.  The partials are
// chunk partials (the tile and wide kernels; STREAM = false), folded in two levels (each
// group's chunks, then the groups), or what the streaming kernel wrote for the request
// (STREAM = true): group partials, folded in ascending group order, or chunk partials,
// decided by xv_stream_grouped() from the same inputs.  NC, NG: the capacity's chunks and
// groups (the partials' strides); wpg: the streaming grid's workgroups per (KV head, request).
// Rows of at most XV_COMBINE_PRE partials (and every row when DEEP = false): every thread
// walks the chain itself, forming the factors from the (m, l) it loads (the first
// XV_COMBINE_PRE partials' loads issued together).  Longer rows when DEEP = true: the
// factors are formed once per partial in LDS (a running maximum as a prefix maximum: a
// per-thread segment, then a scan over the segments; a maximum is exact in any order), and
// the chain's loads run in two alternating register blocks of XV_COMBINE_U partials, one
// block in flight while the other is summed.  Every form folds the same operations in the
// same order.
template <int D, bool DEEP, bool STREAM>
__global__ __launch_bounds__(D)
void xv_attn_combine_kernel(const float* __restrict__ ws_acc, const float* __restrict__ ws_ml,
                            const int32_t* __restrict__ kv_len, uint16_t* __restrict__ o,
                            float* __restrict__ o32, int T, int Hq, int Lmax, int NC, int NG, int wpg)
{
    constexpr int G = XV_ATTN_G;
    const int h = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x;
    int L0 = kv_len[b];
    L0 = L0 < 0 ? 0 : (L0 > Lmax - T ? Lmax - T : L0);
    const int len = L0 + r + 1;
    const int nc = (len + XV_ATTN_C - 1) / XV_ATTN_C;
    const int ng = (nc + G - 1) / G;
    // group partials (uniform over the workgroup): as the streaming kernel chose for the request
    const bool grp = STREAM && xv_stream_grouped((L0 + T + XV_ATTN_C - 1) / XV_ATTN_C, wpg);
    const int NI = grp ? NG : NC;
    const int ni = grp ? ng : nc;               // this row's partials
    // LDS (DEEP): [NIP] a, [NIP] b, [NIP] l b (groups) or l (chunks), then (chunks) [NIP / G] x 3
    // group factors, then [D] scan
    extern __shared__ __attribute__((aligned(16))) float sh[];
    const int NIP = DEEP ? xv_combine_pad(NI) : NI;
    float* sa = sh;
    float* sb = sh + NIP;
    float* sl = sh + 2 * NIP;
    float* ga = sh + 3 * NIP;
    float* gb = ga + (grp ? 0 : NIP / G);
    float* gl = gb + (grp ? 0 : NIP / G);
    float* sred = gl + (grp ? 0 : NIP / G);
    const size_t base = (((size_t)b * T + r) * Hq + h) * NI;
    const float* ap = ws_acc + base * D + tid;
    float L = 0.f, A = 0.f;

    if (!DEEP || ni <= XV_COMBINE_PRE) {       // uniform
        // indices past ni re-read item ni - 1 and are not used
        constexpr int PRE = XV_COMBINE_PRE;
        static_assert(PRE == G, "the first block of loads is one group of chunks");
        float pacc[PRE];
        float2 pml[PRE];
        auto load_block = [&](int i0) __attribute__((always_inline)) {
#pragma unroll
            for (int u = 0; u < PRE; ++u) {
                const int cc = i0 + u < ni ? i0 + u : ni - 1;
                pacc[u] = ap[(size_t)cc * D];
                pml[u] = *reinterpret_cast<const float2*>(ws_ml + (base + cc) * 2);
            }
        };
        float M = -INFINITY;
        if (grp) {
            load_block(0);
#pragma unroll
            for (int u = 0; u < PRE; ++u) {
                if (u < ni) {
                    float fa, fb;
                    xv_fold_factors(M, pml[u].x, fa, fb);
                    L = __builtin_fmaf(L, fa, pml[u].y * fb);
                    A = __builtin_fmaf(A, fa, pacc[u] * fb);
                }
            }
#pragma unroll 4
            for (int cc = PRE; cc < ni; ++cc) {
                const float2 ml = *reinterpret_cast<const float2*>(ws_ml + (base + cc) * 2);
                float fa, fb;
                xv_fold_factors(M, ml.x, fa, fb);
                L = __builtin_fmaf(L, fa, ml.y * fb);
                A = __builtin_fmaf(A, fa, ap[(size_t)cc * D] * fb);
            }
        } else {
            for (int gi = 0; gi < ng; ++gi) {   // a group's chunk loads issued together
                load_block(gi * G);
                float Mg = -INFINITY, Lg = 0.f, Ag = 0.f;
#pragma unroll
                for (int u = 0; u < G; ++u) {
                    if (gi * G + u < nc) {
                        float fa, fb;
                        xv_fold_factors(Mg, pml[u].x, fa, fb);
                        Lg = __builtin_fmaf(Lg, fa, pml[u].y * fb);
                        Ag = __builtin_fmaf(Ag, fa, pacc[u] * fb);
                    }
                }
                float fa, fb;
                xv_fold_factors(M, Mg, fa, fb);
                L = __builtin_fmaf(L, fa, Lg * fb);
                A = __builtin_fmaf(A, fa, Ag * fb);
            }
        }
        (void)sa; (void)sb; (void)sl; (void)ga; (void)gb; (void)gl; (void)sred;
    } else {
        constexpr int U = XV_COMBINE_U;
        // indices past ni re-read item ni - 1 and are not summed
        auto fetch = [&](float (&buf)[U], int i0) __attribute__((always_inline)) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int cn = i0 + u;
                buf[u] = __builtin_nontemporal_load(&ap[(size_t)(cn < ni ? cn : ni - 1) * D]);
            }
        };
        // GRP: each item folds into the row's sums with its factors; chunks: each chunk
        // folds into its group's sum, and a group into the row's sums after its last chunk
        // (a block of loads holds whole groups); an item past ni leaves the sums as they are
        auto fold = [&](const float (&buf)[U], int i0) __attribute__((always_inline)) {
            if (grp) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const bool in = i0 + u < ni;
                    const float L2 = __builtin_fmaf(L, sa[i0 + u], sl[i0 + u]);
                    const float A2 = __builtin_fmaf(A, sa[i0 + u], buf[u] * sb[i0 + u]);
                    L = in ? L2 : L;
                    A = in ? A2 : A;
                }
            } else {
#pragma unroll
                for (int q = 0; q < U / G; ++q) {
                    float Ag = 0.f;
#pragma unroll
                    for (int u = 0; u < G; ++u) {
                        const int c = i0 + q * G + u;
                        const float A2 = __builtin_fmaf(Ag, sa[c], buf[q * G + u] * sb[c]);
                        Ag = c < nc ? A2 : Ag;
                    }
                    const int gi = (i0 + q * G) / G;
                    const bool in = gi < ng;
                    const float L2 = __builtin_fmaf(L, ga[gi], gl[gi]);
                    const float A2 = __builtin_fmaf(A, ga[gi], Ag * gb[gi]);
                    L = in ? L2 : L;
                    A = in ? A2 : A;
                }
            }
        };
        float ba[U], bbuf[U];
        fetch(ba, 0);                           // independent of the factors
        float mseg = -INFINITY;
        int s0, s1;                             // this thread's segment of items (chunks: whole groups)
        if (grp) {
            // (m, l) of the segment's groups: m into sa, l into sl; the segment's maximum
            const int seg = (ni + D - 1) / D;
            s0 = tid * seg;
            s1 = s0 + seg < ni ? s0 + seg : ni;
            for (int cc = s0; cc < s1; ++cc) {
                const float2 ml = *reinterpret_cast<const float2*>(ws_ml + (base + cc) * 2);
                sa[cc] = ml.x;
                sl[cc] = ml.y;
                mseg = fmaxf(mseg, ml.x);
            }
        } else {
            // the segment's groups: each chunk's factors within its group (into sa, sb), the
            // group's (M_g, L_g) (into ga, gl); the segment's maximum over the M_g
            const int seg = (ng + D - 1) / D;
            s0 = tid * seg;
            s1 = s0 + seg < ng ? s0 + seg : ng;
            for (int gi = s0; gi < s1; ++gi) {
                float Mg = -INFINITY, Lg = 0.f;
                const int c1 = (gi + 1) * G < nc ? (gi + 1) * G : nc;
                for (int cc = gi * G; cc < c1; ++cc) {
                    const float2 ml = *reinterpret_cast<const float2*>(ws_ml + (base + cc) * 2);
                    float fa, fb;
                    xv_fold_factors(Mg, ml.x, fa, fb);
                    sa[cc] = fa;
                    sb[cc] = fb;
                    Lg = __builtin_fmaf(Lg, fa, ml.y * fb);
                }
                ga[gi] = Mg;
                gl[gi] = Lg;
                mseg = fmaxf(mseg, Mg);
            }
        }
        sred[tid] = mseg;
        __syncthreads();
        // inclusive prefix maximum over the segments (exact)
        for (int off = 1; off < D; off <<= 1) {
            const float v = tid >= off ? fmaxf(sred[tid], sred[tid - off]) : sred[tid];
            __syncthreads();
            sred[tid] = v;
            __syncthreads();
        }
        // the row-level factors of this thread's items, from the maximum of every earlier one
        float M = tid > 0 ? sred[tid - 1] : -INFINITY;
        for (int cc = s0; cc < s1; ++cc) {
            float fa, fb;
            if (grp) {
                xv_fold_factors(M, sa[cc], fa, fb);
                sa[cc] = fa;
                sb[cc] = fb;
                sl[cc] = sl[cc] * fb;
            } else {
                xv_fold_factors(M, ga[cc], fa, fb);
                ga[cc] = fa;
                gb[cc] = fb;
                gl[cc] = gl[cc] * fb;
            }
        }
        __syncthreads();
        for (int i0 = 0; i0 < ni; i0 += 2 * U) {
            fetch(bbuf, i0 + U);
            fold(ba, i0);
            fetch(ba, i0 + 2 * U);
            fold(bbuf, i0 + U);
        }
    }
    const float ov = A / L;
    const size_t oi = (((size_t)b * T + r) * Hq + h) * D + tid;
    o[oi] = xv_f32_to_bf16(ov);
    if (o32) o32[oi] = ov;
}

// The partial kernel's work split for a call (a choice by grid size only: the
// three kernels give the same bits).
enum XvAttnKind { XV_ATTN_TILE, XV_ATTN_WIDE, XV_ATTN_STREAM };

inline long long xv_tile_items(int B, int T, int Hq, int Hkv, int NC, int ds);

template <int D>
XvAttnKind xv_attn_kind(int B, int T, int Hq, int Hkv, int NC) {
    // one workgroup per (chunk, KV head, request) when those alone fill the chip, or when one
    // per 16-pair tile of each would take more than one round of workgroups (batch 8, 3 chunks:
    // 384 tile workgroups, 30.1 us, against 27.6 us for the wide split and its combine);
    // otherwise one per tile; persistent streaming for long contexts
    const int P = (Hq / Hkv) * T;
    const long long groups = (long long)B * Hkv;
    if (D == 256 && groups * NC >= XV_ATTN_STREAM_MIN && P <= 64) return XV_ATTN_STREAM;
    if ((groups * NC >= XV_ATTN_WIDE_MIN || xv_tile_items(B, T, Hq, Hkv, NC, 1) > xv_cu_count()) &&
        P <= 16 * XV_ATTN_WAVES)
        return XV_ATTN_WIDE;
    return XV_ATTN_TILE;
}

// the streaming grid: about one persistent workgroup per CU, spread evenly over the (KV
// head, request) groups, at most one per chunk group of the capacity
inline int xv_stream_wpg(int B, int Hkv, int NC) {
    const long long groups = (long long)B * Hkv;
    const long long NG = (NC + XV_ATTN_G - 1) / XV_ATTN_G;
    long long wpg = xv_cu_count() / groups;
    wpg = wpg < 1 ? 1 : (wpg > NG ? NG : wpg);
    return (int)wpg;
}

// workgroups of the tile split: (request, KV head, chunk, 16-pair tile, value-dim part)
inline long long xv_tile_items(int B, int T, int Hq, int Hkv, int NC, int ds) {
    const long long ntile = ((long long)(Hq / Hkv) * T + 15) / 16;
    return (long long)B * Hkv * NC * ntile * ds;
}

// Value-dim parts per tile workgroup: at d = 256 two (each workgroup forms half of the
// output dims, so a chunk's work spreads over twice the CUs) when that grid, padded to the
// XCD round robin, leaves `room` CUs of the chip; otherwise one, which halves the grid
// (the work of a chunk on one CU instead of a second round of workgroups).  Both give the
// same bits.
inline int xv_attn_tile_ds(int D, int B, int T, int Hq, int Hkv, int NC, long long room) {
    if (D != 256) return 1;
    const long long n2 = 8 * ((xv_tile_items(B, T, Hq, Hkv, NC, 2) + 7) / 8);
    return n2 <= room ? 2 : 1;
}

// the per-tile split folds its rows in its own launch (each (request, KV head, tile,
// d-part) has a counter; at most 2 d-parts)
inline bool xv_tile_folds(int B, int T, int Hq, int Hkv) {
    return (long long)B * Hkv * (((Hq / Hkv) * T + 15) / 16) * 2 <= XV_ATTN_COUNTERS;
}

inline XvTileArgs xv_tile_args(int ds, const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                               uint16_t* k_cache, uint16_t* v_cache, const int32_t* kv_len,
                               float* ws_acc, float* ws_ml, int B, int T, int Hq, int Hkv, int Lmax, int NC,
                               int NCg, float scale_log2, uint16_t* o, float* o32, int* counters) {
    const int P = (Hq / Hkv) * T;
    const int ntile = (P + 15) / 16;
    const int items = (int)xv_tile_items(B, T, Hq, Hkv, NCg, ds);
    const int per_xcd = (items + 7) / 8;
    const bool fold = xv_tile_folds(B, T, Hq, Hkv);
    return XvTileArgs{q, k_new, v_new, k_cache, v_cache, kv_len, ws_acc, ws_ml,
                      T, Hq, Hkv, Lmax, NC, ntile, items, per_xcd, NCg, scale_log2, o, o32,
                      fold ? counters : nullptr};
}

// scores are kept in log2 units: s * log2(e), so that 2^(s' - m') = e^(s - m)
inline float xv_scale_log2(float scale) { return (float)((double)scale * 1.4426950408889634); }

// NC: the capacity's chunks (the partials' stride); NCg: the chunks any row can see (NC, or
// fewer under the caller's length bound), which sizes the grids and picks the kernels
// The per-tile split also forms the rows' outputs (its in-launch combine, o, o32, counters).
template <int D>
int xv_attn_partials(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                     uint16_t* k_cache, uint16_t* v_cache, const int32_t* kv_len,
                     float* ws_acc, float* ws_ml, uint16_t* o, float* o32, int* counters,
                     int B, int T, int Hq, int Hkv, int Lmax, int NC, int NCg, float scale, hipStream_t st)
{
    (void)hipGetLastError();
    const float scale_log2 = xv_scale_log2(scale);
    const XvAttnKind kind = xv_attn_kind<D>(B, T, Hq, Hkv, NCg);
    if (kind == XV_ATTN_STREAM) {
        const int NG = (NC + XV_ATTN_G - 1) / XV_ATTN_G;
        const XvStreamArgs sa{q, k_new, v_new, k_cache, v_cache, kv_len, ws_acc, ws_ml, nullptr, nullptr,
                              T, Hq, Hkv, Lmax, NC, NG, 0, scale_log2};
        hipLaunchKernelGGL((xv_attn_stream_kernel<D, false>), dim3(xv_stream_wpg(B, Hkv, NCg), Hkv, B),
                           dim3(XV_ATTN_WAVES * 64), 0, st, sa);
    } else if (kind == XV_ATTN_WIDE) {
        hipLaunchKernelGGL(xv_attn_partial_wide_kernel<D>, dim3(NCg, Hkv, B), dim3(XV_ATTN_WAVES * 64), 0, st,
                           q, k_new, v_new, k_cache, v_cache, kv_len, ws_acc, ws_ml,
                           T, Hq, Hkv, Lmax, NC, scale_log2);
    } else {
        const int ds = xv_attn_tile_ds(D, B, T, Hq, Hkv, NCg, xv_cu_count());
        const XvTileArgs ta = xv_tile_args(ds, q, k_new, v_new, k_cache, v_cache, kv_len, ws_acc, ws_ml,
                                           B, T, Hq, Hkv, Lmax, NC, NCg, scale_log2, o, o32, counters);
        if (D == 256 && ds == 2)
            hipLaunchKernelGGL((xv_attn_partial_tile_kernel<D, (D == 256 ? 2 : 1)>), dim3(8 * ta.per_xcd),
                               dim3(XV_ATTN_WAVES * 64), 0, st, ta);
        else
            hipLaunchKernelGGL((xv_attn_partial_tile_kernel<D, 1>), dim3(8 * ta.per_xcd), dim3(XV_ATTN_WAVES * 64),
                               0, st, ta);
    }
    return xv_launch_status();
}

// The combine for chunk partials (the tile and wide kernels) or for what the streaming
// kernel wrote (stream = true, its grid of wpg workgroups per (KV head, request)); NC is the
// capacity's chunk count.
template <int D>
int xv_attn_combine(const float* ws_acc, const float* ws_ml, const int32_t* kv_len, uint16_t* o, float* o32,
                    int B, int T, int Hq, int Lmax, int NC, int NCg, bool stream, int wpg, hipStream_t st)
{
    (void)hipGetLastError();
    const dim3 grid(Hq, T, B), block(D);
    const int NG = (NC + XV_ATTN_G - 1) / XV_ATTN_G;
    const size_t pad = xv_combine_pad(NC);
    const size_t shmem = sizeof(float) * (3 * pad + 3 * (pad / XV_ATTN_G) + D);   // either layout
    if (stream) {
        hipLaunchKernelGGL((xv_attn_combine_kernel<D, true, true>), grid, block, shmem, st,
                           ws_acc, ws_ml, kv_len, o, o32, T, Hq, Lmax, NC, NG, wpg);
    } else if (NCg > 2 * XV_COMBINE_U) {
        hipLaunchKernelGGL((xv_attn_combine_kernel<D, true, false>), grid, block, shmem, st,
                           ws_acc, ws_ml, kv_len, o, o32, T, Hq, Lmax, NC, NG, 0);
    } else {
        hipLaunchKernelGGL((xv_attn_combine_kernel<D, false, false>), grid, block, 0, st,
                           ws_acc, ws_ml, kv_len, o, o32, T, Hq, Lmax, NC, NG, 0);
    }
    return xv_launch_status();
}

template <int D>
int xv_attn_launch(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                   uint16_t* k_cache, uint16_t* v_cache, const int32_t* kv_len,
                   uint16_t* o, float* o32, float* ws_acc, float* ws_ml, int* counters,
                   int B, int T, int Hq, int Hkv, int Lmax, int NC, int NCg, float scale, hipStream_t st)
{
    const int s = xv_attn_partials<D>(q, k_new, v_new, k_cache, v_cache, kv_len, ws_acc, ws_ml, o, o32, counters,
                                      B, T, Hq, Hkv, Lmax, NC, NCg, scale, st);
    if (s != XV_OK) return s;
    const XvAttnKind kind = xv_attn_kind<D>(B, T, Hq, Hkv, NCg);
    if (kind == XV_ATTN_TILE && xv_tile_folds(B, T, Hq, Hkv)) return XV_OK;   // combined in that launch
    const bool stream = kind == XV_ATTN_STREAM;
    return xv_attn_combine<D>(ws_acc, ws_ml, kv_len, o, o32, B, T, Hq, Lmax, NC, NCg, stream,
                              stream ? xv_stream_wpg(B, Hkv, NCg) : 0, st);
}

// GDN and the attention partials side by side in one launch: workgroups
// 0 .. n_attn - 1 are the tile kernel's grid (so its XCD layout is unchanged),
// the rest the GDN grid (gdn_nx column slices x Hv x B).  The two share no data;
// each workgroup runs one body exactly as its own launch would (the same bits),
// in the larger of the two LDS layouts.  Both are latency-bound at small batch,
// so running them together takes about as long as the longer one.
template <int DK, int CPT, int D>
union XvGdnAttnSmem {
    XvGdnSmem<DK, CPT> g;
    XvTileSmem<D> t;
};

template <int DK, int CPT, int D, int DS>
__global__ __launch_bounds__(XV_ATTN_WAVES * 64)
void xv_gdn_attn_kernel(XvGdnArgs ga, XvTileArgs ta, int n_attn, int gdn_nx)
{
    static_assert(XV_GDN_THREADS == XV_ATTN_WAVES * 64, "one workgroup size for both bodies");
    __shared__ __attribute__((aligned(16))) XvGdnAttnSmem<DK, CPT, D> sm;
    const int bid = (int)blockIdx.x;
    if (bid < n_attn) {                          // uniform over the workgroup
        xv_attn_tile_body<D, DS>(ta, bid, sm.t);
        return;
    }
    const int i = bid - n_attn;
    xv_gdn_body<DK, false, CPT>(ga, i % gdn_nx, (i / gdn_nx) % ga.Hv, i / (gdn_nx * ga.Hv), sm.g);
}

// The workspace: XV_ATTN_COUNTERS arrival counters of the per-tile split's in-launch combine
// (at a fixed place, so that every call finds them zero whatever the shapes of the calls
// before it), then the chunk partials' acc, then their (m, l).
size_t xv_attn_ws(int B, int T, int Hq, int d, int Lmax, size_t* acc_bytes) {
    const size_t NC = (size_t)((Lmax + XV_ATTN_C - 1) / XV_ATTN_C);
    const size_t pairs = (size_t)B * T * Hq * NC;
    const size_t a = pairs * (size_t)d * sizeof(float);
    if (acc_bytes) *acc_bytes = a;
    return XV_ATTN_COUNTER_BYTES + a + pairs * 2 * sizeof(float);
}

}  // namespace

extern "C" int xv_attn_chunk_tokens(void) { return XV_ATTN_C; }

extern "C" size_t xv_attn_workspace_bytes(int B, int T, int Hq, int d, int Lmax) {
    if (B <= 0 || T <= 0 || Hq <= 0 || d <= 0 || Lmax <= 0) return 0;
    return xv_attn_ws(B, T, Hq, d, Lmax, nullptr);
}

namespace {

// The argument checks of xv_attn_verify_rows; on success the capacity's chunk count, the
// chunks any row can see (the length bound's, when given) and the workspace's two parts.
int xv_attn_check(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                  const uint16_t* k_cache, const uint16_t* v_cache, const int32_t* kv_len,
                  const uint16_t* o, const float* o32, void* workspace, size_t workspace_bytes,
                  int B, int T, int Hq, int Hkv, int d, int Lmax, float scale, int len_bound,
                  int* NC, int* NCg, float** ws_acc, float** ws_ml, int** counters, bool ws_pointer = true)
{
    XV_REQUIRE(B >= 0 && T >= 1 && T <= 16 && Hkv >= 1 && Hq >= 1 && Hq % Hkv == 0, XV_ERR_SHAPE);
    XV_REQUIRE(d == 64 || d == 128 || d == 256, XV_ERR_SHAPE);
    XV_REQUIRE(Lmax >= T && (Lmax + XV_ATTN_C - 1) / XV_ATTN_C <= XV_ATTN_MAX_NC, XV_ERR_SHAPE);
    {   // partial-kernel workgroups (per request, KV head, chunk, 16 pairs, value-dim part) fit the grid
        const long long ntile = ((long long)(Hq / Hkv) * T + 15) / 16;
        const long long items = (long long)B * Hkv * ((Lmax + XV_ATTN_C - 1) / XV_ATTN_C) * ntile * 2;
        XV_REQUIRE(items <= (1LL << 30), XV_ERR_SHAPE);
    }
    XV_REQUIRE(scale == scale, XV_ERR_SHAPE);
    XV_REQUIRE(len_bound == 0 || len_bound >= T, XV_ERR_SHAPE);
    if (B == 0) return XV_OK;
    XV_REQUIRE(q && k_new && v_new && k_cache && v_cache && kv_len && o && (workspace || !ws_pointer), XV_ERR_NULL);
    XV_REQUIRE(xv_aligned16(q) && xv_aligned16(k_new) && xv_aligned16(v_new) &&
               xv_aligned16(k_cache) && xv_aligned16(v_cache) && xv_aligned(kv_len, 4) &&
               xv_aligned(o, 2) && xv_aligned(o32, 4) && xv_aligned16(workspace), XV_ERR_ALIGN);
    size_t acc_bytes = 0;
    const size_t need = xv_attn_ws(B, T, Hq, d, Lmax, &acc_bytes);
    XV_REQUIRE(workspace_bytes >= need, XV_ERR_WORKSPACE);
    *NC = (Lmax + XV_ATTN_C - 1) / XV_ATTN_C;
    const int nb = len_bound > 0 && len_bound < Lmax ? (len_bound + XV_ATTN_C - 1) / XV_ATTN_C : *NC;
    *NCg = nb < *NC ? nb : *NC;
    *counters = reinterpret_cast<int*>(workspace);
    *ws_acc = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + XV_ATTN_COUNTER_BYTES);
    *ws_ml = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + XV_ATTN_COUNTER_BYTES + acc_bytes);
    return XV_OK;
}

template <int D, int DS>
void xv_gdn_attn_fused_ds(const XvGdnArgs& ga, int dk, int cpt, const XvTileArgs& ta, int B, hipStream_t st)
{
    const int gdn_nx = ga.dv / (XV_GDN_JW * cpt);
    const int n_attn = 8 * ta.per_xcd;
    const dim3 grid(n_attn + gdn_nx * ga.Hv * B), block(XV_ATTN_WAVES * 64);
    if (dk == 128 && cpt == 2) hipLaunchKernelGGL((xv_gdn_attn_kernel<128, 2, D, DS>), grid, block, 0, st, ga, ta, n_attn, gdn_nx);
    else if (dk == 128) hipLaunchKernelGGL((xv_gdn_attn_kernel<128, 1, D, DS>), grid, block, 0, st, ga, ta, n_attn, gdn_nx);
    else if (cpt == 2) hipLaunchKernelGGL((xv_gdn_attn_kernel<64, 2, D, DS>), grid, block, 0, st, ga, ta, n_attn, gdn_nx);
    else hipLaunchKernelGGL((xv_gdn_attn_kernel<64, 1, D, DS>), grid, block, 0, st, ga, ta, n_attn, gdn_nx);
}

template <int D>
int xv_gdn_attn_fused(const XvGdnArgs& ga, int dk, int cpt, int ds, const XvTileArgs& ta, int B, hipStream_t st)
{
    (void)hipGetLastError();
    if (D == 256 && ds == 2) xv_gdn_attn_fused_ds<D, (D == 256 ? 2 : 1)>(ga, dk, cpt, ta, B, st);
    else xv_gdn_attn_fused_ds<D, 1>(ga, dk, cpt, ta, B, st);
    return xv_launch_status();
}

}  // namespace

namespace {

int xv_attn_launch_d(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                     uint16_t* k_cache, uint16_t* v_cache, const int32_t* kv_len,
                     uint16_t* o, float* o32, float* ws_acc, float* ws_ml, int* counters,
                     int B, int T, int Hq, int Hkv, int d, int Lmax, int NC, int NCg, float scale, hipStream_t st)
{
    switch (d) {
        case 64:  return xv_attn_launch<64>(q, k_new, v_new, k_cache, v_cache, kv_len, o, o32, ws_acc,
                                            ws_ml, counters, B, T, Hq, Hkv, Lmax, NC, NCg, scale, st);
        case 128: return xv_attn_launch<128>(q, k_new, v_new, k_cache, v_cache, kv_len, o, o32, ws_acc,
                                             ws_ml, counters, B, T, Hq, Hkv, Lmax, NC, NCg, scale, st);
        default:  return xv_attn_launch<256>(q, k_new, v_new, k_cache, v_cache, kv_len, o, o32, ws_acc,
                                             ws_ml, counters, B, T, Hq, Hkv, Lmax, NC, NCg, scale, st);
    }
}

// The chunk partials of xv_attn_verify_rows_noalloc: one file-scope array on every GPU
// the library runs on, held until the process ends.  In host code its name is only a
// stand-in for the symbol; kernels get the device address that hipGetSymbolAddress
// returns, looked up once per device (with that device current) and kept.
constexpr size_t XV_SCRATCH_BYTES = XV_ATTN_NOALLOC_MAX_BYTES;
static_assert(XV_SCRATCH_BYTES % 256 == 0, "whole 256-byte blocks");
static __device__ __align__(256) unsigned char xv_scratch[XV_SCRATCH_BYTES];

constexpr int XV_SCRATCH_MAX_DEVICES = 64;
std::mutex xv_scratch_mu;
void* xv_scratch_dev[XV_SCRATCH_MAX_DEVICES];

// The current device's copy of xv_scratch (its address, never the host-side name).
int xv_scratch_address(void** out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= XV_SCRATCH_MAX_DEVICES) return XV_ERR_LAUNCH;
    std::lock_guard<std::mutex> lock(xv_scratch_mu);
    if (!xv_scratch_dev[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(xv_scratch)) != hipSuccess || !p) return XV_ERR_LAUNCH;
        xv_scratch_dev[dev] = p;
    }
    *out = xv_scratch_dev[dev];
    return XV_OK;
}

}  // namespace

extern "C" int xv_attn_verify_rows(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                                   uint16_t* k_cache, uint16_t* v_cache, const int32_t* kv_len,
                                   uint16_t* o, float* o32, void* workspace, size_t workspace_bytes,
                                   int B, int T, int Hq, int Hkv, int d, int Lmax, float scale,
                                   int len_bound, void* stream)
{
    int NC = 0, NCg = 0;
    float* ws_acc = nullptr;
    float* ws_ml = nullptr;
    int* counters = nullptr;
    const int s = xv_attn_check(q, k_new, v_new, k_cache, v_cache, kv_len, o, o32, workspace, workspace_bytes,
                                B, T, Hq, Hkv, d, Lmax, scale, len_bound, &NC, &NCg, &ws_acc, &ws_ml, &counters);
    if (s != XV_OK || B == 0) return s;
    return xv_attn_launch_d(q, k_new, v_new, k_cache, v_cache, kv_len, o, o32, ws_acc, ws_ml, counters,
                            B, T, Hq, Hkv, d, Lmax, NC, NCg, scale, reinterpret_cast<hipStream_t>(stream));
}

extern "C" int xv_attn_verify_rows_noalloc(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                                           uint16_t* k_cache, uint16_t* v_cache, const int32_t* kv_len,
                                           uint16_t* o, float* o32,
                                           int B, int T, int Hq, int Hkv, int d, int Lmax, float scale,
                                           int len_bound, void* stream)
{
    int NC = 0, NCg = 0;
    float* ws_acc = nullptr;
    float* ws_ml = nullptr;
    int* counters = nullptr;
    // every argument and the size first (no device call), then the buffer's address
    int s = xv_attn_check(q, k_new, v_new, k_cache, v_cache, kv_len, o, o32, nullptr, XV_SCRATCH_BYTES,
                          B, T, Hq, Hkv, d, Lmax, scale, len_bound, &NC, &NCg, &ws_acc, &ws_ml, &counters, false);
    if (s != XV_OK || B == 0) return s;
    void* ws = nullptr;
    s = xv_scratch_address(&ws);
    if (s != XV_OK) return s;
    size_t acc_bytes = 0;
    (void)xv_attn_ws(B, T, Hq, d, Lmax, &acc_bytes);
    counters = reinterpret_cast<int*>(ws);
    ws_acc = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + XV_ATTN_COUNTER_BYTES);
    ws_ml = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + XV_ATTN_COUNTER_BYTES + acc_bytes);
    return xv_attn_launch_d(q, k_new, v_new, k_cache, v_cache, kv_len, o, o32, ws_acc, ws_ml, counters,
                            B, T, Hq, Hkv, d, Lmax, NC, NCg, scale, reinterpret_cast<hipStream_t>(stream));
}

extern "C" int xv_gdn_attn_verify(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                  const float* a, const float* b,
                                  const uint16_t* k_prev, const uint16_t* v_prev,
                                  const float* a_prev, const float* b_prev,
                                  const int32_t* n_keep_prev, int T_prev,
                                  const float* state_in, const float* state_prev_out,
                                  float* state_kept, float* state_out,
                                  uint16_t* o, float* o32, int Hk, int Hv, int dk, int dv,
                                  const uint16_t* q_attn, const uint16_t* k_new, const uint16_t* v_new,
                                  uint16_t* k_cache, uint16_t* v_cache, const int32_t* kv_len,
                                  uint16_t* o_attn, float* o_attn32, void* workspace, size_t workspace_bytes,
                                  int Hq, int Hkv, int d, int Lmax, float scale,
                                  int B, int T, int len_bound, void* stream)
{
    XvGdnArgs ga{};
    int s = n_keep_prev
        ? xv_gdn_args_after(ga, q, k, v, a, b, k_prev, v_prev, a_prev, b_prev, n_keep_prev, T_prev,
                            state_in, state_prev_out, state_kept, state_out, o, o32, B, T, Hk, Hv, dk, dv)
        : xv_gdn_args_verify(ga, q, k, v, a, b, state_in, state_out, o, o32, B, T, Hk, Hv, dk, dv);
    if (s != XV_OK) return s;
    int NC = 0, NCg = 0;
    float* ws_acc = nullptr;
    float* ws_ml = nullptr;
    int* counters = nullptr;
    s = xv_attn_check(q_attn, k_new, v_new, k_cache, v_cache, kv_len, o_attn, o_attn32, workspace,
                      workspace_bytes, B, T, Hq, Hkv, d, Lmax, scale, len_bound, &NC, &NCg, &ws_acc, &ws_ml,
                      &counters);
    if (s != XV_OK || B == 0) return s;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    // one launch when the attention partials take the tile split and both grids are
    // resident at once (about: workgroups of chunks past every row exit at once);
    // the GDN workgroups then take one column group each if that fits, else two
    bool fuse = false;
    int cpt = 1, ds = 1;
    XvTileArgs ta{};
    switch (d) {
        case 64:  fuse = xv_attn_kind<64>(B, T, Hq, Hkv, NCg) == XV_ATTN_TILE; break;
        case 128: fuse = xv_attn_kind<128>(B, T, Hq, Hkv, NCg) == XV_ATTN_TILE; break;
        default:  fuse = xv_attn_kind<256>(B, T, Hq, Hkv, NCg) == XV_ATTN_TILE; break;
    }
    if (fuse) {
        // the GDN workgroups take one column group each if everything fits, else two; the
        // tile grid takes two value-dim parts if that still fits beside them, else one
        const long long cus = xv_cu_count();
        const long long gdn1 = (long long)(dv / XV_GDN_JW) * Hv * B;
        const bool two_col = dv % (2 * XV_GDN_JW) == 0;
        fuse = false;
        for (int dsv = (d == 256 ? 2 : 1); dsv >= 1 && !fuse; --dsv) {
            const long long n_attn = 8 * ((xv_tile_items(B, T, Hq, Hkv, NCg, dsv) + 7) / 8);
            if (n_attn + gdn1 <= XV_FUSE_ONE_COL * cus) { fuse = true; cpt = 1; ds = dsv; }
            else if (two_col && n_attn + gdn1 / 2 <= XV_FUSE_TWO_COL * cus) { fuse = true; cpt = 2; ds = dsv; }
        }
        if (fuse)
            ta = xv_tile_args(ds, q_attn, k_new, v_new, k_cache, v_cache, kv_len, ws_acc, ws_ml, B, T, Hq, Hkv,
                              Lmax, NC, NCg, xv_scale_log2(scale), o_attn, o_attn32, counters);
    }
    if (!fuse) {
        s = n_keep_prev
            ? xv_gdn_verify_after(q, k, v, a, b, k_prev, v_prev, a_prev, b_prev, n_keep_prev, T_prev, state_in,
                                  state_prev_out, state_kept, state_out, o, o32, B, T, Hk, Hv, dk, dv, stream)
            : xv_gdn_verify(q, k, v, a, b, state_in, state_out, o, o32, B, T, Hk, Hv, dk, dv, stream);
        if (s != XV_OK) return s;
        return xv_attn_verify_rows(q_attn, k_new, v_new, k_cache, v_cache, kv_len, o_attn, o_attn32, workspace,
                                   workspace_bytes, B, T, Hq, Hkv, d, Lmax, scale, len_bound, stream);
    }
    switch (d) {
        case 64:  s = xv_gdn_attn_fused<64>(ga, dk, cpt, ds, ta, B, st); break;
        case 128: s = xv_gdn_attn_fused<128>(ga, dk, cpt, ds, ta, B, st); break;
        default:  s = xv_gdn_attn_fused<256>(ga, dk, cpt, ds, ta, B, st); break;
    }
    if (s != XV_OK || ta.counters) return s;    // the attention workgroups combined their rows
    switch (d) {
        case 64:  return xv_attn_combine<64>(ws_acc, ws_ml, kv_len, o_attn, o_attn32, B, T, Hq, Lmax, NC, NCg, false, 0, st);
        case 128: return xv_attn_combine<128>(ws_acc, ws_ml, kv_len, o_attn, o_attn32, B, T, Hq, Lmax, NC, NCg, false, 0, st);
        default:  return xv_attn_combine<256>(ws_acc, ws_ml, kv_len, o_attn, o_attn32, B, T, Hq, Lmax, NC, NCg, false, 0, st);
    }
}

// ---------------------------------------------------------------------------
// Prefill: P rows appended at once, each row with the decode row's arithmetic.
// ---------------------------------------------------------------------------
namespace {


// kv_len[b] += n (one thread per request), after the kernels that read it.
__global__ void xv_kv_advance_kernel(int32_t* __restrict__ kv_len, int B, int n)
{
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b < B) kv_len[b] += n;
}

// Rows r = 0..P-1 of k_new / v_new ([B][P][Hkv][d]) to cache positions L0 + r.
__global__ void xv_kv_append_kernel(const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
                                    uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache,
                                    const int32_t* __restrict__ kv_len, int P, int Hkv, int d, int Lmax)
{
    const int gpr = d / 8;
    const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long long)P * Hkv * gpr) return;
    const int b = blockIdx.y;
    const int c = (int)(idx % gpr);
    const int h = (int)((idx / gpr) % Hkv);
    const int r = (int)(idx / ((long long)gpr * Hkv));
    int L0 = kv_len[b];
    L0 = L0 < 0 ? 0 : (L0 > Lmax - P ? Lmax - P : L0);
    const size_t src = (((size_t)b * P + r) * Hkv + h) * d + c * 8;
    const size_t dst = (((size_t)b * Hkv + h) * Lmax + L0 + r) * d + c * 8;
    xv_store16(k_cache + dst, xv_load16(k_new + src));
    xv_store16(v_cache + dst, xv_load16(v_new + src));
}

// Attention of P appended rows: the rows go into the cache first, then the streaming
// kernel in prefill mode (one workgroup per block of 64 (row, head) pairs; each row gets the
// decode row's chunk partials and two-level fold), then the lengths advance when asked.
template <int D>
int xv_attn_prefill_launch(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                           uint16_t* k_cache, uint16_t* v_cache, int32_t* kv_len,
                           uint16_t* o, float* o32, int B, int P, int Hq, int Hkv, int Lmax, float scale,
                           int advance, hipStream_t st)
{
    (void)hipGetLastError();
    const long long gran = (long long)P * Hkv * (D / 8);
    hipLaunchKernelGGL(xv_kv_append_kernel, dim3((unsigned)((gran + 255) / 256), B), dim3(256), 0, st,
                       k_new, v_new, k_cache, v_cache, kv_len, P, Hkv, D, Lmax);
    int s = xv_launch_status();
    if (s != XV_OK) return s;
    const int NRB = ((Hq / Hkv) * P + XV_ATTN_SPAIRS - 1) / XV_ATTN_SPAIRS;
    const XvStreamArgs sa{q, nullptr, nullptr, k_cache, v_cache, kv_len, nullptr, nullptr, o, o32,
                          P, Hq, Hkv, Lmax, 0, 0, NRB, xv_scale_log2(scale)};
    hipLaunchKernelGGL((xv_attn_stream_kernel<D, true>), dim3(NRB * Hkv * B), dim3(XV_ATTN_WAVES * 64), 0, st, sa);
    s = xv_launch_status();
    if (s != XV_OK || !advance) return s;
    hipLaunchKernelGGL(xv_kv_advance_kernel, dim3((B + 63) / 64), dim3(64), 0, st, kv_len, B, P);
    return xv_launch_status();
}

}  // namespace

extern "C" int xv_attn_prefill(const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                               uint16_t* k_cache, uint16_t* v_cache, int32_t* kv_len,
                               uint16_t* o, float* o32, int B, int P, int Hq, int Hkv, int d, int Lmax,
                               float scale, int advance, void* stream)
{
    XV_REQUIRE(B >= 0 && P >= 1 && Hkv >= 1 && Hq >= 1 && Hq % Hkv == 0, XV_ERR_SHAPE);
    XV_REQUIRE(d == 64 || d == 128 || d == 256, XV_ERR_SHAPE);
    XV_REQUIRE(Lmax >= P && (Lmax + XV_ATTN_C - 1) / XV_ATTN_C <= XV_ATTN_MAX_NC, XV_ERR_SHAPE);
    XV_REQUIRE((long long)((Hq / Hkv) * (long long)P + XV_ATTN_SPAIRS - 1) / XV_ATTN_SPAIRS * Hkv * B < (1LL << 31),
               XV_ERR_SHAPE);
    XV_REQUIRE((long long)P * Hkv * (d / 8) / 256 < (1LL << 31) && B < 65536, XV_ERR_SHAPE);
    XV_REQUIRE(scale == scale, XV_ERR_SHAPE);
    if (B == 0) return XV_OK;
    XV_REQUIRE(q && k_new && v_new && k_cache && v_cache && kv_len && o, XV_ERR_NULL);
    XV_REQUIRE(xv_aligned16(q) && xv_aligned16(k_new) && xv_aligned16(v_new) && xv_aligned16(k_cache) &&
               xv_aligned16(v_cache) && xv_aligned(kv_len, 4) && xv_aligned(o, 2) && xv_aligned(o32, 4),
               XV_ERR_ALIGN);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    switch (d) {
        case 64:  return xv_attn_prefill_launch<64>(q, k_new, v_new, k_cache, v_cache, kv_len, o, o32, B, P, Hq,
                                                    Hkv, Lmax, scale, advance, st);
        case 128: return xv_attn_prefill_launch<128>(q, k_new, v_new, k_cache, v_cache, kv_len, o, o32, B, P, Hq,
                                                     Hkv, Lmax, scale, advance, st);
        default:  return xv_attn_prefill_launch<256>(q, k_new, v_new, k_cache, v_cache, kv_len, o, o32, B, P, Hq,
                                                     Hkv, Lmax, scale, advance, st);
    }
}
