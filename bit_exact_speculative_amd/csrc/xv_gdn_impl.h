// xv_gdn_impl.h -- the GDN verify / rollback device code (the per-token rule, its
// fixed-order dot, and the workgroup body), shared by the GDN launches and by
// the launch that runs GDN and attention side by side.  The description of the
// arithmetic and the work mapping is at the top of xv_gdn.hip.
#pragma once

#include "xv_common.h"

namespace {


constexpr int XV_GDN_JW = 32;       // value indices per column group (8 waves x 4)
constexpr int XV_GDN_LPJ = 16;      // lanes per value index
constexpr int XV_GDN_THREADS = XV_GDN_JW * XV_GDN_LPJ;
constexpr int XV_GDN_TMAX = 16;
constexpr int XV_GDN_TM = 2 * XV_GDN_TMAX;     // rows one launch stages: replayed + this call's

// Exact lane moves within each row of 16 lanes (DPP): swap with lane^1, lane^2,
// mirror each half-row (lane i <-> 7 - i), mirror the row (lane i <-> 15 - i).
__device__ __forceinline__ float xv_dpp_xor1(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float xv_dpp_xor2(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ float xv_dpp_mirror8(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
}
__device__ __forceinline__ float xv_dpp_mirror16(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
}

// The one dot product of the rule, sum_i s_i x_i over the dk key indices of a state
// column.  The dk indices form 16 partials of P = dk / 16 consecutive indices; a partial
// is two fp32 chains, over its even and its odd indices in ascending order, then their
// sum; the 16 partials meet in a balanced tree, ((p0 + p1) + (p2 + p3)) + ..., level by
// level.  A kernel may spread a column over L = 1, 2, 4, 8 or 16 lanes: lane ig of the L
// holds the R = dk / L indices [ig R, ig R + R), forms its 16 / L partials and the tree's
// first levels over them in registers, and the last log2 L levels run across the lanes
// (DPP within each row of 16 lanes: lane^1, lane^2, the mirrored half of each 8, the
// mirrored half of the 16).  Each tree node adds the same two values in every
// arrangement (fp32 addition is commutative), so the result has the same bits for every
// L, and every lane of a column ends with them.
template <int P>
__device__ __forceinline__ float xv_gdn_partial(const float* s, const float* x) {
    static_assert(P % 2 == 0, "two chains");
    float c0 = s[0] * x[0];
    float c1 = s[1] * x[1];
#pragma unroll
    for (int r = 2; r < P; r += 2) {
        c0 = __builtin_fmaf(s[r], x[r], c0);
        c1 = __builtin_fmaf(s[r + 1], x[r + 1], c1);
    }
    return c0 + c1;
}

template <int L, int R>
__device__ __forceinline__ float xv_gdn_dot(const float (&s)[R], const float (&x)[R]) {
    static_assert(L == 1 || L == 2 || L == 4 || L == 8 || L == 16, "L divides 16");
    constexpr int PL = 16 / L;                       // partials per lane
    constexpr int P = R / PL;                        // indices per partial
    float p[PL];
#pragma unroll
    for (int g = 0; g < PL; ++g) p[g] = xv_gdn_partial<P>(s + g * P, x + g * P);
#pragma unroll
    for (int w = 1; w < PL; w *= 2)                  // in-lane tree levels
#pragma unroll
        for (int g = 0; g < PL; g += 2 * w) p[g] = p[g] + p[g + w];
    float t = p[0];
    if constexpr (L >= 2) t = t + xv_dpp_xor1(t);
    if constexpr (L >= 4) t = t + xv_dpp_xor2(t);
    if constexpr (L >= 8) t = t + xv_dpp_mirror8(t);
    if constexpr (L >= 16) t = t + xv_dpp_mirror16(t);
    return t;
}

// The one per-token state update (decode, verify and rollback all call this).
template <int L, int R>
__device__ __forceinline__ void xv_gdn_token(float (&s)[R], const float (&kk)[R],
                                             float vj, float at, float bt) {
#pragma unroll
    for (int r = 0; r < R; ++r) s[r] = at * s[r];
    const float kv = xv_gdn_dot<L, R>(s, kk);
    const float u = bt * (vj - kv);
#pragma unroll
    for (int r = 0; r < R; ++r) s[r] = __builtin_fmaf(u, kk[r], s[r]);
}

// What one launch runs, per request b: first n_pre = clamp(n_pre[b], 0, Tp) rows
// of a previous call (its k, v, a, b; no outputs), then the T rows of this call
// (q, k, v, a, b; outputs o), all with xv_gdn_token, from the state S_in; when
// S_alt is given and n_pre == Tp, from S_alt with no replay instead.  The state
// after the replayed rows goes to S_mid (when given), the final state to S_out.
//   verify          : no previous rows (n_pre NULL), T rows
//   rollback        : previous rows = the verify's, n_pre = n_keep, T = 0; n == Tp
//                     leaves S_out as it is (it holds S_T); kv_len[b] += n
//   verify after    : the previous call's kept rows replayed (or its S_T taken),
//                     then T rows; S_mid receives the kept state of the previous call
struct XvGdnArgs {
    const uint16_t* kp; const uint16_t* vp; const float* ap; const float* bp;   // previous rows
    const int32_t* n_pre;                   // [B] previous rows to replay, or NULL
    int Tp;                                 // rows per request of the previous call
    const float* S_alt;                     // S_T of the previous call, or NULL
    const uint16_t* q; const uint16_t* k; const uint16_t* v; const float* a; const float* b;
    int T;                                  // rows of this call (0: rollback)
    const float* S_in; float* S_mid; float* S_out;
    uint16_t* o; float* o32;
    int32_t* kv_len;                        // rollback: += n
    int Hk, Hv, dv;
};

// LDS of one workgroup that owns 32 * CPT value indices.
template <int DK, int CPT>
struct XvGdnSmem {
    static constexpr int W = XV_GDN_JW * CPT;
    static constexpr int SP = W + 1;                 // state slab row pitch (floats)
    float skq[XV_GDN_TM][2][DK];                     // k, q rows, fp32
    uint16_t sv[XV_GDN_TM][W];
    float sab[XV_GDN_TM][2];
    float sst[DK * SP];                              // the state slab [i][W values]
};

// Stage the rows of tokens 0..n-1 of a launch (the np replayed rows of the previous call
// first, then this call's) for the W value indices [j0, j0 + W) of value head h of request
// b into LDS: k and q widened to fp32, v as bf16, a and b.  Every load is issued before any
// LDS store (straight-line, clamped to token 0), so the staging costs one round trip.
template <int DK, int W, int NT>
__device__ __forceinline__ void xv_gdn_stage(const XvGdnArgs A, int b, int h, int g, int j0, int np, int n,
                                             float (*skq)[2][DK], uint16_t (*sv)[W], float (*sab)[2])
{
    if (n <= 0) return;                      // uniform
    const int tid = threadIdx.x;
    const int Hk = A.Hk, Hv = A.Hv, dv = A.dv, T = A.T, Tp = A.Tp;
    constexpr int TM = XV_GDN_TM;
    constexpr int CH = DK / 8;               // 16-byte chunks per k or q row
    constexpr int KQ_PER = (TM * 2 * CH + NT - 1) / NT;
    constexpr int V_PER = (TM * W + NT - 1) / NT;
    // row t of the launch: replayed row t of the previous call, or row t - np of this one
    auto kq_src = [&](int t, int which) -> const uint16_t* {
        if (t < np) return A.kp + (((size_t)b * Tp + t) * Hk + g) * DK;
        const size_t row = ((size_t)b * T + (t - np)) * Hk + g;
        return (which == 0 ? A.k : A.q) + row * DK;
    };
    xv_u32x4 kq[KQ_PER];
    uint16_t vv[V_PER];
    float abv = 0.f;
#pragma unroll
    for (int e = 0; e < KQ_PER; ++e) {
        int idx = tid + e * NT;
        idx = idx < n * 2 * CH ? idx : 0;
        const int t = idx / (2 * CH), rem = idx % (2 * CH);
        const int which = rem / CH, c = rem % CH;   // 0: k, 1: q (a replayed row: k again)
        kq[e] = xv_load16(kq_src(t, which) + c * 8);
    }
#pragma unroll
    for (int e = 0; e < V_PER; ++e) {
        int idx = tid + e * NT;
        idx = idx < n * W ? idx : 0;
        const int t = idx / W, c = idx % W;
        const int jj = j0 + c;
        vv[e] = t < np ? A.vp[(((size_t)b * Tp + t) * Hv + h) * dv + jj]
                       : A.v[(((size_t)b * T + (t - np)) * Hv + h) * dv + jj];
    }
    {
        const int idx = tid < 2 * n ? tid : 0;
        const int t = idx >> 1;
        abv = t < np ? ((idx & 1) ? A.bp : A.ap)[((size_t)b * Tp + t) * Hv + h]
                     : ((idx & 1) ? A.b : A.a)[((size_t)b * T + (t - np)) * Hv + h];
    }
#pragma unroll
    for (int e = 0; e < KQ_PER; ++e) {
        const int idx = tid + e * NT;
        if (idx < n * 2 * CH) {
            const int t = idx / (2 * CH), rem = idx % (2 * CH);
            float* dst = &skq[t][rem / CH][(rem % CH) * 8];
            xv_f32x4 lo4, hi4;
#pragma unroll
            for (int w2 = 0; w2 < 2; ++w2) {
                lo4[2 * w2] = xv_bf16_lo(kq[e][w2]);
                lo4[2 * w2 + 1] = xv_bf16_hi(kq[e][w2]);
                hi4[2 * w2] = xv_bf16_lo(kq[e][2 + w2]);
                hi4[2 * w2 + 1] = xv_bf16_hi(kq[e][2 + w2]);
            }
            *reinterpret_cast<xv_f32x4*>(dst) = lo4;
            *reinterpret_cast<xv_f32x4*>(dst + 4) = hi4;
        }
    }
#pragma unroll
    for (int e = 0; e < V_PER; ++e) {
        const int idx = tid + e * NT;
        if (idx < n * W) sv[idx / W][idx % W] = vv[e];
    }
    if (tid < 2 * n) sab[tid >> 1][tid & 1] = abv;
}

// The workgroup (bx, h, b): value indices [bx W, bx W + W) of value head h of
// request b, W = 32 CPT.  Thread (wave, lane) holds key indices ig R .. ig R + R - 1
// (ig = lane % 16) of the CPT columns jw + 32 c, jw = 4 wave + lane / 16: each
// column is updated exactly as with one column per thread, the CPT columns only
// interleave their instructions.
template <int DK, bool ROLLBACK, int CPT>
__device__ __forceinline__ void xv_gdn_body(const XvGdnArgs A, int bx, int h, int b, XvGdnSmem<DK, CPT>& sm)
{
    constexpr int NT = XV_GDN_THREADS;
    constexpr int R = DK / XV_GDN_LPJ;
    constexpr int W = XV_GDN_JW * CPT;
    constexpr int SP = W + 1;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int ig = lane & 15;                // key-index group: i in [ig*R, ig*R + R)
    const int jl = lane >> 4;
    const int jw = wave * 4 + jl;            // first value index within the workgroup's slice
    const int j0 = bx * W;
    const int Hk = A.Hk, Hv = A.Hv, dv = A.dv, T = A.T, Tp = A.Tp;
    const int g = h / (Hv / Hk);

    // the state slab S[i][j0 .. j0 + W) moves through LDS so that global reads and
    // writes are 16-byte, W / 4 threads per row
    constexpr int GPR = W / 4;               // 16-byte granules per slab row
    constexpr int SROWS = NT / GPR;          // slab rows per pass
    constexpr int SPASS = DK / SROWS;
    static_assert(DK % SROWS == 0, "the slab must split into whole passes");
    const size_t slab = (size_t)(b * Hv + h) * DK * dv + j0 + (tid % GPR) * 4;
    xv_f32x4 sl[SPASS];
    auto load_slab = [&](const float* S0) {
#pragma unroll
        for (int e = 0; e < SPASS; ++e)
            sl[e] = __builtin_nontemporal_load(reinterpret_cast<const xv_f32x4*>(S0 + slab + (size_t)(tid / GPR + e * SROWS) * dv));
    };
    // the slab's loads from S_in go out before n_pre is known: S_in is the start state unless
    // every previous row was kept, when the slab is read again from S_alt
    load_slab(A.S_in);

    int np = 0;
    if (A.n_pre) {
        np = A.n_pre[b];
        np = np < 0 ? 0 : (np > Tp ? Tp : np);
        if (ROLLBACK) {
            if (bx == 0 && h == 0 && tid == 0) A.kv_len[b] += np;
            if (np == Tp) return;            // state_out already holds S_T
        } else if (np == Tp && A.S_alt) {
            load_slab(A.S_alt);              // every previous row kept: its S_T, nothing to replay
            np = 0;
        }
    }
    const int nm = ROLLBACK ? 0 : T;         // rows of this call
    const int n = np + nm;

    xv_gdn_stage<DK, W, NT>(A, b, h, g, j0, np, n, sm.skq, sm.sv, sm.sab);
#pragma unroll
    for (int e = 0; e < SPASS; ++e)
#pragma unroll
        for (int c = 0; c < 4; ++c) sm.sst[(tid / GPR + e * SROWS) * SP + (tid % GPR) * 4 + c] = sl[e][c];
    __syncthreads();
    float s[CPT][R];                         // this lane's part of its columns, for the whole call
#pragma unroll
    for (int c = 0; c < CPT; ++c)
#pragma unroll
        for (int r = 0; r < R; ++r) s[c][r] = sm.sst[(ig * R + r) * SP + jw + XV_GDN_JW * c];

    // the slab of a state: own slots to LDS, then 16-byte rows out.  The stores are
    // non-temporal: no one reads a state in the same step, and dirty state lines left in
    // the caches would be written back while the next kernel (the weight stream of the
    // projections) competes for HBM; streamed out, they drain during this kernel.
    auto store_state = [&](float* __restrict__ dst) {
        __syncthreads();                     // every lane is done reading the slab
#pragma unroll
        for (int c = 0; c < CPT; ++c)
#pragma unroll
            for (int r = 0; r < R; ++r) sm.sst[(ig * R + r) * SP + jw + XV_GDN_JW * c] = s[c][r];
        __syncthreads();
#pragma unroll
        for (int e = 0; e < SPASS; ++e) {
            xv_f32x4 out;
#pragma unroll
            for (int c = 0; c < 4; ++c) out[c] = sm.sst[(tid / GPR + e * SROWS) * SP + (tid % GPR) * 4 + c];
            __builtin_nontemporal_store(out, reinterpret_cast<xv_f32x4*>(dst + slab + (size_t)(tid / GPR + e * SROWS) * dv));
        }
    };

    // Two register sets used alternately: token t's rows are in one while token t+1's are
    // read from LDS into the other (no copies between them).
    float k0[R], q0[R], k1[R], q1[R];
    float v0[CPT], v1[CPT];
    float a0 = 0.f, b0 = 0.f, a1 = 0.f, b1 = 0.f;
    auto fetch = [&](int t, float (&kk)[R], float (&qq)[R], float (&vv2)[CPT], float& aa, float& bb) {
#pragma unroll
        for (int c = 0; c < R / 4; ++c) {
            const xv_f32x4 k4 = *reinterpret_cast<const xv_f32x4*>(&sm.skq[t][0][ig * R + c * 4]);
#pragma unroll
            for (int e = 0; e < 4; ++e) kk[c * 4 + e] = k4[e];
            if (!ROLLBACK) {
                const xv_f32x4 q4 = *reinterpret_cast<const xv_f32x4*>(&sm.skq[t][1][ig * R + c * 4]);
#pragma unroll
                for (int e = 0; e < 4; ++e) qq[c * 4 + e] = q4[e];
            }
        }
#pragma unroll
        for (int c = 0; c < CPT; ++c) vv2[c] = xv_bf16_to_f32(sm.sv[t][jw + XV_GDN_JW * c]);
        aa = sm.sab[t][0];
        bb = sm.sab[t][1];
    };
    auto step = [&](int t, const float (&kk)[R], const float (&qq)[R], const float (&vv2)[CPT], float aa, float bb) {
        if (!ROLLBACK && A.S_mid && t == np) store_state(A.S_mid);   // uniform: the kept state
#pragma unroll
        for (int c = 0; c < CPT; ++c) xv_gdn_token<XV_GDN_LPJ, R>(s[c], kk, vv2[c], aa, bb);
        if (!ROLLBACK && t >= np) {
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
                const float ot = xv_gdn_dot<XV_GDN_LPJ, R>(s[c], qq);
                if (ig == 0) {
                    const size_t oi = (((size_t)b * T + (t - np)) * Hv + h) * dv + j0 + jw + XV_GDN_JW * c;
                    A.o[oi] = xv_f32_to_bf16(ot);
                    if (A.o32) A.o32[oi] = ot;
                }
            }
        }
    };
    // The next row's LDS reads are issued on every path (row n - 1 again past the end, never
    // used), so the wait before a token's update covers only the reads of that token's rows.
    if (n > 0) fetch(0, k0, q0, v0, a0, b0);
    for (int t = 0; t < n; t += 2) {            // uniform
        fetch(t + 1 < n ? t + 1 : n - 1, k1, q1, v1, a1, b1);
        step(t, k0, q0, v0, a0, b0);
        if (t + 1 < n) {
            fetch(t + 2 < n ? t + 2 : n - 1, k0, q0, v0, a0, b0);
            step(t + 1, k1, q1, v1, a1, b1);
        }
    }
    if (!ROLLBACK && A.S_mid && n == np) store_state(A.S_mid);      // no rows of this call
    store_state(A.S_out);
}


int xv_gdn_check(const void* k, const void* v, const void* a, const void* b,
                 const void* sin, const void* sout, int B, int T, int Hk, int Hv, int dk, int dv,
                 int tmax = XV_GDN_TMAX)
{
    XV_REQUIRE(B >= 0 && T >= 1 && T <= tmax && Hk >= 1 && Hv >= 1 && Hv % Hk == 0, XV_ERR_SHAPE);
    XV_REQUIRE(dk == 64 || dk == 128, XV_ERR_SHAPE);
    XV_REQUIRE(dv >= 32 && dv <= 128 && dv % 32 == 0, XV_ERR_SHAPE);
    if (B == 0) return XV_OK;
    XV_REQUIRE(k && v && a && b && sin && sout, XV_ERR_NULL);
    XV_REQUIRE(xv_aligned16(k) && xv_aligned(v, 2) && xv_aligned(a, 4) && xv_aligned(b, 4) &&
               xv_aligned16(sin) && xv_aligned16(sout), XV_ERR_ALIGN);
    XV_REQUIRE(sin != sout, XV_ERR_ALIAS);
    return XV_OK;
}


// Prefill: the T rows of a long prompt (any T) through the same per-token routine, state
// in registers for the whole call.  Rows move through LDS in blocks of 16: the next
// block's loads are issued before the current block is computed, and stored to the other
// LDS buffer after it.  Outputs for every row; S_in -> S_out.
constexpr int XV_GDN_PB = 16;

template <int DK>
struct XvGdnPrefillSmem {
    static constexpr int SP = XV_GDN_JW + 1;
    float skq[2][XV_GDN_PB][2][DK];
    uint16_t sv[2][XV_GDN_PB][XV_GDN_JW];
    float sab[2][XV_GDN_PB][2];
    float sst[DK * SP];
};

template <int DK>
__device__ __forceinline__ void xv_gdn_prefill_body(const XvGdnArgs A, int bx, int h, int b,
                                                    XvGdnPrefillSmem<DK>& sm)
{
    constexpr int NT = XV_GDN_THREADS;
    constexpr int R = DK / XV_GDN_LPJ;
    constexpr int W = XV_GDN_JW;
    constexpr int SP = W + 1;
    constexpr int PB = XV_GDN_PB;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int ig = lane & 15;
    const int jw = wave * 4 + (lane >> 4);
    const int j0 = bx * W;
    const int Hk = A.Hk, Hv = A.Hv, dv = A.dv, T = A.T;
    const int g = h / (Hv / Hk);

    constexpr int GPR = W / 4;
    constexpr int SROWS = NT / GPR;
    constexpr int SPASS = DK / SROWS;
    const size_t slab = (size_t)(b * Hv + h) * DK * dv + j0 + (tid % GPR) * 4;
    xv_f32x4 sl[SPASS];
#pragma unroll
    for (int e = 0; e < SPASS; ++e)
        sl[e] = __builtin_nontemporal_load(reinterpret_cast<const xv_f32x4*>(A.S_in + slab + (size_t)(tid / GPR + e * SROWS) * dv));

    // one block's rows: every load issued first (clamped to the call's first row), stored later
    constexpr int CH = DK / 8;
    constexpr int KQ_PER = (PB * 2 * CH + NT - 1) / NT;
    constexpr int V_PER = (PB * W + NT - 1) / NT;
    xv_u32x4 kq[KQ_PER];
    uint16_t vv[V_PER];
    float abv = 0.f;
    auto fetch_block = [&](int t0, int n) {
#pragma unroll
        for (int e = 0; e < KQ_PER; ++e) {
            int idx = tid + e * NT;
            idx = idx < n * 2 * CH ? idx : 0;
            const int t = t0 + idx / (2 * CH), rem = idx % (2 * CH);
            const size_t row = ((size_t)b * T + t) * Hk + g;
            kq[e] = xv_load16((rem / CH == 0 ? A.k : A.q) + row * DK + (rem % CH) * 8);
        }
#pragma unroll
        for (int e = 0; e < V_PER; ++e) {
            int idx = tid + e * NT;
            idx = idx < n * W ? idx : 0;
            vv[e] = A.v[(((size_t)b * T + t0 + idx / W) * Hv + h) * dv + j0 + idx % W];
        }
        const int idx = tid < 2 * n ? tid : 0;
        abv = ((idx & 1) ? A.b : A.a)[((size_t)b * T + t0 + (idx >> 1)) * Hv + h];
    };
    auto stage_block = [&](int buf, int n) {
#pragma unroll
        for (int e = 0; e < KQ_PER; ++e) {
            const int idx = tid + e * NT;
            if (idx < n * 2 * CH) {
                const int t = idx / (2 * CH), rem = idx % (2 * CH);
                float* dst = &sm.skq[buf][t][rem / CH][(rem % CH) * 8];
                xv_f32x4 lo4, hi4;
#pragma unroll
                for (int w2 = 0; w2 < 2; ++w2) {
                    lo4[2 * w2] = xv_bf16_lo(kq[e][w2]);
                    lo4[2 * w2 + 1] = xv_bf16_hi(kq[e][w2]);
                    hi4[2 * w2] = xv_bf16_lo(kq[e][2 + w2]);
                    hi4[2 * w2 + 1] = xv_bf16_hi(kq[e][2 + w2]);
                }
                *reinterpret_cast<xv_f32x4*>(dst) = lo4;
                *reinterpret_cast<xv_f32x4*>(dst + 4) = hi4;
            }
        }
#pragma unroll
        for (int e = 0; e < V_PER; ++e) {
            const int idx = tid + e * NT;
            if (idx < n * W) sm.sv[buf][idx / W][idx % W] = vv[e];
        }
        if (tid < 2 * n) sm.sab[buf][tid >> 1][tid & 1] = abv;
    };

    const int nb = (T + PB - 1) / PB;
    fetch_block(0, T < PB ? T : PB);
#pragma unroll
    for (int e = 0; e < SPASS; ++e)
#pragma unroll
        for (int c = 0; c < 4; ++c) sm.sst[(tid / GPR + e * SROWS) * SP + (tid % GPR) * 4 + c] = sl[e][c];
    stage_block(0, T < PB ? T : PB);
    __syncthreads();
    float s[R];
#pragma unroll
    for (int r = 0; r < R; ++r) s[r] = sm.sst[(ig * R + r) * SP + jw];

    // two register sets, used alternately: token t's rows are in one while token t+1's are
    // read from LDS into the other (no copies between them)
    float k0[R], q0[R], k1[R], q1[R];
    float v0 = 0.f, a0 = 0.f, b0 = 0.f, v1 = 0.f, a1 = 0.f, b1 = 0.f;
    for (int blk = 0; blk < nb; ++blk) {
        const int buf = blk & 1;
        const int t0 = blk * PB;
        const int n = T - t0 < PB ? T - t0 : PB;
        const int t1 = t0 + PB;
        const int n1 = T - t1 < PB ? T - t1 : PB;
        if (blk + 1 < nb) fetch_block(t1, n1);   // uniform: the next block's loads in flight
        auto fetch = [&](int t, float (&kk)[R], float (&qq)[R], float& vv2, float& aa, float& bb) {
#pragma unroll
            for (int c = 0; c < R / 4; ++c) {
                const xv_f32x4 k4 = *reinterpret_cast<const xv_f32x4*>(&sm.skq[buf][t][0][ig * R + c * 4]);
                const xv_f32x4 q4 = *reinterpret_cast<const xv_f32x4*>(&sm.skq[buf][t][1][ig * R + c * 4]);
#pragma unroll
                for (int e = 0; e < 4; ++e) { kk[c * 4 + e] = k4[e]; qq[c * 4 + e] = q4[e]; }
            }
            vv2 = xv_bf16_to_f32(sm.sv[buf][t][jw]);
            aa = sm.sab[buf][t][0];
            bb = sm.sab[buf][t][1];
        };
        auto out = [&](int t, const float (&qq)[R]) {
            const float ot = xv_gdn_dot<XV_GDN_LPJ, R>(s, qq);
            if (ig == 0) {
                const size_t oi = (((size_t)b * T + t0 + t) * Hv + h) * dv + j0 + jw;
                A.o[oi] = xv_f32_to_bf16(ot);
                if (A.o32) A.o32[oi] = ot;
            }
        };
        fetch(0, k0, q0, v0, a0, b0);
        for (int t = 0; t < n; t += 2) {        // uniform; reads on every path, as in verify
            fetch(t + 1 < n ? t + 1 : n - 1, k1, q1, v1, a1, b1);
            xv_gdn_token<XV_GDN_LPJ, R>(s, k0, v0, a0, b0);
            out(t, q0);
            if (t + 1 < n) {
                fetch(t + 2 < n ? t + 2 : n - 1, k0, q0, v0, a0, b0);
                xv_gdn_token<XV_GDN_LPJ, R>(s, k1, v1, a1, b1);
                out(t + 1, q1);
            }
        }
        if (blk + 1 < nb) stage_block(buf ^ 1, n1);   // the other buffer: last read a block ago
        __syncthreads();
    }
    // the slab out
#pragma unroll
    for (int r = 0; r < R; ++r) sm.sst[(ig * R + r) * SP + jw] = s[r];
    __syncthreads();
#pragma unroll
    for (int e = 0; e < SPASS; ++e) {
        xv_f32x4 out;
#pragma unroll
        for (int c = 0; c < 4; ++c) out[c] = sm.sst[(tid / GPR + e * SROWS) * SP + (tid % GPR) * 4 + c];
        *reinterpret_cast<xv_f32x4*>(A.S_out + slab + (size_t)(tid / GPR + e * SROWS) * dv) = out;
    }
}

// The argument checks of xv_gdn_verify and the launch arguments (B == 0: checked, nothing to run).
inline int xv_gdn_args_verify(XvGdnArgs& args, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const float* a, const float* b, const float* state_in, float* state_out,
                              uint16_t* o, float* o32, int B, int T, int Hk, int Hv, int dk, int dv)
{
    int s = xv_gdn_check(k, v, a, b, state_in, state_out, B, T, Hk, Hv, dk, dv);
    if (s != XV_OK || B == 0) return s;
    XV_REQUIRE(q && o, XV_ERR_NULL);
    XV_REQUIRE(xv_aligned16(q) && xv_aligned(o, 2) && xv_aligned(o32, 4), XV_ERR_ALIGN);
    args = XvGdnArgs{};
    args.q = q; args.k = k; args.v = v; args.a = a; args.b = b; args.T = T;
    args.S_in = state_in; args.S_out = state_out; args.o = o; args.o32 = o32;
    args.Hk = Hk; args.Hv = Hv; args.dv = dv;
    return XV_OK;
}

// The argument checks of xv_gdn_verify_after and the launch arguments.
inline int xv_gdn_args_after(XvGdnArgs& args, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             const float* a, const float* b,
                             const uint16_t* k_prev, const uint16_t* v_prev, const float* a_prev,
                             const float* b_prev, const int32_t* n_keep_prev, int T_prev,
                             const float* state_prev_in, const float* state_prev_out,
                             float* state_kept, float* state_out, uint16_t* o, float* o32,
                             int B, int T, int Hk, int Hv, int dk, int dv)
{
    int s = xv_gdn_check(k, v, a, b, state_prev_in, state_out, B, T, Hk, Hv, dk, dv);
    if (s != XV_OK) return s;
    XV_REQUIRE(T_prev >= 1 && T_prev <= XV_GDN_TMAX, XV_ERR_SHAPE);
    if (B == 0) return XV_OK;
    XV_REQUIRE(q && o && k_prev && v_prev && a_prev && b_prev && n_keep_prev && state_prev_out && state_kept,
               XV_ERR_NULL);
    XV_REQUIRE(xv_aligned16(q) && xv_aligned(o, 2) && xv_aligned(o32, 4) && xv_aligned16(k_prev) &&
               xv_aligned(v_prev, 2) && xv_aligned(a_prev, 4) && xv_aligned(b_prev, 4) &&
               xv_aligned(n_keep_prev, 4) && xv_aligned16(state_prev_out) && xv_aligned16(state_kept),
               XV_ERR_ALIGN);
    XV_REQUIRE(state_out != state_prev_out && state_kept != state_prev_in && state_kept != state_prev_out &&
               state_kept != state_out, XV_ERR_ALIAS);
    args = XvGdnArgs{};
    args.kp = k_prev; args.vp = v_prev; args.ap = a_prev; args.bp = b_prev;
    args.n_pre = n_keep_prev; args.Tp = T_prev; args.S_alt = state_prev_out;
    args.q = q; args.k = k; args.v = v; args.a = a; args.b = b; args.T = T;
    args.S_in = state_prev_in; args.S_mid = state_kept; args.S_out = state_out;
    args.o = o; args.o32 = o32;
    args.Hk = Hk; args.Hv = Hv; args.dv = dv;
    return XV_OK;
}

}  // namespace
