// xv_gdn.hip -- gated-delta-net verify and rollback on an fp32 state.
//
// The post's first verify change: verify must run the GDN recurrence with the
// decode arithmetic, because the old verify kernel tiled the state in another
// order and used a different beta precision.  Here there is exactly one
// per-token routine, xv_gdn_token(), used by decode (T = 1), verify (any T) and
// the rollback recompute; its dk-reduction order is fixed at compile time and
// depends on nothing but dk.
//
// Per value head h, value index j, the column S[j][0..dk) evolves on its own:
//     s_i <- a s_i                         (decay, one fp32 multiply each)
//     kv   = sum_i s_i k_i                 (fixed-order dot, below)
//     u    = b (v_j - kv)
//     s_i <- fma(u, k_i, s_i)
//     o_j  = sum_i s_i q_i                 (same fixed-order dot)
// which is S_t = a S_{t-1} (I - b k k^T) + b v k^T, o = S_t q.
//
// The fixed dot order (xv_gdn_dot): the dk key indices form 16 partials of dk/16
// consecutive indices, each two fp32 chains (even and odd indices, ascending) then
// their sum; the partials meet in a balanced tree ((p0 + p1) + (p2 + p3)) + ...
// A kernel may spread a column over L lanes (L dividing 16): each lane forms its
// 16/L partials and the first tree levels in registers, the last log2 L levels run
// across the lanes by DPP.  Every tree node adds the same two values whatever L is
// (fp32 addition is commutative), so the bits do not depend on L, and every lane of
// a column ends with them: all lanes of a column compute the same u.
//
// Two work mappings (gfx950, wave64), the same arithmetic:
//  - 16 lanes per column (few requests: the shortest per-token dependency chain,
//    and a batch-1 call still gives every SIMD more than one wave to interleave):
//    a workgroup of 8 waves owns 32 value indices of one (request, value head) (64,
//    two columns per lane, when it shares a launch with attention and the chip is
//    short of CUs for one column); each lane holds dk/16 consecutive key indices of
//    its column in VGPRs for the whole call; the state slab moves through LDS so
//    that its global reads and writes are 16-byte.
//  - 4 lanes per column (many requests: a quarter of the cross-lane steps and of the
//    per-lane overhead per column, so the VALU issues about 40% fewer instructions per
//    state element): a workgroup of 4 waves owns 64 value indices, a lane dk/4 key
//    indices of one column, read and written straight from global memory (each
//    instruction moves four 64-byte runs of a state row).
// The state is read once and written once per call; the rows of all tokens are
// staged in LDS (k and q already widened to fp32) before the token loop starts.
#include "xv_gdn_impl.h"

namespace {

// Six waves per SIMD (at most 80 VGPRs; two 8-byte addresses go to scratch outside the token
// loop): three workgroups share a CU, which their LDS (51 KB each at dk = 128) also allows,
// so a batch of 8 (1536 workgroups) runs in two rounds instead of three.
template <int DK, bool ROLLBACK, int CPT>
__global__ __launch_bounds__(XV_GDN_THREADS, 6)
void xv_gdn_kernel(XvGdnArgs A)
{
    __shared__ __attribute__((aligned(16))) XvGdnSmem<DK, CPT> sm;
    xv_gdn_body<DK, ROLLBACK, CPT>(A, blockIdx.x, blockIdx.y, blockIdx.z, sm);
}

template <int DK>
__global__ __launch_bounds__(XV_GDN_THREADS)
void xv_gdn_prefill_kernel(XvGdnArgs A)
{
    __shared__ __attribute__((aligned(16))) XvGdnPrefillSmem<DK> sm;
    xv_gdn_prefill_body<DK>(A, blockIdx.x, blockIdx.y, blockIdx.z, sm);
}

// 4 lanes per column: a workgroup of 4 waves owns 64 value indices of one (request,
// value head); lane (jc, ig) = 4 jc + ig of wave w holds key indices ig R .. ig R + R - 1
// of value index 16 w + jc, R = dk / 4.  Three workgroups share a CU (at most 168 VGPRs).
constexpr int XV_GDN4_WAVES = 4;
constexpr int XV_GDN4_W = XV_GDN4_WAVES * 16;

constexpr int XV_GDN4_SP = XV_GDN4_W;       // row pitch (floats) of the outgoing half slab (unpadded: three
                                            // workgroups per CU must still fit their LDS)
static_assert(XV_GDN4_W == 64 && XV_GDN4_WAVES * 64 == 256, "the slab store: 16 threads per 64-float row");

template <int DK>
struct XvGdn4Smem {
    float skq[XV_GDN_TM][2][DK];
    uint16_t sv[XV_GDN_TM][XV_GDN4_W];
    float sab[XV_GDN_TM][2];
    float sst[DK / 2][XV_GDN4_SP];           // half of the state slab on its way out
};

template <int DK, int DV, bool ROLLBACK>
__global__ __launch_bounds__(XV_GDN4_WAVES * 64, 3)
void xv_gdn4_kernel(XvGdnArgs A)
{
    constexpr int L = 4;
    constexpr int R = DK / L;
    constexpr int W = XV_GDN4_W;
    __shared__ __attribute__((aligned(16))) XvGdn4Smem<DK> sm;
    const int bx = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int ig = lane & (L - 1);
    const int jw = (tid >> 6) * 16 + (lane >> 2);   // value index within the workgroup
    const int j0 = bx * W;
    const int Hv = A.Hv, T = A.T, Tp = A.Tp;
    const int g = h / (Hv / A.Hk);

    // the state loads from S_in go out before n_pre is known: S_in is the start state unless
    // every previous row was kept, when the state is read again from S_alt
    const size_t sofs = ((size_t)(b * Hv + h) * DK + ig * R) * DV + j0 + jw;
    float s[R];
#pragma unroll
    for (int r = 0; r < R; ++r) s[r] = A.S_in[sofs + (size_t)r * DV];

    int np = 0;
    if (A.n_pre) {
        np = A.n_pre[b];
        np = np < 0 ? 0 : (np > Tp ? Tp : np);
        if (ROLLBACK) {
            if (bx == 0 && h == 0 && tid == 0) A.kv_len[b] += np;
            if (np == Tp) return;                // state_out already holds S_T
        } else if (np == Tp && A.S_alt) {        // every previous row kept: its S_T, nothing to replay
#pragma unroll
            for (int r = 0; r < R; ++r) s[r] = A.S_alt[sofs + (size_t)r * DV];
            np = 0;
        }
    }
    const int n = np + (ROLLBACK ? 0 : T);
    xv_gdn_stage<DK, W, XV_GDN4_WAVES * 64>(A, b, h, g, j0, np, n, sm.skq, sm.sv, sm.sab);
    __syncthreads();

    // the slab out in two halves of dk / 2 rows through LDS, so that every store is a
    // 16-byte piece of a 256-byte row run (non-temporal: see the L = 16 helper)
    const size_t slab0 = (size_t)(b * Hv + h) * DK * DV + j0;
    auto store_state = [&](float* __restrict__ dst) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            __syncthreads();                     // the half buffer is free
            if ((ig >> 1) == half) {             // lanes holding rows half dk/2 ..
#pragma unroll
                for (int r = 0; r < R; ++r) sm.sst[(ig & 1) * R + r][jw] = s[r];
            }
            __syncthreads();
#pragma unroll
            for (int e = 0; e < DK / 32; ++e) {
                const int rr = (tid >> 4) + 16 * e, cc = (tid & 15) * 4;
                const xv_f32x4 out = *reinterpret_cast<const xv_f32x4*>(&sm.sst[rr][cc]);
                __builtin_nontemporal_store(out, reinterpret_cast<xv_f32x4*>(dst + slab0 + (size_t)(half * (DK / 2) + rr) * DV + cc));
            }
        }
    };
    auto read_row = [&](int t, int which, float (&x)[R]) {
#pragma unroll
        for (int c = 0; c < R / 4; ++c) {
            const xv_f32x4 v4 = *reinterpret_cast<const xv_f32x4*>(&sm.skq[t][which][ig * R + c * 4]);
#pragma unroll
            for (int e = 0; e < 4; ++e) x[c * 4 + e] = v4[e];
        }
    };
    float kk[R], qq[R];
    if (n > 0) read_row(0, 0, kk);
    for (int t = 0; t < n; ++t) {                // uniform
        if (!ROLLBACK && A.S_mid && t == np) store_state(A.S_mid);   // the kept state
        const bool out = !ROLLBACK && t >= np;
        if (out) read_row(t, 1, qq);
        xv_gdn_token<L, R>(s, kk, xv_bf16_to_f32(sm.sv[t][jw]), sm.sab[t][0], sm.sab[t][1]);
        read_row(t + 1 < n ? t + 1 : t, 0, kk);  // the next token's k (read on every path)
        if (out) {
            const float ot = xv_gdn_dot<L, R>(s, qq);
            if (ig == 0) {
                const size_t oi = (((size_t)b * T + (t - np)) * Hv + h) * DV + j0 + jw;
                A.o[oi] = xv_f32_to_bf16(ot);
                if (A.o32) A.o32[oi] = ot;
            }
        }
    }
    if (!ROLLBACK && A.S_mid && n == np) store_state(A.S_mid);      // no rows of this call
    store_state(A.S_out);
}

// 4 lanes per column when the 16-lane grid would take more than about two workgroups per
// CU (the same bits either way).
inline bool xv_gdn_use4(int B, int Hv, int dv) {
    return (dv == 64 || dv == 128) && (long long)B * Hv * (dv / XV_GDN4_W) >= 2LL * xv_cu_count();
}

template <bool ROLLBACK>
int xv_gdn_launch(const XvGdnArgs& args, int B, int dk, hipStream_t st)
{
    (void)hipGetLastError();
    if (xv_gdn_use4(B, args.Hv, args.dv)) {
        dim3 grid(args.dv / XV_GDN4_W, args.Hv, B), block(XV_GDN4_WAVES * 64);
        if (dk == 128 && args.dv == 128) hipLaunchKernelGGL((xv_gdn4_kernel<128, 128, ROLLBACK>), grid, block, 0, st, args);
        else if (dk == 128) hipLaunchKernelGGL((xv_gdn4_kernel<128, 64, ROLLBACK>), grid, block, 0, st, args);
        else if (args.dv == 128) hipLaunchKernelGGL((xv_gdn4_kernel<64, 128, ROLLBACK>), grid, block, 0, st, args);
        else hipLaunchKernelGGL((xv_gdn4_kernel<64, 64, ROLLBACK>), grid, block, 0, st, args);
        return xv_launch_status();
    }
    // one column group per workgroup: the shortest latency when the GDN runs alone
    dim3 grid(args.dv / XV_GDN_JW, args.Hv, B), block(XV_GDN_THREADS);
    if (dk == 128) hipLaunchKernelGGL((xv_gdn_kernel<128, ROLLBACK, 1>), grid, block, 0, st, args);
    else hipLaunchKernelGGL((xv_gdn_kernel<64, ROLLBACK, 1>), grid, block, 0, st, args);
    return xv_launch_status();
}

}  // namespace

extern "C" int xv_gdn_verify(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                             const float* a, const float* b,
                             const float* state_in, float* state_out,
                             uint16_t* o, float* o32,
                             int B, int T, int Hk, int Hv, int dk, int dv, void* stream)
{
    XvGdnArgs args{};
    const int s = xv_gdn_args_verify(args, q, k, v, a, b, state_in, state_out, o, o32, B, T, Hk, Hv, dk, dv);
    if (s != XV_OK || B == 0) return s;
    return xv_gdn_launch<false>(args, B, dk, reinterpret_cast<hipStream_t>(stream));
}

extern "C" int xv_gdn_verify_after(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                   const float* a, const float* b,
                                   const uint16_t* k_prev, const uint16_t* v_prev,
                                   const float* a_prev, const float* b_prev,
                                   const int32_t* n_keep_prev, int T_prev,
                                   const float* state_prev_in, const float* state_prev_out,
                                   float* state_kept, float* state_out,
                                   uint16_t* o, float* o32,
                                   int B, int T, int Hk, int Hv, int dk, int dv, void* stream)
{
    XvGdnArgs args{};
    const int s = xv_gdn_args_after(args, q, k, v, a, b, k_prev, v_prev, a_prev, b_prev, n_keep_prev, T_prev,
                                    state_prev_in, state_prev_out, state_kept, state_out, o, o32,
                                    B, T, Hk, Hv, dk, dv);
    if (s != XV_OK || B == 0) return s;
    return xv_gdn_launch<false>(args, B, dk, reinterpret_cast<hipStream_t>(stream));
}

extern "C" int xv_gdn_prefill(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const float* a, const float* b,
                              const float* state_in, float* state_out,
                              uint16_t* o, float* o32,
                              int B, int T, int Hk, int Hv, int dk, int dv, void* stream)
{
    int s = xv_gdn_check(k, v, a, b, state_in, state_out, B, T, Hk, Hv, dk, dv, 1 << 30);
    if (s != XV_OK || B == 0) return s;
    XV_REQUIRE(q && o, XV_ERR_NULL);
    XV_REQUIRE(xv_aligned16(q) && xv_aligned(o, 2) && xv_aligned(o32, 4), XV_ERR_ALIGN);
    XvGdnArgs args{};
    args.q = q; args.k = k; args.v = v; args.a = a; args.b = b; args.T = T;
    args.S_in = state_in; args.S_out = state_out; args.o = o; args.o32 = o32;
    args.Hk = Hk; args.Hv = Hv; args.dv = dv;
    dim3 grid(dv / XV_GDN_JW, Hv, B), block(XV_GDN_THREADS);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (dk == 128) hipLaunchKernelGGL(xv_gdn_prefill_kernel<128>, grid, block, 0, st, args);
    else hipLaunchKernelGGL(xv_gdn_prefill_kernel<64>, grid, block, 0, st, args);
    return xv_launch_status();
}

extern "C" int xv_rollback_to_prefix(const uint16_t* k, const uint16_t* v,
                                     const float* a, const float* b,
                                     const float* state_in, float* state_out,
                                     int32_t* kv_len, const int32_t* n_keep,
                                     int B, int T, int Hk, int Hv, int dk, int dv, void* stream)
{
    int s = xv_gdn_check(k, v, a, b, state_in, state_out, B, T, Hk, Hv, dk, dv);
    if (s != XV_OK || B == 0) return s;
    XV_REQUIRE(kv_len && n_keep, XV_ERR_NULL);
    XV_REQUIRE(xv_aligned(kv_len, 4) && xv_aligned(n_keep, 4), XV_ERR_ALIGN);
    XvGdnArgs args{};
    args.kp = k; args.vp = v; args.ap = a; args.bp = b; args.n_pre = n_keep; args.Tp = T;
    args.T = 0; args.S_in = state_in; args.S_out = state_out; args.kv_len = kv_len;
    args.Hk = Hk; args.Hv = Hv; args.dv = dv;
    return xv_gdn_launch<true>(args, B, dk, reinterpret_cast<hipStream_t>(stream));
}
