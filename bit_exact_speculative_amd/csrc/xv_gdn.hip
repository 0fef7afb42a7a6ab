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
// Work mapping (gfx950, wave64): a workgroup of 8 waves owns 32 value indices
// of one (request, value head) (64, two columns per lane, when it shares a launch
// with attention and the chip is short of CUs for one column); in a wave,
// 16 lanes share a column and each holds R = dk/16 consecutive key indices of it
// in VGPRs, for the whole call (so the recurrence's dependency chain per token is
// short, and a batch-1 call still gives every SIMD more than one wave to
// interleave).
// The fixed dot order: in each lane four fp32 chains over i mod 4 in ascending
// i, combined as (c0 + c1) + (c2 + c3); then a butterfly over the 16 lanes
// (DPP: partner lane^1, lane^2, the mirrored half of each 8, the mirrored
// half of the 16).  Every lane ends with the same bits (each step adds the
// same two values in either order), so all lanes of a column compute the same
// u.  The state is read once and written once per call; the rows of all
// tokens are staged in LDS (k and q already widened to fp32) before the token
// loop starts.
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

template <bool ROLLBACK>
int xv_gdn_launch(const XvGdnArgs& args, int B, int dk, hipStream_t st)
{
    // one column group per workgroup: the shortest latency when the GDN runs alone
    dim3 grid(args.dv / XV_GDN_JW, args.Hv, B), block(XV_GDN_THREADS);
    (void)hipGetLastError();
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
