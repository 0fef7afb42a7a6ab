// xv_greedy.hip -- greedy (temperature 0) acceptance of draft tokens on device.
//
// The post compares greedy decoding at temperature zero on token ids.  For each
// verify row the id is the argmax of the row's logits, ties going to the lowest
// index; the drafts are accepted while each equals the id produced by the row
// before it.  The argmax is unique, so the reduction order below does not
// matter for the result (the comparison is exact and total on finite values).
//
// Two kernels on the caller's stream: one workgroup per verify row reduces the
// row (running (value, index) per thread over a strided slice, then lane
// shuffles and LDS across the waves) and optionally forms the id's logprob,
// then one thread per request counts the accepted drafts.
#include "xv_greedy_impl.h"

namespace {

constexpr int XV_GREEDY_THREADS = 256;
constexpr int XV_GREEDY_WAVES = XV_GREEDY_THREADS / 64;

// One workgroup per verify row (grid T x B), one pass over the row: the argmax
// of the logits and, when lp is given, the logprob of that id.  Thread t owns the
// 16-column blocks t, t + 256, t + 512, ... of the row (block b: columns
// 16b .. 16b + 15, the last block may be partial), read as four 16-byte loads
// (VEC: rows 16-byte aligned, N % 4 == 0) or sixteen 4-byte loads; the order of
// everything below is the same either way, and columns past the row re-read its
// last element and are masked out.
//
// Logprob of the argmax (post, first paragraph: logprobs compared as well as
// ids), lp = -ln S with S = sum_n e^(z_n - max z), in an order fixed by N:
//  * a block's pair (m, s) is its maximum and sum_c e^(z_c - m), the sum as a
//    butterfly over the columns (c with c ^ 8, then ^ 4, ^ 2, ^ 1);
//  * pairs combine as (m1, s1) + (m2, s2) = (M, s1 e^(m1 - M) + s2 e^(m2 - M)),
//    M = max(m1, m2), an empty pair (-inf, 0) contributing nothing; block b
//    belongs to chain b mod 256, whose blocks fold left to right; the chains then
//    meet in a butterfly (chain ^ 1, ^ 2, ..., ^ 32) within each group of 64 and
//    the four groups fold left to right (every butterfly level adds two partials
//    that its partner adds the other way round, so all agree).
// Each e^x is 2^(x log2 e) on the hardware exp2; M is exact (a maximum), so
// lp = -ln S.  None of it depends on T, B or the other rows, and a producer that
// forms the 16-column blocks itself (in any order) can reproduce it.
template <bool VEC>
__device__ __forceinline__ void xv_row_block(const float* __restrict__ la, const float* __restrict__ lb,
                                             size_t row, int N, int blk, float (&x)[16]) {
    const int nb = (N + 15) >> 4;
    const int bc = blk < nb ? blk : nb - 1;
    if (VEC) {
        // N % 4 == 0: the block's four 16-byte groups, a group past the row re-reading the last
        const int G = N >> 2;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int gi = bc * 4 + q4;
            const int gc = gi < G ? gi : G - 1;
            const float4 va = reinterpret_cast<const float4*>(la + row)[gc];
            float4 vb = va;
            if (lb) vb = reinterpret_cast<const float4*>(lb + row)[gc];
            x[4 * q4] = va.x; x[4 * q4 + 1] = va.y; x[4 * q4 + 2] = va.z; x[4 * q4 + 3] = va.w;
            if (lb) {
                x[4 * q4] = x[4 * q4] + vb.x; x[4 * q4 + 1] = x[4 * q4 + 1] + vb.y;
                x[4 * q4 + 2] = x[4 * q4 + 2] + vb.z; x[4 * q4 + 3] = x[4 * q4 + 3] + vb.w;
            }
        }
    } else {
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            const int n = 16 * bc + c;
            const int nc = n < N ? n : N - 1;
            x[c] = la[row + nc];
            if (lb) x[c] = x[c] + lb[row + nc];
        }
    }
}

constexpr int XV_GREEDY_BPP = 2;      // blocks per thread per pass, all loaded before any compare

// One row's scan by 256 threads (ltid = 0..255): the thread's chain of 16-column blocks
// and its running argmax, then the 64-lane butterflies.
template <bool VEC>
__device__ __forceinline__ void xv_row_scan(const float* __restrict__ la, const float* __restrict__ lb,
                                            size_t row, int N, int ltid, bool want_lp,
                                            float& best, int& bn, float& cm, float& cs)
{
    const int nb = (N + 15) >> 4;
    best = -INFINITY;
    bn = N;                                      // sentinel: after every real index
    cm = -INFINITY; cs = 0.f;                    // this thread's chain: blocks ltid + 256 i
    for (int b0 = ltid; b0 < nb; b0 += XV_GREEDY_THREADS * XV_GREEDY_BPP) {
        float x[XV_GREEDY_BPP][16];
#pragma unroll
        for (int u = 0; u < XV_GREEDY_BPP; ++u) xv_row_block<VEC>(la, lb, row, N, b0 + u * XV_GREEDY_THREADS, x[u]);
#pragma unroll
        for (int u = 0; u < XV_GREEDY_BPP; ++u) {
            const int blk = b0 + u * XV_GREEDY_THREADS;
            float bm = -INFINITY;
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                const int n = 16 * blk + c;
                const bool ok = blk < nb && n < N;
                if (ok && xv_better(x[u][c], n, best, bn)) { best = x[u][c]; bn = n; }
                bm = ok ? fmaxf(bm, x[u][c]) : bm;
            }
            if (want_lp) {                       // uniform
                float e[16];
#pragma unroll
                for (int c = 0; c < 16; ++c) {
                    const bool ok = blk < nb && 16 * blk + c < N;
                    e[c] = ok ? __builtin_amdgcn_exp2f((x[u][c] - bm) * XV_LOG2E) : 0.f;
                }
#pragma unroll
                for (int c = 0; c < 8; ++c) e[c] = e[c] + e[c + 8];
#pragma unroll
                for (int c = 0; c < 4; ++c) e[c] = e[c] + e[c + 4];
#pragma unroll
                for (int c = 0; c < 2; ++c) e[c] = e[c] + e[c + 2];
                xv_lse_add(cm, cs, bm, e[0] + e[1]);
            }
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float ov = __shfl_xor(best, off);
        const int on = __shfl_xor(bn, off);
        if (xv_better(ov, on, best, bn)) { best = ov; bn = on; }
    }
    if (want_lp) {
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) xv_lse_add(cm, cs, __shfl_xor(cm, off), __shfl_xor(cs, off));
    }
}

// The four waves of a row folded left to right: the id (lowest index among the maxima) and
// lp = -ln S.
__device__ __forceinline__ void xv_row_fold(const float* sv, const int* sn, const float* sm, const float* ssum,
                                            int N, int& id, float& lpv)
{
    float best = sv[0];
    int bn = sn[0];
    for (int w = 1; w < XV_GREEDY_WAVES; ++w)
        if (xv_better(sv[w], sn[w], best, bn)) { best = sv[w]; bn = sn[w]; }
    id = bn < N ? bn : 0;
    float m = sm[0], sum = ssum[0];
    for (int w = 1; w < XV_GREEDY_WAVES; ++w) xv_lse_add(m, sum, sm[w], ssum[w]);
    lpv = xv_neg_log(sum);
}

template <bool VEC>
__global__ __launch_bounds__(XV_GREEDY_THREADS)
void xv_argmax_kernel(const float* __restrict__ la, const float* __restrict__ lb, int T, int N,
                      int32_t* __restrict__ ids, float* __restrict__ lp)
{
    __shared__ float sv[XV_GREEDY_WAVES];
    __shared__ int sn[XV_GREEDY_WAVES];
    __shared__ float sm[XV_GREEDY_WAVES], ssum[XV_GREEDY_WAVES];
    const int t = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x;
    float best, cm, cs;
    int bn;
    xv_row_scan<VEC>(la, lb, ((size_t)b * T + t) * N, N, tid, lp != nullptr, best, bn, cm, cs);
    if ((tid & 63) == 0) { sv[tid >> 6] = best; sn[tid >> 6] = bn; sm[tid >> 6] = cm; ssum[tid >> 6] = cs; }
    __syncthreads();
    if (tid == 0) {
        int id;
        float lpv;
        xv_row_fold(sv, sn, sm, ssum, N, id, lpv);
        ids[(size_t)b * T + t] = id;
        if (lp) lp[(size_t)b * T + t] = lpv;
    }
}

// One thread per request: accepted drafts = leading rows whose id equals the next draft.
// All of the request's ids and drafts are loaded before the first compare (one round trip).
// kv_len (optional): the request's cached length grows by the kept rows.
__global__ void xv_accept_kernel(const int32_t* __restrict__ draft, const int32_t* __restrict__ ids,
                                 int B, int T, int32_t* __restrict__ n_keep, int32_t* __restrict__ kv_len)
{
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    const int acc = xv_accepted(T, [&](int t) { return draft[(size_t)b * T + t]; },
                                [&](int t) { return ids[(size_t)b * T + t]; });
    n_keep[b] = acc + 1;
    if (kv_len) kv_len[b] += acc + 1;
}

// xv_argmax_kernel and xv_accept_kernel in one launch, for callers with a workspace: each
// row's workgroup stores its id with a device-coherent store, waits for it, and counts the
// row in its request's counter; the workgroup that sees the request's last row loads the
// request's ids (device-coherent loads) and counts the accepted drafts, exactly as
// xv_accept_kernel does, then resets the counter to zero.
template <bool VEC>
__global__ __launch_bounds__(XV_GREEDY_THREADS)
void xv_argmax_accept_kernel(const float* __restrict__ la, const float* __restrict__ lb,
                             const int32_t* __restrict__ draft, int T, int N, int32_t* ids,
                             float* __restrict__ lp, int32_t* __restrict__ n_keep, int32_t* __restrict__ kv_len,
                             int* __restrict__ counters)
{
    __shared__ float sv[XV_GREEDY_WAVES];
    __shared__ int sn[XV_GREEDY_WAVES];
    __shared__ float sm[XV_GREEDY_WAVES], ssum[XV_GREEDY_WAVES];
    const int t = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x;
    float best, cm, cs;
    int bn;
    xv_row_scan<VEC>(la, lb, ((size_t)b * T + t) * N, N, tid, lp != nullptr, best, bn, cm, cs);
    if ((tid & 63) == 0) { sv[tid >> 6] = best; sn[tid >> 6] = bn; sm[tid >> 6] = cm; ssum[tid >> 6] = cs; }
    __syncthreads();
    if (tid != 0) return;
    int id;
    float lpv;
    xv_row_fold(sv, sn, sm, ssum, N, id, lpv);
    __hip_atomic_store(&ids[(size_t)b * T + t], id, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (lp) lp[(size_t)b * T + t] = lpv;
    __builtin_amdgcn_s_waitcnt(0x0F70);          // vmcnt(0): the id store has completed
    if (atomicAdd(&counters[b], 1) != T - 1) return;
    const int acc = xv_accepted(T, [&](int r) { return draft[(size_t)b * T + r]; },
                                [&](int r) { return (int)__hip_atomic_load(&ids[(size_t)b * T + r], __ATOMIC_RELAXED,
                                                                            __HIP_MEMORY_SCOPE_AGENT); });
    n_keep[b] = acc + 1;
    if (kv_len) kv_len[b] += acc + 1;
    __hip_atomic_store(&counters[b], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

namespace xv_detail {

int xv_greedy_accept_counted(const float* logits_a, const float* logits_b, const int32_t* draft,
                             int B, int T, int N, int32_t* ids, int32_t* n_keep, float* logprob,
                             int32_t* kv_len, int* counters, void* stream)
{
    (void)hipGetLastError();
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const bool vec = (N % 4 == 0) && xv_aligned16(logits_a) && xv_aligned16(logits_b);
    const dim3 grid(T, B), block(XV_GREEDY_THREADS);
    if (vec)
        hipLaunchKernelGGL(xv_argmax_accept_kernel<true>, grid, block, 0, st, logits_a, logits_b, draft, T, N, ids,
                           logprob, n_keep, kv_len, counters);
    else
        hipLaunchKernelGGL(xv_argmax_accept_kernel<false>, grid, block, 0, st, logits_a, logits_b, draft, T, N, ids,
                           logprob, n_keep, kv_len, counters);
    return xv_launch_status();
}

}  // namespace xv_detail

extern "C" int xv_greedy_accept(const float* logits_a, const float* logits_b, const int32_t* draft,
                                int B, int T, int N, int32_t* ids, int32_t* n_keep, float* logprob,
                                int32_t* kv_len, void* stream)
{
    XV_REQUIRE(B >= 0 && T >= 1 && T <= XV_TMAX && N >= 1, XV_ERR_SHAPE);
    if (B == 0) return XV_OK;
    XV_REQUIRE(logits_a && draft && ids && n_keep, XV_ERR_NULL);
    XV_REQUIRE(xv_aligned(logits_a, 4) && xv_aligned(logits_b, 4) && xv_aligned(draft, 4) &&
               xv_aligned(ids, 4) && xv_aligned(n_keep, 4) && xv_aligned(logprob, 4) &&
               xv_aligned(kv_len, 4), XV_ERR_ALIGN);
    (void)hipGetLastError();
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    // 16-byte loads when every row starts 16-byte aligned; the argmax is the same either way
    const bool vec = (N % 4 == 0) && xv_aligned16(logits_a) && xv_aligned16(logits_b);
    const dim3 grid(T, B), block(XV_GREEDY_THREADS);
    if (vec) hipLaunchKernelGGL(xv_argmax_kernel<true>, grid, block, 0, st, logits_a, logits_b, T, N, ids, logprob);
    else hipLaunchKernelGGL(xv_argmax_kernel<false>, grid, block, 0, st, logits_a, logits_b, T, N, ids, logprob);
    const int s1 = xv_launch_status();
    if (s1 != XV_OK) return s1;
    hipLaunchKernelGGL(xv_accept_kernel, dim3((B + 63) / 64), dim3(64), 0, st, draft, ids, B, T, n_keep, kv_len);
    return xv_launch_status();
}
