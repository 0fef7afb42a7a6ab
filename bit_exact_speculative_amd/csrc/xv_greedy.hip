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
// shuffles and LDS across the waves), then one thread per request counts the
// accepted drafts.
#include "xv_common.h"

namespace {

constexpr int XV_GREEDY_THREADS = 256;
constexpr int XV_GREEDY_WAVES = XV_GREEDY_THREADS / 64;
constexpr int XV_TMAX = 16;           // verify rows per request, at most
constexpr int XV_GREEDY_UNROLL = 4;   // strides per pass, all loaded before any compare

__device__ __forceinline__ bool xv_better(float v1, int n1, float v0, int n0) {
    return v1 > v0 || (v1 == v0 && n1 < n0);
}

// One workgroup per verify row (grid T x B): argmax of the row's logits.
// VEC: 16-byte loads (rows 16-byte aligned, N % 4 == 0); otherwise 4-byte loads.
// Indices past the row re-read its last element and are masked out.
template <bool VEC>
__global__ __launch_bounds__(XV_GREEDY_THREADS)
void xv_argmax_kernel(const float* __restrict__ la, const float* __restrict__ lb, int T, int N,
                      int32_t* __restrict__ ids)
{
    __shared__ float sv[XV_GREEDY_WAVES];
    __shared__ int sn[XV_GREEDY_WAVES];
    const int t = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x;
    const size_t row = ((size_t)b * T + t) * N;
    float best = -INFINITY;
    int bn = N;                                  // sentinel: after every real index
    if (VEC) {
        const float4* pa = reinterpret_cast<const float4*>(la + row);
        const float4* pb = reinterpret_cast<const float4*>(lb ? lb + row : la + row);
        const int N4 = N >> 2;
        for (int v0 = tid; v0 < N4; v0 += XV_GREEDY_THREADS * XV_GREEDY_UNROLL) {
            float4 va[XV_GREEDY_UNROLL], vb[XV_GREEDY_UNROLL];
#pragma unroll
            for (int u = 0; u < XV_GREEDY_UNROLL; ++u) {
                const int v = v0 + u * XV_GREEDY_THREADS;
                const int vc = v < N4 ? v : N4 - 1;
                va[u] = pa[vc];
                vb[u] = pb[vc];
            }
#pragma unroll
            for (int u = 0; u < XV_GREEDY_UNROLL; ++u) {
                const int v = v0 + u * XV_GREEDY_THREADS;
                if (v < N4) {
                    float4 x = va[u];
                    if (lb) { x.x = x.x + vb[u].x; x.y = x.y + vb[u].y; x.z = x.z + vb[u].z; x.w = x.w + vb[u].w; }
                    const int n = 4 * v;
                    if (xv_better(x.x, n, best, bn)) { best = x.x; bn = n; }
                    if (xv_better(x.y, n + 1, best, bn)) { best = x.y; bn = n + 1; }
                    if (xv_better(x.z, n + 2, best, bn)) { best = x.z; bn = n + 2; }
                    if (xv_better(x.w, n + 3, best, bn)) { best = x.w; bn = n + 3; }
                }
            }
        }
    } else {
        for (int n0 = tid; n0 < N; n0 += XV_GREEDY_THREADS * XV_GREEDY_UNROLL) {
            float va[XV_GREEDY_UNROLL], vb[XV_GREEDY_UNROLL];
#pragma unroll
            for (int u = 0; u < XV_GREEDY_UNROLL; ++u) {
                const int n = n0 + u * XV_GREEDY_THREADS;
                const int nc = n < N ? n : N - 1;
                va[u] = la[row + nc];
                vb[u] = lb ? lb[row + nc] : 0.f;
            }
#pragma unroll
            for (int u = 0; u < XV_GREEDY_UNROLL; ++u) {
                const int n = n0 + u * XV_GREEDY_THREADS;
                const float x = lb ? va[u] + vb[u] : va[u];
                if (n < N && xv_better(x, n, best, bn)) { best = x; bn = n; }
            }
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float ov = __shfl_xor(best, off);
        const int on = __shfl_xor(bn, off);
        if (xv_better(ov, on, best, bn)) { best = ov; bn = on; }
    }
    if ((tid & 63) == 0) { sv[tid >> 6] = best; sn[tid >> 6] = bn; }
    __syncthreads();
    if (tid == 0) {
        for (int w = 1; w < XV_GREEDY_WAVES; ++w)
            if (xv_better(sv[w], sn[w], best, bn)) { best = sv[w]; bn = sn[w]; }
        ids[(size_t)b * T + t] = bn < N ? bn : 0;
    }
}

// One thread per request: accepted drafts = leading rows whose id equals the next draft.
// All of the request's ids and drafts are loaded before the first compare (one round trip).
__global__ void xv_accept_kernel(const int32_t* __restrict__ draft, const int32_t* __restrict__ ids,
                                 int B, int T, int32_t* __restrict__ n_keep)
{
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    int dr[XV_TMAX], id[XV_TMAX];
#pragma unroll
    for (int t = 0; t < XV_TMAX; ++t) {
        const int tc = t < T ? t : T - 1;
        dr[t] = draft[(size_t)b * T + tc];
        id[t] = ids[(size_t)b * T + tc];
    }
    int acc = 0;
    bool run = true;
#pragma unroll
    for (int t = 0; t + 1 < XV_TMAX; ++t) {
        run = run && t + 1 < T && dr[t + 1] == id[t];
        acc += run ? 1 : 0;
    }
    n_keep[b] = acc + 1;
}

}  // namespace

extern "C" int xv_greedy_accept(const float* logits_a, const float* logits_b, const int32_t* draft,
                                int B, int T, int N, int32_t* ids, int32_t* n_keep, void* stream)
{
    XV_REQUIRE(B >= 0 && T >= 1 && T <= XV_TMAX && N >= 1, XV_ERR_SHAPE);
    if (B == 0) return XV_OK;
    XV_REQUIRE(logits_a && draft && ids && n_keep, XV_ERR_NULL);
    XV_REQUIRE(xv_aligned(logits_a, 4) && xv_aligned(logits_b, 4) && xv_aligned(draft, 4) &&
               xv_aligned(ids, 4) && xv_aligned(n_keep, 4), XV_ERR_ALIGN);
    (void)hipGetLastError();
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    // 16-byte loads when every row starts 16-byte aligned; the argmax is the same either way
    const bool vec = (N % 4 == 0) && xv_aligned16(logits_a) && xv_aligned16(logits_b);
    const dim3 grid(T, B), block(XV_GREEDY_THREADS);
    if (vec) hipLaunchKernelGGL(xv_argmax_kernel<true>, grid, block, 0, st, logits_a, logits_b, T, N, ids);
    else hipLaunchKernelGGL(xv_argmax_kernel<false>, grid, block, 0, st, logits_a, logits_b, T, N, ids);
    const int s1 = xv_launch_status();
    if (s1 != XV_OK) return s1;
    hipLaunchKernelGGL(xv_accept_kernel, dim3((B + 63) / 64), dim3(64), 0, st, draft, ids, B, T, n_keep);
    return xv_launch_status();
}
