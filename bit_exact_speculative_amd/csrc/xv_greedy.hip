// xv_greedy.hip -- greedy (temperature 0) acceptance of draft tokens on device.
//
// The post compares greedy decoding at temperature zero on token ids.  For each
// verify row the id is the argmax of the row's logits, ties going to the lowest
// index; the drafts are accepted while each equals the id produced by the row
// before it.  The argmax is unique, so the reduction order below does not
// matter for the result (the comparison is exact and total on finite values).
//
// One 1024-thread workgroup per request scans all T rows at once: every thread
// keeps a running (value, index) per row over a strided slice, then the rows
// are reduced across the wave with lane shuffles and across the 16 waves in
// LDS, and thread 0 counts the accepted drafts.
#include "xv_common.h"

namespace {

constexpr int XV_GREEDY_THREADS = 1024;
constexpr int XV_GREEDY_WAVES = XV_GREEDY_THREADS / 64;
constexpr int XV_TMAX = 16;           // verify rows per request, at most

__device__ __forceinline__ bool xv_better(float v1, int n1, float v0, int n0) {
    return v1 > v0 || (v1 == v0 && n1 < n0);
}

// TT >= T rows per pass; rows past T re-read row T-1 and are ignored, so the
// loads of all rows are straight-line code and stay in flight together.
template <int TT>
__global__ __launch_bounds__(XV_GREEDY_THREADS)
void xv_greedy_kernel(const float* __restrict__ la, const float* __restrict__ lb,
                      const int32_t* __restrict__ draft, int T, int N,
                      int32_t* __restrict__ ids, int32_t* __restrict__ n_keep)
{
    __shared__ float sv[XV_GREEDY_WAVES][TT];
    __shared__ int sn[XV_GREEDY_WAVES][TT];
    __shared__ int sid[TT];
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;

    float best[TT];
    int bn[TT];
    size_t rowoff[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        best[t] = -INFINITY;
        bn[t] = N;                                   // sentinel: after every real index
        rowoff[t] = ((size_t)b * T + (t < T ? t : T - 1)) * N;
    }
    for (int n = tid; n < N; n += XV_GREEDY_THREADS) {
        float val[TT];
#pragma unroll
        for (int t = 0; t < TT; ++t) val[t] = la[rowoff[t] + n];
        if (lb) {
#pragma unroll
            for (int t = 0; t < TT; ++t) val[t] = val[t] + lb[rowoff[t] + n];
        }
#pragma unroll
        for (int t = 0; t < TT; ++t)
            if (xv_better(val[t], n, best[t], bn[t])) { best[t] = val[t]; bn[t] = n; }
    }
#pragma unroll
    for (int t = 0; t < TT; ++t) {
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const float ov = __shfl_xor(best[t], off);
            const int on = __shfl_xor(bn[t], off);
            if (xv_better(ov, on, best[t], bn[t])) { best[t] = ov; bn[t] = on; }
        }
        if (lane == 0) { sv[wave][t] = best[t]; sn[wave][t] = bn[t]; }
    }
    __syncthreads();
    if (tid < T) {
        float bv = sv[0][tid];
        int bi = sn[0][tid];
        for (int w = 1; w < XV_GREEDY_WAVES; ++w)
            if (xv_better(sv[w][tid], sn[w][tid], bv, bi)) { bv = sv[w][tid]; bi = sn[w][tid]; }
        const int id = bi < N ? bi : 0;
        ids[(size_t)b * T + tid] = id;
        sid[tid] = id;
    }
    __syncthreads();
    if (tid == 0) {
        int acc = 0;
        while (acc + 1 < T && draft[(size_t)b * T + acc + 1] == sid[acc]) ++acc;
        n_keep[b] = acc + 1;
    }
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
    const dim3 grid(B), block(XV_GREEDY_THREADS);
    if (T <= 1)
        hipLaunchKernelGGL(xv_greedy_kernel<1>, grid, block, 0, st, logits_a, logits_b, draft, T, N, ids, n_keep);
    else if (T <= 4)
        hipLaunchKernelGGL(xv_greedy_kernel<4>, grid, block, 0, st, logits_a, logits_b, draft, T, N, ids, n_keep);
    else if (T <= 9)
        hipLaunchKernelGGL(xv_greedy_kernel<9>, grid, block, 0, st, logits_a, logits_b, draft, T, N, ids, n_keep);
    else
        hipLaunchKernelGGL(xv_greedy_kernel<16>, grid, block, 0, st, logits_a, logits_b, draft, T, N, ids, n_keep);
    return xv_launch_status();
}
