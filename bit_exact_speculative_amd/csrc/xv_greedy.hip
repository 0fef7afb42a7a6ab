// xv_greedy.hip -- greedy (temperature 0) acceptance of draft tokens on device.
//
// The post compares greedy decoding at temperature zero on token ids.  For each
// verify row the id is the argmax of the row's logits, ties going to the lowest
// index; the drafts are accepted while each equals the id produced by the row
// before it.  The argmax result is unique, so the reduction order below does
// not matter for the bits (the comparison is exact and total on finite values).
#include "xv_common.h"

namespace {

constexpr int XV_GREEDY_THREADS = 256;

__device__ __forceinline__ bool xv_better(float v1, int n1, float v0, int n0) {
    return v1 > v0 || (v1 == v0 && n1 < n0);
}

__global__ __launch_bounds__(XV_GREEDY_THREADS)
void xv_greedy_kernel(const float* __restrict__ la, const float* __restrict__ lb,
                      const int32_t* __restrict__ draft, int T, int N,
                      int32_t* __restrict__ ids, int32_t* __restrict__ n_keep)
{
    __shared__ float sv[XV_GREEDY_THREADS];
    __shared__ int sn[XV_GREEDY_THREADS];
    __shared__ int sid[16];
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    for (int t = 0; t < T; ++t) {
        const size_t row = ((size_t)b * T + t) * N;
        float best = -INFINITY;
        int bn = N;                              // sentinel: larger than any index
        for (int n = tid; n < N; n += XV_GREEDY_THREADS) {
            const float val = lb ? la[row + n] + lb[row + n] : la[row + n];
            if (xv_better(val, n, best, bn)) { best = val; bn = n; }
        }
        sv[tid] = best;
        sn[tid] = bn;
        __syncthreads();
        for (int s = XV_GREEDY_THREADS / 2; s > 0; s >>= 1) {
            if (tid < s && xv_better(sv[tid + s], sn[tid + s], sv[tid], sn[tid])) {
                sv[tid] = sv[tid + s];
                sn[tid] = sn[tid + s];
            }
            __syncthreads();
        }
        if (tid == 0) {
            const int id = sn[0] < N ? sn[0] : 0;
            ids[(size_t)b * T + t] = id;
            sid[t] = id;
        }
        __syncthreads();
    }
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
    XV_REQUIRE(B >= 0 && T >= 1 && T <= 16 && N >= 1, XV_ERR_SHAPE);
    if (B == 0) return XV_OK;
    XV_REQUIRE(logits_a && draft && ids && n_keep, XV_ERR_NULL);
    XV_REQUIRE(xv_aligned(logits_a, 4) && xv_aligned(logits_b, 4) && xv_aligned(draft, 4) &&
               xv_aligned(ids, 4) && xv_aligned(n_keep, 4), XV_ERR_ALIGN);
    (void)hipGetLastError();
    hipLaunchKernelGGL(xv_greedy_kernel, dim3(B), dim3(XV_GREEDY_THREADS), 0,
                       reinterpret_cast<hipStream_t>(stream), logits_a, logits_b, draft, T, N,
                       ids, n_keep);
    return xv_launch_status();
}
