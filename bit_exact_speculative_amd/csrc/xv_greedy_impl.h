// xv_greedy_impl.h -- the greedy-acceptance arithmetic shared by the stand-alone greedy
// kernels (xv_greedy.hip) and the head GEMM that forms its block partials itself
// (xv_gemm.hip).  Both produce the same ids, logprobs and counts bit for bit because
// they run these functions in the order described with xv_row_scan in xv_greedy.hip:
//  * a 16-column block's pair (m, s): m its maximum, s = sum_c e^(z_c - m) as a
//    butterfly over the columns (c with c ^ 8, then ^ 4, ^ 2, ^ 1);
//  * chain j (j = 0..255) folds the pairs of blocks j, j + 256, j + 512, ... left to
//    right from the empty pair (-inf, 0) with xv_lse_add;
//  * the chains of each group of 64 meet in a butterfly (chain ^ 1, ^ 2, ..., ^ 32),
//    the four groups fold left to right, and lp = -ln S.
// The argmax (lowest index among the maxima) is unique, so its reduction order is free.
#pragma once

#include "xv_common.h"

constexpr int XV_TMAX = 16;           // verify rows per request, at most
constexpr float XV_LOG2E = 1.4426950408889634f;

__device__ __forceinline__ bool xv_better(float v1, int n1, float v0, int n0) {
    return v1 > v0 || (v1 == v0 && n1 < n0);
}

// (m, s) += (m2, s2): (M, s e^(m - M) + s2 e^(m2 - M)), M = max(m, m2); an empty pair
// (-inf, 0) contributes nothing.  Each e^x is 2^(x log2 e) on the hardware exp2.
__device__ __forceinline__ void xv_lse_add(float& m, float& s, float m2, float s2) {
    const float mm = fmaxf(m, m2);
    const float t1 = m == -INFINITY ? 0.f : s * __builtin_amdgcn_exp2f((m - mm) * XV_LOG2E);
    const float t2 = m2 == -INFINITY ? 0.f : s2 * __builtin_amdgcn_exp2f((m2 - mm) * XV_LOG2E);
    m = mm;
    s = t1 + t2;
}

// lp = -ln S (S > 0: the row's maximum contributes e^0 = 1)
__device__ __forceinline__ float xv_neg_log(float s) {
    constexpr float LN2 = 0.6931471805599453f;
    return -(__builtin_amdgcn_logf(s) * LN2);
}

// Accepted drafts of one request: the leading rows whose id equals the next row's draft.
// draft_of(t) and id_of(t) give row t's draft and id; all are read before the first compare.
template <typename DraftFn, typename IdFn>
__device__ __forceinline__ int xv_accepted(int T, DraftFn draft_of, IdFn id_of) {
    int dr[XV_TMAX], id[XV_TMAX];
#pragma unroll
    for (int t = 0; t < XV_TMAX; ++t) {
        const int tc = t < T ? t : T - 1;
        dr[t] = draft_of(tc);
        id[t] = id_of(tc);
    }
    int acc = 0;
    bool run = true;
#pragma unroll
    for (int t = 0; t + 1 < XV_TMAX; ++t) {
        run = run && t + 1 < T && dr[t + 1] == id[t];
        acc += run ? 1 : 0;
    }
    return acc;
}
