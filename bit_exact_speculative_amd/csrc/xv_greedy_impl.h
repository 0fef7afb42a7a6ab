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

// Lane moves within each row of 16 lanes (DPP; every source lane lies in the row):
// XOR1 / XOR2 give lane c ^ 1 / c ^ 2, ROR8 lane c ^ 8, ROR12 lane (c + 4) mod 16, and
// HALF_MIRROR lane 7 - c within each 8.  Where a butterfly level has made lanes c and c ^ m
// equal, a move to any lane of the partner's class gives the partner's value: ROR12 after
// the ^ 8 level stands for ^ 4, HALF_MIRROR after the ^ 1 and ^ 2 levels for ^ 4.
constexpr int XV_DPP_XOR1 = 0xB1, XV_DPP_XOR2 = 0x4E, XV_DPP_ROR8 = 0x128, XV_DPP_ROR12 = 0x12C,
              XV_DPP_HALF_MIRROR = 0x141;
template <int CTRL>
__device__ __forceinline__ float xv_dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int xv_dpp(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

// lp = -ln S (S > 0: the row's maximum contributes e^0 = 1)
__device__ __forceinline__ float xv_neg_log(float s) {
    constexpr float LN2 = 0.6931471805599453f;
    return -(__builtin_amdgcn_logf(s) * LN2);
}

// The argmax and acceptance of xv_greedy_accept in one launch (the same bits), with one
// arrival counter per request in counters[0 .. B) (zero on entry, zero on exit); arguments
// as xv_greedy_accept, already checked by the caller.
namespace xv_detail {
__attribute__((visibility("hidden")))
int xv_greedy_accept_counted(const float* logits_a, const float* logits_b, const int32_t* draft,
                             int B, int T, int N, int32_t* ids, int32_t* n_keep, float* logprob,
                             int32_t* kv_len, int* counters, void* stream);
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
