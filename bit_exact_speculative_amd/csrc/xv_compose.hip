// xv_compose.hip -- the steps that join the verify kernels into a decoding
// step of one synthetic hybrid layer: the token embedding gather in front of
// the projection GEMMs, and the split of the projection rows into the
// per-head operands of the GDN and attention calls.
//
// The post (first paragraph) checks that speculative and plain greedy decoding
// give the same token ids and logprobs.  That holds for a whole step only if
// every step between the verify kernels is also a per-row function: here each
// output row is computed from its own input row alone, with a fixed order for
// the one reduction (the sum of squares of an L2 normalisation).
//
// Column layout of the projection rows (a reading; the pages name the model,
// not its tensor layout):
//   y1: GDN q (Hk*dk) | GDN k (Hk*dk) | GDN v (Hv*dv) | ...
//   y2: attention q (Hq*d) | attention k (Hkv*d) | attention v (Hkv*d) |
//       decay logit (Hv) | beta logit (Hv) | ...
// q and k of the GDN are L2-normalised per head, u / sqrt(sum u^2 + 1e-6);
// decay a = 1 / (1 + e^alpha) (= exp(-softplus(alpha))), beta b = 1 / (1 + e^-beta).
#include "xv_common.h"
#include <math.h>

namespace {

constexpr int XV_CMP_THREADS = 256;
constexpr float XV_L2_EPS = 1e-6f;

// x[m][:] = table[tokens[m]][:]  (ids clamped to [0, V)); one workgroup per row.
__global__ __launch_bounds__(XV_CMP_THREADS)
void xv_embed_kernel(const uint16_t* __restrict__ table, const int32_t* __restrict__ tokens,
                     int V, int H, uint16_t* __restrict__ x)
{
    const int m = blockIdx.x;
    int id = tokens[m];
    id = id < 0 ? 0 : (id >= V ? V - 1 : id);
    const uint16_t* src = table + (size_t)id * H;
    uint16_t* dst = x + (size_t)m * H;
    for (int g = threadIdx.x; g < H / 8; g += XV_CMP_THREADS)
        xv_store16(dst + g * 8, xv_load16(src + g * 8));
}

// One workgroup per row.  LPH = dk / 8 lanes per head, each holding 8 values;
// the sum of squares runs over the lane's 8 values in order, then a butterfly
// over the head's lanes (each level adds two equal-order partials, so every
// lane ends with the same bits).
template <int DK>
__global__ __launch_bounds__(XV_CMP_THREADS)
void xv_split_kernel(const uint16_t* __restrict__ y1, const uint16_t* __restrict__ y2, int N1, int N2,
                     int Hk, int Hv, int dv, int Hq, int Hkv, int d,
                     uint16_t* __restrict__ q, uint16_t* __restrict__ k, uint16_t* __restrict__ v,
                     float* __restrict__ a, float* __restrict__ b,
                     uint16_t* __restrict__ qa, uint16_t* __restrict__ kn, uint16_t* __restrict__ vn)
{
    constexpr int LPH = DK / 8;
    constexpr int HPP = XV_CMP_THREADS / LPH;           // heads per pass
    const int m = blockIdx.x;
    const int tid = threadIdx.x;
    const uint16_t* r1 = y1 + (size_t)m * N1;
    const uint16_t* r2 = y2 + (size_t)m * N2;

    // GDN q and k heads: 2 Hk of them, q first
    const int lh = tid % LPH, hh = tid / LPH;
    for (int h0 = 0; h0 < 2 * Hk; h0 += HPP) {
        const int h = h0 + hh;
        if (h < 2 * Hk) {                               // whole heads (LPH divides 64)
            const xv_u32x4 raw = xv_load16(r1 + (size_t)h * DK + lh * 8);
            float u[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) { u[2 * e] = xv_bf16_lo(raw[e]); u[2 * e + 1] = xv_bf16_hi(raw[e]); }
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ss = ss + u[e] * u[e];
#pragma unroll
            for (int off = LPH / 2; off > 0; off >>= 1) ss = ss + __shfl_xor(ss, off, LPH);
            const float rn = 1.0f / sqrtf(ss + XV_L2_EPS);
            xv_u32x4 outv;
#pragma unroll
            for (int e = 0; e < 4; ++e) outv[e] = xv_pack_bf16x2(u[2 * e] * rn, u[2 * e + 1] * rn);
            uint16_t* dst = h < Hk ? q + ((size_t)m * Hk + h) * DK : k + ((size_t)m * Hk + (h - Hk)) * DK;
            xv_store16(dst + lh * 8, outv);
        }
    }

    // copies in 16-byte granules: GDN v from y1; attention q, k, v from y2
    const int gv = Hv * dv / 8, gq = Hq * d / 8, gk = Hkv * d / 8;
    const uint16_t* v_src = r1 + 2 * Hk * DK;
    for (int g = tid; g < gv + gq + 2 * gk; g += XV_CMP_THREADS) {
        if (g < gv) xv_store16(v + (size_t)m * Hv * dv + g * 8, xv_load16(v_src + g * 8));
        else if (g < gv + gq) xv_store16(qa + (size_t)m * Hq * d + (g - gv) * 8, xv_load16(r2 + (g - gv) * 8));
        else if (g < gv + gq + gk)
            xv_store16(kn + (size_t)m * Hkv * d + (g - gv - gq) * 8, xv_load16(r2 + Hq * d + (g - gv - gq) * 8));
        else
            xv_store16(vn + (size_t)m * Hkv * d + (g - gv - gq - gk) * 8,
                       xv_load16(r2 + Hq * d + Hkv * d + (g - gv - gq - gk) * 8));
    }

    // decay and beta per value head
    const uint16_t* gate = r2 + Hq * d + 2 * Hkv * d;
    for (int h = tid; h < Hv; h += XV_CMP_THREADS) {
        const float alpha = xv_bf16_to_f32(gate[h]);
        const float beta = xv_bf16_to_f32(gate[Hv + h]);
        a[(size_t)m * Hv + h] = 1.0f / (1.0f + expf(alpha));
        b[(size_t)m * Hv + h] = 1.0f / (1.0f + expf(-beta));
    }
}

}  // namespace

extern "C" int xv_embed_rows(const uint16_t* table, const int32_t* tokens, int M, int V, int H,
                             uint16_t* x, void* stream)
{
    XV_REQUIRE(M >= 0 && V >= 1 && H >= 8 && H % 8 == 0, XV_ERR_SHAPE);
    if (M == 0) return XV_OK;
    XV_REQUIRE(table && tokens && x, XV_ERR_NULL);
    XV_REQUIRE(xv_aligned16(table) && xv_aligned16(x) && xv_aligned(tokens, 4), XV_ERR_ALIGN);
    (void)hipGetLastError();
    hipLaunchKernelGGL(xv_embed_kernel, dim3(M), dim3(XV_CMP_THREADS), 0,
                       reinterpret_cast<hipStream_t>(stream), table, tokens, V, H, x);
    return xv_launch_status();
}

extern "C" int xv_split_projections(const uint16_t* y1, const uint16_t* y2, int M, int N1, int N2,
                                    int Hk, int Hv, int dk, int dv, int Hq, int Hkv, int d,
                                    uint16_t* q, uint16_t* k, uint16_t* v, float* a, float* b,
                                    uint16_t* q_attn, uint16_t* k_new, uint16_t* v_new, void* stream)
{
    XV_REQUIRE(M >= 0 && Hk >= 1 && Hv >= 1 && Hq >= 1 && Hkv >= 1, XV_ERR_SHAPE);
    XV_REQUIRE((dk == 64 || dk == 128) && dv >= 8 && dv % 8 == 0 && d >= 8 && d % 8 == 0, XV_ERR_SHAPE);
    XV_REQUIRE(N1 % 8 == 0 && N2 % 8 == 0, XV_ERR_SHAPE);
    XV_REQUIRE((long long)N1 >= 2LL * Hk * dk + (long long)Hv * dv, XV_ERR_SHAPE);
    XV_REQUIRE((long long)N2 >= (long long)Hq * d + 2LL * Hkv * d + 2LL * Hv, XV_ERR_SHAPE);
    if (M == 0) return XV_OK;
    XV_REQUIRE(y1 && y2 && q && k && v && a && b && q_attn && k_new && v_new, XV_ERR_NULL);
    XV_REQUIRE(xv_aligned16(y1) && xv_aligned16(y2) && xv_aligned16(q) && xv_aligned16(k) &&
               xv_aligned16(v) && xv_aligned16(q_attn) && xv_aligned16(k_new) && xv_aligned16(v_new) &&
               xv_aligned(a, 4) && xv_aligned(b, 4), XV_ERR_ALIGN);
    (void)hipGetLastError();
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (dk == 128)
        hipLaunchKernelGGL(xv_split_kernel<128>, dim3(M), dim3(XV_CMP_THREADS), 0, st, y1, y2, N1, N2,
                           Hk, Hv, dv, Hq, Hkv, d, q, k, v, a, b, q_attn, k_new, v_new);
    else
        hipLaunchKernelGGL(xv_split_kernel<64>, dim3(M), dim3(XV_CMP_THREADS), 0, st, y1, y2, N1, N2,
                           Hk, Hv, dv, Hq, Hkv, d, q, k, v, a, b, q_attn, k_new, v_new);
    return xv_launch_status();
}
