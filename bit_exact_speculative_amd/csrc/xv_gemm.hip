// xv_gemm.hip -- small-M bf16 projection GEMM, y = x W^T, streaming W once.
//
// The post's DeepGEMM paragraph: at small batch the decode GEMMs are bound by
// reading the weights, and routing them to one tile whose bits do not depend on
// M fixed both speed and exactness (recipe card, runtime env: the M <= 16 gate).
//
// Design (gfx950):
//  * A workgroup owns XV_GEMM_CB blocks of 16 output columns and all rows.
//    Its XV_GEMM_WAVES wavefronts split K into that many contiguous ranges of
//    32-wide k-steps; the split is a function of K alone.
//  * Each wave streams its W slice with 16-byte loads (one 64-byte run per
//    column per instruction) and feeds v_mfma_f32_16x16x32_bf16 with x as the
//    A operand (16 rows per tile, rows >= M zero) and W as the B operand.
//    Every row tile of the call is applied to the same W fragments, so W is
//    read from HBM once whatever M is.
//  * The per-wave fp32 partials are summed through LDS in wave order 0..7.
//  Row m's result is therefore the same chain of MFMAs over the same k-steps
//  followed by the same 8-term ordered sum, for any M and any position of m in
//  its tile: the M-independent reduction order the bit-exact route needs.
#include "xv_common.h"

namespace {

constexpr int XV_GEMM_CB = 2;       // 16-column blocks per workgroup
constexpr int XV_GEMM_WAVES = 8;    // K ranges per workgroup (one per wave)
constexpr int XV_GEMM_UNROLL = 4;   // k-steps in flight per wave
constexpr int XV_GEMM_MT_MAX = 8;   // 16-row tiles per pass over W

template <int MT>
__global__ __launch_bounds__(XV_GEMM_WAVES * 64)
void xv_gemm_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                    uint16_t* __restrict__ y, float* __restrict__ y32,
                    int M, int N, int K, int mt0)
{
    __shared__ float red[XV_GEMM_WAVES][XV_GEMM_CB][64][4];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int n0 = blockIdx.x * (XV_GEMM_CB * 16);
    const int KS = K >> 5;
    const int ks0 = (wave * KS) / XV_GEMM_WAVES;
    const int ks1 = ((wave + 1) * KS) / XV_GEMM_WAVES;

    bool cvalid[XV_GEMM_CB];
    const uint16_t* wp[XV_GEMM_CB];
#pragma unroll
    for (int cb = 0; cb < XV_GEMM_CB; ++cb) {
        cvalid[cb] = (n0 + cb * 16) < N;                     // uniform per wave
        const int col = cvalid[cb] ? n0 + cb * 16 + lr : 0;
        wp[cb] = w + (size_t)col * K + lg * 8;
    }
    bool rvalid[MT];
    const uint16_t* xp[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        const int row = (mt0 + t) * 16 + lr;
        rvalid[t] = row < M;
        xp[t] = x + (size_t)(rvalid[t] ? row : 0) * K + lg * 8;
    }

    xv_f32x4 acc[MT][XV_GEMM_CB];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int cb = 0; cb < XV_GEMM_CB; ++cb) acc[t][cb] = xv_f32x4{0.f, 0.f, 0.f, 0.f};

    const xv_u32x4 zero = {0u, 0u, 0u, 0u};
    for (int ks = ks0; ks < ks1; ks += XV_GEMM_UNROLL) {
        xv_u32x4 wf[XV_GEMM_UNROLL][XV_GEMM_CB];
        xv_u32x4 xf[XV_GEMM_UNROLL][MT];
#pragma unroll
        for (int u = 0; u < XV_GEMM_UNROLL; ++u) {
            if (ks + u < ks1) {
#pragma unroll
                for (int cb = 0; cb < XV_GEMM_CB; ++cb)
                    wf[u][cb] = cvalid[cb] ? xv_load16(wp[cb] + (size_t)(ks + u) * 32) : zero;
#pragma unroll
                for (int t = 0; t < MT; ++t)
                    xf[u][t] = rvalid[t] ? xv_load16(xp[t] + (size_t)(ks + u) * 32) : zero;
            }
        }
#pragma unroll
        for (int u = 0; u < XV_GEMM_UNROLL; ++u) {
            if (ks + u < ks1) {
#pragma unroll
                for (int t = 0; t < MT; ++t)
#pragma unroll
                    for (int cb = 0; cb < XV_GEMM_CB; ++cb)
                        acc[t][cb] = xv_mfma16x16x32(xf[u][t], wf[u][cb], acc[t][cb]);
            }
        }
    }

    // Ordered cross-wave sum: out = (((p0 + p1) + p2) + ... + p7).
    const int tid = threadIdx.x;
    const int rr = tid / (XV_GEMM_CB * 16);          // row within the tile, 0..15
    const int cc = tid % (XV_GEMM_CB * 16);          // column within the workgroup
    const int scb = cc >> 4;
    const int slane = (cc & 15) + 16 * (rr >> 2);
    const int si = rr & 3;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
#pragma unroll
        for (int cb = 0; cb < XV_GEMM_CB; ++cb)
            *reinterpret_cast<xv_f32x4*>(&red[wave][cb][lane][0]) = acc[t][cb];
        __syncthreads();
        float s = red[0][scb][slane][si];
#pragma unroll
        for (int wv = 1; wv < XV_GEMM_WAVES; ++wv) s = s + red[wv][scb][slane][si];
        const int row = (mt0 + t) * 16 + rr;
        const int col = n0 + cc;
        if (row < M && col < N) {
            y[(size_t)row * N + col] = xv_f32_to_bf16(s);
            if (y32) y32[(size_t)row * N + col] = s;
        }
        __syncthreads();
    }
}

template <int MT>
void xv_gemm_launch(const uint16_t* x, const uint16_t* w, uint16_t* y, float* y32,
                    int M, int N, int K, int mt0, hipStream_t st)
{
    const int cols = XV_GEMM_CB * 16;
    dim3 grid((N + cols - 1) / cols), block(XV_GEMM_WAVES * 64);
    hipLaunchKernelGGL(xv_gemm_kernel<MT>, grid, block, 0, st, x, w, y, y32, M, N, K, mt0);
}

}  // namespace

extern "C" int xv_gemm_small_m(const uint16_t* x, const uint16_t* w, uint16_t* y, float* y32,
                               int M, int N, int K, void* stream)
{
    XV_REQUIRE(M >= 0 && N >= 16 && N % 16 == 0 && K >= 32 && K % 32 == 0, XV_ERR_SHAPE);
    if (M == 0) return XV_OK;
    XV_REQUIRE(x && w && y, XV_ERR_NULL);
    XV_REQUIRE(xv_aligned16(x) && xv_aligned16(w) && xv_aligned(y, 2) && xv_aligned(y32, 4),
               XV_ERR_ALIGN);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    const int tiles = (M + 15) / 16;
    for (int mt0 = 0; mt0 < tiles; mt0 += XV_GEMM_MT_MAX) {
        const int mt = tiles - mt0 < XV_GEMM_MT_MAX ? tiles - mt0 : XV_GEMM_MT_MAX;
        switch (mt) {
            case 1: xv_gemm_launch<1>(x, w, y, y32, M, N, K, mt0, st); break;
            case 2: xv_gemm_launch<2>(x, w, y, y32, M, N, K, mt0, st); break;
            case 3: xv_gemm_launch<3>(x, w, y, y32, M, N, K, mt0, st); break;
            case 4: xv_gemm_launch<4>(x, w, y, y32, M, N, K, mt0, st); break;
            case 5: xv_gemm_launch<5>(x, w, y, y32, M, N, K, mt0, st); break;
            case 6: xv_gemm_launch<6>(x, w, y, y32, M, N, K, mt0, st); break;
            case 7: xv_gemm_launch<7>(x, w, y, y32, M, N, K, mt0, st); break;
            default: xv_gemm_launch<8>(x, w, y, y32, M, N, K, mt0, st); break;
        }
        int s = xv_launch_status();
        if (s != XV_OK) return s;
    }
    return XV_OK;
}
