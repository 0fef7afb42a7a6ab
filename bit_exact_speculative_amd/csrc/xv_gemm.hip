// xv_gemm.hip -- small-M bf16 projection GEMM, y = x W^T, streaming W once.
//
// The post's DeepGEMM paragraph: at small batch the decode GEMMs are bound by
// reading the weights, and routing them to one tile whose bits do not depend on
// M fixed both speed and exactness (recipe card, runtime env: the M <= 16 gate).
//
// Arithmetic (the same for every M, every row position and every launch shape):
//   K is cut into XV_GEMM_WAVES = 16 contiguous ranges of 32-wide k-steps (the
//   cut depends on K alone).  For each 16-column block, wave w runs one chain of
//   v_mfma_f32_16x16x32_bf16 over its range in ascending k-step order (x rows as
//   the A operand, W rows as the B operand), and the 16 range partials are
//   summed in wave order: ((p0 + p1) + p2) + ... + p15.  The result is rounded
//   to bf16 (nearest even) and optionally stored in fp32 as well.
//
// Work mapping (gfx950):
//  * Persistent workgroups of 16 waves, a few per CU; workgroup i walks the
//    column blocks i, i + grid, i + 2 grid, ...  All of its waves stream their
//    K range of the block's 16 W rows with 16-byte loads, double-buffered in
//    registers across column blocks so loads stay in flight through the
//    per-block reduction barriers.  Loads are straight-line code: addresses are
//    clamped into the buffers instead of branched around.
//  * The x fragments of a wave's K range are loaded into registers once per
//    row-tile group and reused for every column block (small M), or re-read
//    from L2 per k-step when they would not fit (many row tiles).  Where x comes
//    from does not change any arithmetic.
//  * Up to XV_GEMM_MT_MAX row tiles share one pass over W; rows >= M are zeroed
//    after their (clamped) load.
//  * With several row tiles and many column blocks, a K-loop variant instead
//    gives each wave whole output tiles: it runs the 16 range chains of a tile
//    one after the other and folds them in range order, the same operations.
#include "xv_common.h"
#include "xv_greedy_impl.h"
#include <hip/hip_ext.h>

namespace {

constexpr int XV_GEMM_WAVES = 16;   // K ranges per column block; fixes the sum order
constexpr int XV_GEMM_THREADS = XV_GEMM_WAVES * 64;
constexpr int XV_GEMM_MT_MAX = 5;   // 16-row tiles per pass over W (more would spill registers)

// Ordered sum of the 16 wave partials of one column block and the store.  Returns the
// last tile's sum of the calling thread's (row, column) for threads below 256 (row
// 16 (mt0 + MT - 1) + threadIdx.x / 16, column 16 blk + threadIdx.x % 16), 0 otherwise.
// With store false the caller stores that sum itself (MT = 1).
template <int MT>
__device__ __forceinline__ float xv_gemm_finish(float (&red)[XV_GEMM_WAVES][64][4], xv_f32x4 (&acc)[MT],
                                                int lane, int wave, int blk, int mt0, int M, int N,
                                                uint16_t* __restrict__ y, float* __restrict__ y32,
                                                bool store = true)
{
    float kept = 0.f;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        *reinterpret_cast<xv_f32x4*>(&red[wave][lane][0]) = acc[t];
        acc[t] = xv_f32x4{0.f, 0.f, 0.f, 0.f};
        __syncthreads();
        if (threadIdx.x < 256) {
            const int rr = threadIdx.x >> 4, cc = threadIdx.x & 15;
            const int slane = cc + 16 * (rr >> 2), si = rr & 3;
            float sum = red[0][slane][si];
#pragma unroll
            for (int wv = 1; wv < XV_GEMM_WAVES; ++wv) sum = sum + red[wv][slane][si];
            const int row = (mt0 + t) * 16 + rr;
            const int col = blk * 16 + cc;
            if (row < M && store) {
                y[(size_t)row * N + col] = xv_f32_to_bf16(sum);
                if (y32) y32[(size_t)row * N + col] = sum;
            }
            kept = sum;
        }
        __syncthreads();
    }
    return kept;
}

// x fragments in registers: a wave's range has at most KSW k-steps, streamed in
// two stages of U = KSW / 2 per column block (stage positions are compile-time).
template <int MT, int KSW>
__global__ __launch_bounds__(XV_GEMM_THREADS)
void xv_gemm_xreg_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                         uint16_t* __restrict__ y, float* __restrict__ y32,
                         int M, int N, int K, int mt0)
{
    constexpr int U = KSW / 2;
    __shared__ float red[XV_GEMM_WAVES][64][4];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int KS = K >> 5;
    const int ks0 = (wave * KS) / XV_GEMM_WAVES;
    const int nks = ((wave + 1) * KS) / XV_GEMM_WAVES - ks0;
    const int last = nks > 0 ? nks - 1 : 0;
    const int nblk = N >> 4;
    const int grid = gridDim.x;
    if ((int)blockIdx.x >= nblk) return;      // uniform over the workgroup
    const xv_u32x4 zero = {0u, 0u, 0u, 0u};

    xv_u32x4 xr[KSW][MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        const int row = (mt0 + t) * 16 + lr;
        const bool ok = row < M;
        const uint16_t* xp = x + (size_t)(ok ? row : M - 1) * K + (size_t)ks0 * 32 + lg * 8;
#pragma unroll
        for (int j = 0; j < KSW; ++j) {
            const xv_u32x4 v = xv_load16(xp + (size_t)(j < nks ? j : last) * 32);
            xr[j][t] = ok ? v : zero;
        }
    }
    const uint16_t* wl = w + (size_t)lr * K + (size_t)ks0 * 32 + lg * 8;
    auto load_half = [&](xv_u32x4 (&wf)[U], int blk, int half) {
        const uint16_t* wb = wl + (size_t)blk * 16 * K;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = half * U + u;
            wf[u] = xv_load16(wb + (size_t)(j < nks ? j : last) * 32);
        }
    };
    xv_f32x4 acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = xv_f32x4{0.f, 0.f, 0.f, 0.f};
    auto mma_half = [&](xv_u32x4 (&wf)[U], int half) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = half * U + u;
            if (j < nks) {
#pragma unroll
                for (int t = 0; t < MT; ++t) acc[t] = xv_mfma16x16x32(xr[j][t], wf[u], acc[t]);
            }
        }
    };

    xv_u32x4 w0[U], w1[U];
    int blk = blockIdx.x;
    load_half(w0, blk, 0);
    for (;;) {
        // prefetch the next block's first half; after the last block re-read the
        // half just loaded (a cache hit) so the loads stay straight-line code
        const bool more = blk + grid < nblk;
        load_half(w1, blk, 1);
        mma_half(w0, 0);
        load_half(w0, more ? blk + grid : blk, more ? 0 : 1);
        mma_half(w1, 1);
        xv_gemm_finish<MT>(red, acc, lane, wave, blk, mt0, M, N, y, y32);
        blk += grid;
        if (blk >= nblk) break;
    }
}

// Up to two GEMMs with the same M and K in one launch (the other variants take
// one): their column blocks form one list, problem 0's first.  With a shared x,
// workgroup i walks blocks i, i + grid, ... of the list (neighbouring workgroups
// read neighbouring blocks); with two different x, workgroup i takes the
// contiguous range [i nblk / grid, (i + 1) nblk / grid), so that few workgroups
// cross from problem 0 to problem 1 (a crossing reloads the x fragments, a stall
// in the stream).  Either way the chip stays balanced over the union, and per
// block the arithmetic is the single-GEMM kernel's.
struct XvGemmPair {
    const uint16_t* x[2];
    const uint16_t* w[2];
    uint16_t* y[2];
    float* y32[2];
    int N[2];
};

// LDS row pitch (bf16 elements) for rows of n bf16 values that 16 lanes read as MFMA
// fragments (lane lr: row lr, lane quarter lg: granule lg): the smallest pitch >= n of
// 4k + 2 16-byte granules.  The bank-conflict counter on gfx950 fits 16-byte accesses served
// for two lane octets at a time (0-7 with 16-23, 8-15 with 24-31, ...); such a pitch puts
// rows 0..7 at granules lg and lg + 1 on sixteen distinct 16-byte bank groups (measured: 128-
// and 144-byte rows conflict, 160-byte rows do not).
constexpr int xv_frag_pitch(int n) {
    const int g = (n + 7) / 8;
    return (g + (6 - g % 4) % 4) * 8;
}
static_assert(xv_frag_pitch(64) == 80 && xv_frag_pitch(320) == 336 && xv_frag_pitch(160) == 176 &&
              xv_frag_pitch(80) == 80, "pitch rule");

// Greedy acceptance fused into the head GEMM (one row tile, both halves of the head):
// the workgroup that formed column block i of both problems holds z = logits_a + logits_b
// of that block for every row (threads 0..255: row tid / 16, column tid % 16).  It forms
// the block's pair (m, s) and its argmax, stores them, and the last workgroup to arrive
// (a counter in the workspace) folds the pairs of every row in the greedy kernel's order,
// writes ids and logprobs, counts the accepted drafts and resets the counter.
//
// The pairs cross workgroups (and XCDs) through device-scope accesses only: stores and
// loads with device coherence (relaxed atomics at agent scope, which the compiler emits as
// plain loads and stores with that scope bit), the stores completed (vmcnt 0) before the
// workgroup's barrier and its counter increment, the loads issued only by the workgroup
// that saw the final count.  No L2 write-back or invalidation is needed for them (a fence
// at agent scope would do both, once per wave, for data that never enters a non-coherent
// cache line).
struct XvHeadPair {
    uint64_t ms;                // m (low word) and s (high word), fp32 bits
    uint32_t n;                 // the block's argmax column
    uint32_t pad;
};
static_assert(sizeof(XvHeadPair) == 16, "pair layout");

struct XvHeadGreedy {
    const int32_t* draft;       // int32 [B][T]
    int32_t* ids;               // int32 [B][T]
    int32_t* n_keep;            // int32 [B]
    float* lp;                  // fp32 [B][T] or null
    int32_t* kv_len;            // int32 [B] or null
    XvHeadPair* pairs;          // [B T][N / 16]
    int* counter;               // 0 on entry, 0 on exit
    int B, T;
};

__device__ __forceinline__ void xv_pair_store(XvHeadPair* p, float m, float s, int n) {
    const uint64_t ms = (uint64_t)__float_as_uint(m) | ((uint64_t)__float_as_uint(s) << 32);
    __hip_atomic_store(&p->ms, ms, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&p->n, (uint32_t)n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void xv_pair_load(const XvHeadPair* p, float& m, float& s, int& n) {
    const uint64_t ms = __hip_atomic_load(&p->ms, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    n = (int)__hip_atomic_load(&p->n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    m = __uint_as_float((uint32_t)ms);
    s = __uint_as_float((uint32_t)(ms >> 32));
}

// dr: row tid's draft (tid < B T) and kv: kv_len[tid] (tid < B), loaded at the kernel's start
// (nothing else writes them during the call); store_b: stores the second
// block's outputs (after the pairs, so that the wait for the pair stores does not wait for them).
template <typename StoreFn>
__device__ __forceinline__ void xv_head_greedy_tail(const XvHeadGreedy& g, float za, float zb, int blk,
                                                    int M, int N, int dr, int kv, StoreFn store_b)
{
    __shared__ int s_last;
    __shared__ int s_ids[XV_TMAX], s_draft[XV_TMAX];
    __shared__ float s_cm[XV_TMAX][256], s_cs[XV_TMAX][256], s_bv[XV_TMAX][256];   // last workgroup: chains
    __shared__ int s_bn[XV_TMAX][256];
    const int tid = threadIdx.x, lane = tid & 63;
    const int nb = N >> 4;
    if (tid < 256) {                              // waves 0..3, uniform: row tid / 16, column tid % 16
        const int rr = tid >> 4, cc = tid & 15;
        const float z = za + zb;
        float bm = z, best = z;
        int bn = blk * 16 + cc;
        // the block's maximum and argmax (exact in any order), then the sum of e^(z - m) in the
        // butterfly order c ^ 8, ^ 4, ^ 2, ^ 1 (each lane adds its partner's value to its own)
        auto mx = [&](float ov, int on) {
            bm = fmaxf(bm, ov);
            if (xv_better(ov, on, best, bn)) { best = ov; bn = on; }
        };
        mx(xv_dpp<XV_DPP_ROR8>(best), xv_dpp<XV_DPP_ROR8>(bn));
        mx(xv_dpp<XV_DPP_ROR12>(best), xv_dpp<XV_DPP_ROR12>(bn));
        mx(xv_dpp<XV_DPP_XOR2>(best), xv_dpp<XV_DPP_XOR2>(bn));
        mx(xv_dpp<XV_DPP_XOR1>(best), xv_dpp<XV_DPP_XOR1>(bn));
        float e = __builtin_amdgcn_exp2f((z - bm) * XV_LOG2E);
        e = e + xv_dpp<XV_DPP_ROR8>(e);
        e = e + xv_dpp<XV_DPP_ROR12>(e);
        e = e + xv_dpp<XV_DPP_XOR2>(e);
        e = e + xv_dpp<XV_DPP_XOR1>(e);
        if (cc == 0 && rr < M) xv_pair_store(g.pairs + (size_t)rr * nb + blk, bm, e, bn);
        __builtin_amdgcn_s_waitcnt(0x0F70);       // vmcnt(0): the pair stores have completed
        store_b();
    }
    if (tid < M) s_draft[tid] = dr;
    __syncthreads();
    if (tid == 0) s_last = atomicAdd(g.counter, 1) == (int)gridDim.x - 1;
    __syncthreads();
    if (!s_last) return;                          // uniform over the workgroup
    // The last workgroup.  Chain c (c < 256) of row r folds blocks c, c + 256, ... left to right
    // from the empty pair; thread tid forms chains tid + 1024 u (row task / 256, chain task % 256),
    // so that each wave's loads read 64 consecutive pairs, all of a thread's loads issued together.
    const int nu = (M * 256 + XV_GEMM_THREADS - 1) / XV_GEMM_THREADS;   // uniform
    {
        float cm[4], cs[4], bv[4];
        int bi[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {             // straight-line: tasks past the rows read pair 0
            const int task = tid + u * XV_GEMM_THREADS, r = task >> 8, c = task & 255;
            const size_t at = u < nu && r < M ? (size_t)r * nb + (c < nb ? c : nb - 1) : 0;
            xv_pair_load(g.pairs + at, bv[u], cs[u], bi[u]);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int task = tid + u * XV_GEMM_THREADS, r = task >> 8, c = task & 255;
            if (u >= nu || r >= M) continue;      // uniform per wave
            const bool ok = c < nb;
            const float m1 = bv[u], s1 = cs[u];
            cm[u] = -INFINITY;
            cs[u] = 0.f;
            xv_lse_add(cm[u], cs[u], ok ? m1 : -INFINITY, ok ? s1 : 0.f);
            bv[u] = ok ? bv[u] : -INFINITY;
            bi[u] = ok ? bi[u] : N;
            for (int b = c + 256; b < nb; b += 256) {
                float m2, s2;
                int n2;
                xv_pair_load(g.pairs + (size_t)r * nb + b, m2, s2, n2);
                xv_lse_add(cm[u], cs[u], m2, s2);
                if (xv_better(m2, n2, bv[u], bi[u])) { bv[u] = m2; bi[u] = n2; }
            }
            s_cm[r][c] = cm[u];
            s_cs[r][c] = cs[u];
            s_bv[r][c] = bv[u];
            s_bn[r][c] = bi[u];
        }
    }
    __syncthreads();
    // Thread t < 32 M: row r = t / 32, group q = (t / 8) % 4 of 64 chains, chains 64 q + 8 k + j
    // (k = t % 8, j = 0..7).  The group's tree (node c at distance h becomes lse(node c,
    // node c + h)) runs over j in registers for h = 1, 2, 4 and across the group's 8 lanes for
    // h = 8, 16, 32, where each lane combines its node with the partner's (the two lanes of a
    // pair form the same bits, fp32 addition being commutative); the four groups then fold
    // left to right.  The argmax is exact in any order.
    const int r = tid >> 5, q = (tid >> 3) & 3, k = tid & 7;
    if (r < M) {                                  // whole 8-lane groups
        float cm[8], cs[8], bv[8];
        int bi[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int c = 64 * q + 8 * k + j;
            cm[j] = s_cm[r][c];
            cs[j] = s_cs[r][c];
            bv[j] = s_bv[r][c];
            bi[j] = s_bn[r][c];
        }
#pragma unroll
        for (int h = 1; h < 8; h *= 2)
#pragma unroll
            for (int j = 0; j < 8; j += 2 * h) {
                xv_lse_add(cm[j], cs[j], cm[j + h], cs[j + h]);
                if (xv_better(bv[j + h], bi[j + h], bv[j], bi[j])) { bv[j] = bv[j + h]; bi[j] = bi[j + h]; }
            }
        float m = cm[0], sm = cs[0], best = bv[0];
        int bn = bi[0];
        auto level = [&](float m2, float s2, float ov, int on) {
            xv_lse_add(m, sm, m2, s2);
            if (xv_better(ov, on, best, bn)) { best = ov; bn = on; }
        };
        level(xv_dpp<XV_DPP_XOR1>(m), xv_dpp<XV_DPP_XOR1>(sm), xv_dpp<XV_DPP_XOR1>(best), xv_dpp<XV_DPP_XOR1>(bn));
        level(xv_dpp<XV_DPP_XOR2>(m), xv_dpp<XV_DPP_XOR2>(sm), xv_dpp<XV_DPP_XOR2>(best), xv_dpp<XV_DPP_XOR2>(bn));
        level(xv_dpp<XV_DPP_HALF_MIRROR>(m), xv_dpp<XV_DPP_HALF_MIRROR>(sm), xv_dpp<XV_DPP_HALF_MIRROR>(best),
              xv_dpp<XV_DPP_HALF_MIRROR>(bn));
        // groups 1..3 of the row (lanes +8, +16, +24 of its 32), folded after group 0
        const int row0 = lane & ~31;
        float gm[3], gs[3], gv[3];
        int gn[3];
#pragma unroll
        for (int u = 0; u < 3; ++u) {
            const int src = row0 + 8 * (u + 1);
            gm[u] = __shfl(m, src);
            gs[u] = __shfl(sm, src);
            gv[u] = __shfl(best, src);
            gn[u] = __shfl(bn, src);
        }
#pragma unroll
        for (int u = 0; u < 3; ++u) {
            xv_lse_add(m, sm, gm[u], gs[u]);
            if (xv_better(gv[u], gn[u], best, bn)) { best = gv[u]; bn = gn[u]; }
        }
        if ((tid & 31) == 0) {
            const int id = bn < N ? bn : 0;
            g.ids[r] = id;
            if (g.lp) g.lp[r] = xv_neg_log(sm);
            s_ids[r] = id;
        }
    }
    __syncthreads();
    if (tid < g.B) {
        const int acc = xv_accepted(g.T, [&](int t) { return s_draft[tid * g.T + t]; },
                                    [&](int t) { return s_ids[tid * g.T + t]; });
        g.n_keep[tid] = acc + 1;
        if (g.kv_len) g.kv_len[tid] = kv + acc + 1;
    }
    if (tid == 0) __hip_atomic_store(g.counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// W staged through LDS: the workgroup streams each column block's 16 rows with
// 1 KB contiguous wave loads (each 16-byte granule of a stage is one thread's
// load) into a padded LDS stage; each wave then reads the MFMA B fragments of its
// own K range from LDS.  A column block is NS stages of SL k-steps (stage s holds
// the ranges of waves s*16/NS .. (s+1)*16/NS - 1); even and odd stages have a
// register buffer each, so while one stage is consumed the next two are in
// flight.  x fragments of the wave's range live in registers.  Same K split,
// MFMA chains and ordered sum as the other variants.
// Requires K = NS * SL * 32 and SL * NS = 16 * KSW (the 16 ranges split evenly).
// GR: the head with its greedy acceptance; the grid is N / 16 workgroups of two problems
// with N columns each and contig = 0, so that workgroup i computes column block i of
// problem 0 and then of problem 1 (each wave reloads its x fragments right after its
// MFMAs of the first block), then runs xv_head_greedy_tail.
template <int KSW, int SL, int NS, bool GR>
__global__ __launch_bounds__(XV_GEMM_THREADS)
void xv_gemm_wlds_kernel(XvGemmPair pp, int M, int K, int mt0, int contig, XvHeadGreedy hg)
{
    static_assert(NS % 2 == 0 && SL * NS == XV_GEMM_WAVES * KSW, "stages must split the ranges evenly");
    static_assert(XV_GEMM_WAVES % NS == 0, "each stage must hold whole K ranges of the same number of waves");
    constexpr int WPS = XV_GEMM_WAVES / NS;         // waves whose ranges a stage holds
    constexpr int PITCH = xv_frag_pitch(SL * 32);   // LDS row pitch (bf16)
    constexpr int PER_ROW = SL * 4;                 // 16-byte granules per row per stage
    constexpr int TOTAL = 16 * PER_ROW;
    constexpr int GPT = (TOTAL + XV_GEMM_THREADS - 1) / XV_GEMM_THREADS;
    __shared__ float red[XV_GEMM_WAVES][64][4];
    __shared__ __attribute__((aligned(16))) uint16_t stage[16 * PITCH];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int ks0 = wave * KSW;
    const int my_stage = wave / WPS;
    const int nb0 = pp.N[0] >> 4;
    const int nblk = nb0 + (pp.N[1] >> 4);
    const int grid = gridDim.x;
    // this workgroup's blocks: b0, b0 + step, ... below bend
    const int b0 = contig ? (int)(((long long)blockIdx.x * nblk) / grid) : (int)blockIdx.x;
    const int bend = contig ? (int)(((long long)(blockIdx.x + 1) * nblk) / grid) : nblk;
    const int bstep = contig ? 1 : grid;
    if (b0 >= bend) return;                         // uniform over the workgroup
    const xv_u32x4 zero = {0u, 0u, 0u, 0u};

    xv_u32x4 xr[KSW];
    auto load_x = [&](const uint16_t* __restrict__ x) {
        const int row = mt0 * 16 + lr;
        const bool ok = row < M;
        const uint16_t* xp = x + (size_t)(ok ? row : M - 1) * K + (size_t)ks0 * 32 + lg * 8;
#pragma unroll
        for (int j = 0; j < KSW; ++j) xr[j] = xv_load16(xp + j * 32);
        // rows >= M: zeroed, or under GR left as copies of row M - 1 (MFMA rows are
        // independent and those rows are never stored), so that the reload is not waited for here
        if (!GR) {
#pragma unroll
            for (int j = 0; j < KSW; ++j) xr[j] = ok ? xr[j] : zero;
        }
    };
    int cur = b0 >= nb0 ? 1 : 0;
    load_x(pp.x[cur]);
    int dr = 0, kv = 0;                             // GR: row tid's draft, request tid's cache length
    if (GR && tid < M) dr = hg.draft[tid];
    if (GR && hg.kv_len && tid < hg.B) kv = hg.kv_len[tid];

    // this thread's granules: (row, 16-byte column) of a stage, the same for every stage
    int goff[GPT], loff[GPT];
#pragma unroll
    for (int i = 0; i < GPT; ++i) {
        int g = tid + i * XV_GEMM_THREADS;
        g = g < TOTAL ? g : TOTAL - 1;
        const int r = g / PER_ROW, c = g % PER_ROW;
        goff[i] = r * K + c * 8;
        loff[i] = r * PITCH + c * 8;
    }
    auto load_stage = [&](xv_u32x4 (&gr)[GPT], int blk, int st) {
        const uint16_t* base = (blk < nb0 ? pp.w[0] + (size_t)blk * 16 * K
                                          : pp.w[1] + (size_t)(blk - nb0) * 16 * K) + st * (SL * 32);
#pragma unroll
        for (int i = 0; i < GPT; ++i)
            gr[i] = xv_load16_nt(base + goff[i]);
    };
    auto store_stage = [&](const xv_u32x4 (&gr)[GPT]) {
#pragma unroll
        for (int i = 0; i < GPT; ++i)
            if (TOTAL % XV_GEMM_THREADS == 0 || tid + i * XV_GEMM_THREADS < TOTAL)
                *reinterpret_cast<xv_u32x4*>(stage + loff[i]) = gr[i];
    };
    xv_f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float za = 0.f, zb = 0.f;                       // GR: this thread's sums of problems 0 and 1

    xv_u32x4 g0[GPT], g1[GPT];
    int blk = b0;
    load_stage(g0, blk, 0);
    load_stage(g1, blk, 1);
    for (;;) {
        const int nb = blk + bstep;
        const bool more = nb < bend;
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            xv_u32x4 (&gr)[GPT] = (st & 1) ? g1 : g0;
            __syncthreads();                        // LDS stage free
            store_stage(gr);
            // this buffer's next stage: st + 2 of this block, else of the next block;
            // past the end re-read the stage just stored (a cache hit)
            if (st + 2 < NS) load_stage(gr, blk, st + 2);
            else load_stage(gr, more ? nb : blk, more ? st + 2 - NS : st);
            __syncthreads();
            if (my_stage == st) {                   // uniform per wave
                const uint16_t* bp = stage + lr * PITCH + (ks0 - st * SL) * 32 + lg * 8;
#pragma unroll
                for (int j = 0; j < KSW; ++j)
                    acc = xv_mfma16x16x32(xr[j], *reinterpret_cast<const xv_u32x4*>(bp + j * 32), acc);
                // GR: this wave's x fragments of problem 1, in flight through the block's other stages
                if (GR && more && nb >= nb0 && cur == 0) load_x(pp.x[1]);
            }
        }
        const bool cross = more && nb >= nb0 && cur == 0;   // uniform: next block in problem 1
        xv_f32x4 accs[1] = {acc};
        const float z = xv_gemm_finish<1>(red, accs, lane, wave, blk - cur * nb0, mt0, M, pp.N[cur], pp.y[cur],
                                          pp.y32[cur], !(GR && cur == 1));
        if (cur == 0) za = z;
        else zb = z;
        acc = xv_f32x4{0.f, 0.f, 0.f, 0.f};
        if (!more) break;
        blk = nb;
        if (cross) {
            cur = 1;
            if (!GR && pp.x[1] != pp.x[0]) load_x(pp.x[1]);     // uniform; a shared x is kept
        }
    }
    if constexpr (GR) {
        xv_head_greedy_tail(hg, za, zb, b0, M, pp.N[0], dr, kv, [&] {
            const int row = tid >> 4, col = b0 * 16 + (tid & 15), N1 = pp.N[1];
            if (row < M) {
                pp.y[1][(size_t)row * N1 + col] = xv_f32_to_bf16(zb);
                if (pp.y32[1]) pp.y32[1][(size_t)row * N1 + col] = zb;
            }
        });
    }
}

// Many row tiles (M > 16): there are enough 16 x 16 output tiles to fill the
// chip without splitting K over waves.  A workgroup of 4 waves owns MT row tiles
// x NB column blocks (wave v takes column block v % NB and every (4/NB)-th row
// tile from v / NB) and walks K in ascending k-steps, W and x staged through
// double-buffered LDS (KC k-steps per stage, the next stage prefetched in
// registers).  For each of its tiles a wave runs the 16 range chains one after
// the other: a chain restarts from zero at its range's first k-step, and a
// finished range is folded into a running sum in range order (sum = p0, then
// sum + p1, ...).  Those are exactly the operations of the K-split kernels, so
// every output bit is the same as theirs.
constexpr int XV_KL_WAVES = 4;
constexpr int XV_KL_THREADS = XV_KL_WAVES * 64;

template <int MT, int NB, int KC>
__global__ __launch_bounds__(XV_KL_THREADS)
void xv_gemm_kloop_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                          uint16_t* __restrict__ y, float* __restrict__ y32,
                          int M, int N, int K, int mt0)
{
    constexpr int NTH = XV_KL_THREADS;
    constexpr int RW = XV_KL_WAVES / NB;        // waves sharing a column block
    constexpr int MTW = (MT + RW - 1) / RW;     // row tiles per wave (the last may be past MT)
    // LDS row pitch (bf16): rows fall 4 banks apart (the fragment-read pitch would take the
    // widest instance past half the CU's LDS)
    constexpr int PITCH = KC * 32 + 8;
    constexpr int WROWS = NB * 16;
    constexpr int XROWS = MT * 16;
    constexpr int GR = KC * 4;                  // 16-byte granules per row per stage
    constexpr int WPT = (WROWS * GR + NTH - 1) / NTH;
    constexpr int XPT = (XROWS * GR + NTH - 1) / NTH;
    static_assert(XV_KL_WAVES % NB == 0, "column blocks must divide the waves");
    __shared__ __attribute__((aligned(16))) uint16_t sw[2][WROWS * PITCH];
    __shared__ __attribute__((aligned(16))) uint16_t sx[2][XROWS * PITCH];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int wcb = wave % NB;                  // the wave's column block within the workgroup
    const int wt0 = wave / NB;                  // its row tiles: wt0, wt0 + RW, ...
    const int KS = K >> 5;
    const int nst = (KS + KC - 1) / KC;
    const int col0 = blockIdx.x * WROWS;        // first W row (output column) of the workgroup
    const xv_u32x4 zero = {0u, 0u, 0u, 0u};

    // this thread's granules of a stage: (row, 16-byte column); addresses clamped into the buffers
    const uint16_t* wsrc[WPT];
    int wl[WPT];
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
        int g = tid + i * NTH;
        g = g < WROWS * GR ? g : WROWS * GR - 1;
        const int r = g / GR, c = g % GR;
        const int wr = col0 + r < N ? col0 + r : N - 1;
        wsrc[i] = w + (size_t)wr * K + c * 8;
        wl[i] = r * PITCH + c * 8;
    }
    const uint16_t* xsrc[XPT];
    int xl[XPT];
    bool xok[XPT];
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        int g = tid + i * NTH;
        g = g < XROWS * GR ? g : XROWS * GR - 1;
        const int r = g / GR, c = g % GR;
        const int xr = mt0 * 16 + r;
        xok[i] = xr < M;
        xsrc[i] = x + (size_t)(xr < M ? xr : M - 1) * K + c * 8;
        xl[i] = r * PITCH + c * 8;
    }
    xv_u32x4 wreg[WPT], xreg[XPT];
    auto load = [&](int s) {                    // stage s; columns past K re-read the row's last granule
#pragma unroll
        for (int i = 0; i < WPT; ++i) {
            const int c8 = ((tid + i * NTH) % GR) * 8;
            wreg[i] = xv_load16(wsrc[i] + (s * (KC * 32) + c8 < K ? s * (KC * 32) : K - 8 - c8));
        }
#pragma unroll
        for (int i = 0; i < XPT; ++i) {
            const int c8 = ((tid + i * NTH) % GR) * 8;
            xreg[i] = xv_load16(xsrc[i] + (s * (KC * 32) + c8 < K ? s * (KC * 32) : K - 8 - c8));
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < WPT; ++i)
            if ((WROWS * GR) % NTH == 0 || tid + i * NTH < WROWS * GR)
                *reinterpret_cast<xv_u32x4*>(&sw[buf][wl[i]]) = wreg[i];
#pragma unroll
        for (int i = 0; i < XPT; ++i)
            if ((XROWS * GR) % NTH == 0 || tid + i * NTH < XROWS * GR)
                *reinterpret_cast<xv_u32x4*>(&sx[buf][xl[i]]) = xok[i] ? xreg[i] : zero;
    };

    xv_f32x4 acc[MTW], sum[MTW];
#pragma unroll
    for (int t = 0; t < MTW; ++t) { acc[t] = xv_f32x4{0.f, 0.f, 0.f, 0.f}; sum[t] = acc[t]; }
    int r = 0;                                  // the range whose chains are running
    auto fold = [&]() {                         // range r is complete
#pragma unroll
        for (int t = 0; t < MTW; ++t) {
            sum[t] = r == 0 ? acc[t] : sum[t] + acc[t];
            acc[t] = xv_f32x4{0.f, 0.f, 0.f, 0.f};
        }
        ++r;
    };

    load(0);
    store(0);
    load(nst > 1 ? 1 : 0);
    __syncthreads();
    for (int s = 0; s < nst; ++s) {
        const int buf = s & 1;
#pragma unroll
        for (int j = 0; j < KC; ++j) {
            const int ks = s * KC + j;
            while (r < XV_GEMM_WAVES && ((r + 1) * KS) / XV_GEMM_WAVES <= ks) fold();   // uniform
            if (ks < KS) {
                const xv_u32x4 bf = *reinterpret_cast<const xv_u32x4*>(&sw[buf][(wcb * 16 + lr) * PITCH + j * 32 + lg * 8]);
#pragma unroll
                for (int t = 0; t < MTW; ++t) {
                    const int tt = wt0 + t * RW < MT ? wt0 + t * RW : MT - 1;   // past MT: computed, not stored
                    acc[t] = xv_mfma16x16x32(*reinterpret_cast<const xv_u32x4*>(&sx[buf][(tt * 16 + lr) * PITCH + j * 32 + lg * 8]),
                                             bf, acc[t]);
                }
            }
        }
        if (s + 1 < nst) {                      // stage s+1 into the other buffer, stage s+2 in flight
            store(buf ^ 1);
            load(s + 2 < nst ? s + 2 : s + 1);
        }
        __syncthreads();
    }
    while (r < XV_GEMM_WAVES) fold();

    const int cb = blockIdx.x * NB + wcb;
    if (cb >= (N >> 4)) return;
#pragma unroll
    for (int t = 0; t < MTW; ++t) {
        const int tt = wt0 + t * RW;
        if (tt >= MT) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = (mt0 + tt) * 16 + 4 * lg + i;
            if (row < M) {
                const size_t o = (size_t)row * N + cb * 16 + lr;
                y[o] = xv_f32_to_bf16(sum[t][i]);
                if (y32) y32[o] = sum[t][i];
            }
        }
    }
}

// Many rows (prefill): 128 x 128 output tiles, 4 waves of 64 x 64 (4 x 4 MFMA
// tiles each), K walked in ascending k-steps with x and W staged through
// double-buffered LDS, KC k-steps per stage, the next stage's loads in flight in
// registers.  For each of its output tiles a wave runs the 16 range chains one
// after the other and folds each finished range into the running sum in range
// order, the operations of the other variants: a row's bits are its bits at any M.
// Workgroup i takes column tile i / mb and row tile i % mb (the row tiles of one
// column tile run together, so its W rows are read from HBM about once).
constexpr int XV_BIG_BM = 128, XV_BIG_BN = 128, XV_BIG_KC = 2;
constexpr int XV_BIG_MIN_M = 256;   // rows from which the tiled kernel runs
constexpr int XV_BIG_THREADS = 256;

__global__ __launch_bounds__(XV_BIG_THREADS, 2)
void xv_gemm_big_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                        uint16_t* __restrict__ y, float* __restrict__ y32, int M, int N, int K, int mb)
{
    constexpr int NTH = XV_BIG_THREADS;
    constexpr int KC = XV_BIG_KC;
    // LDS row pitch (bf16): 160-byte rows; two workgroups' buffers then fill the CU's 160 KB
    constexpr int PITCH = xv_frag_pitch(KC * 32);
    constexpr int GR = KC * 4;                  // 16-byte granules per row per stage
    constexpr int XG = XV_BIG_BM * GR / NTH;    // x granules per thread per stage
    constexpr int WG = XV_BIG_BN * GR / NTH;
    static_assert(XV_BIG_BM * GR % NTH == 0 && XV_BIG_BN * GR % NTH == 0, "granules must split evenly");
    __shared__ __attribute__((aligned(16))) uint16_t sx[2][XV_BIG_BM * PITCH];
    __shared__ __attribute__((aligned(16))) uint16_t sw[2][XV_BIG_BN * PITCH];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int wm = wave & 1, wn = wave >> 1;    // the wave's 64 x 64 quarter
    const int m0 = ((int)blockIdx.x % mb) * XV_BIG_BM;
    const int n0 = ((int)blockIdx.x / mb) * XV_BIG_BN;
    const int KS = K >> 5;
    const int nst = (KS + KC - 1) / KC;

    // this thread's granules of a stage: rows tid / GR + i (NTH / GR), column tid % GR, the
    // same for every stage; rows past the buffers re-read the last one
    constexpr int RSTEP = NTH / GR;
    const int r0 = tid / GR, c8 = (tid % GR) * 8;
    const int l0 = r0 * PITCH + c8;
    xv_u32x4 xreg[XG], wreg[WG];
    auto load = [&](int s) {                    // stage s; columns past K re-read the row's last granule
        const int k0 = s * (KC * 32);
        const int kc = k0 + c8 < K ? k0 + c8 : K - 8;
#pragma unroll
        for (int i = 0; i < XG; ++i) {
            const int row = m0 + r0 + i * RSTEP < M ? m0 + r0 + i * RSTEP : M - 1;
            xreg[i] = xv_load16(x + (size_t)row * K + kc);
        }
#pragma unroll
        for (int i = 0; i < WG; ++i) {
            const int col = n0 + r0 + i * RSTEP < N ? n0 + r0 + i * RSTEP : N - 1;
            wreg[i] = xv_load16(w + (size_t)col * K + kc);
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < XG; ++i) *reinterpret_cast<xv_u32x4*>(&sx[buf][l0 + i * RSTEP * PITCH]) = xreg[i];
#pragma unroll
        for (int i = 0; i < WG; ++i) *reinterpret_cast<xv_u32x4*>(&sw[buf][l0 + i * RSTEP * PITCH]) = wreg[i];
    };

    xv_f32x4 acc[4][4], sum[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) { acc[i][j] = xv_f32x4{0.f, 0.f, 0.f, 0.f}; sum[i][j] = acc[i][j]; }
    int r = 0;                                  // the range whose chains are running
    auto fold = [&]() {                         // range r is complete
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                sum[i][j] = r == 0 ? acc[i][j] : sum[i][j] + acc[i][j];
                acc[i][j] = xv_f32x4{0.f, 0.f, 0.f, 0.f};
            }
        ++r;
    };

    load(0);
    store(0);
    load(nst > 1 ? 1 : 0);
    __syncthreads();
    for (int s = 0; s < nst; ++s) {
        const int buf = s & 1;
#pragma unroll
        for (int jj = 0; jj < KC; ++jj) {
            const int ks = s * KC + jj;
            while (r < XV_GEMM_WAVES && ((r + 1) * KS) / XV_GEMM_WAVES <= ks) fold();   // uniform
            if (ks < KS) {
                xv_u32x4 af[4], bf[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    af[i] = *reinterpret_cast<const xv_u32x4*>(&sx[buf][(wm * 64 + i * 16 + lr) * PITCH + jj * 32 + lg * 8]);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    bf[j] = *reinterpret_cast<const xv_u32x4*>(&sw[buf][(wn * 64 + j * 16 + lr) * PITCH + jj * 32 + lg * 8]);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[i][j] = xv_mfma16x16x32(af[i], bf[j], acc[i][j]);
            }
        }
        if (s + 1 < nst) {                      // stage s+1 into the other buffer, stage s+2 in flight
            store(buf ^ 1);
            load(s + 2 < nst ? s + 2 : s + 1);
        }
        __syncthreads();
    }
    while (r < XV_GEMM_WAVES) fold();

#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = n0 + wn * 64 + j * 16 + lr;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = m0 + wm * 64 + i * 16 + 4 * lg + e;
                if (row < M && col < N) {
                    const size_t o = (size_t)row * N + col;
                    y[o] = xv_f32_to_bf16(sum[i][j][e]);
                    if (y32) y32[o] = sum[i][j][e];
                }
            }
        }
}

// 2 to 5 row tiles (a batch of requests' verify rows) and K = 5120 or 6144: the 16 ranges
// have KSW = K / 512 k-steps each.  A workgroup (16 waves) owns NBW column blocks of one
// problem of the pair and walks K in parts of KSP k-steps (a range may end inside a part).  A
// part's x slice (all row tiles) and W slice (the NBW blocks) are staged by every thread
// into one of two LDS buffers while the other buffer is consumed (one barrier per part),
// with the loads of the next two parts in flight in two register buffers.  Compute wave
// (t, g) owns row tile t and column blocks g BG .. g BG + BG - 1: per k-step it reads the
// A fragment once and one B fragment per block.  Per tile one chain per range from zero,
// folded into the running sum in range order: the bits of every other variant.  Each W
// byte is read once; x is re-read from L2 by every workgroup (it is small).
template <int MT, int KSP, int NBW>
__global__ __launch_bounds__(XV_GEMM_THREADS)
void xv_gemm_mt_kernel(XvGemmPair pp, int M, int K, int nwg0)
{
    constexpr int NT = XV_GEMM_THREADS;
    constexpr int XR = MT * 16, WR = NBW * 16;  // rows of a part: x, W
    constexpr int GR = KSP * 4;                 // 16-byte granules per row of a part
    constexpr int PITCH = xv_frag_pitch(KSP * 32);  // LDS row pitch (bf16)
    constexpr int GPT = ((XR + WR) * GR + NT - 1) / NT;
    constexpr int BG = NBW < 4 ? NBW : 4;       // column blocks per compute wave
    constexpr int NBG = (NBW + BG - 1) / BG;
    static_assert(MT * NBG <= XV_GEMM_WAVES, "one compute wave per (row tile, block group)");
    constexpr int SPARE = (XR + WR) * PITCH;    // a 16-byte slot past the rows: stores of unused granules
    __shared__ __attribute__((aligned(16))) uint16_t sm[2][SPARE + 8];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int cur = (int)blockIdx.x < nwg0 ? 0 : 1;
    const int blk0 = ((int)blockIdx.x - cur * nwg0) * NBW;     // first column block, local to the problem
    const uint16_t* __restrict__ x = pp.x[cur];
    const uint16_t* __restrict__ w = pp.w[cur];
    const int N = pp.N[cur];
    const int NPARTS = (K >> 5) / KSP;
    const int KSW = (K >> 5) / XV_GEMM_WAVES;   // k-steps per K range (a range may end inside a part)

    // this thread's granules of a part: g = tid + i NT over the x rows, then the W rows;
    // rows past the buffers re-read the last one (their outputs are not stored).  Granules
    // past the part load granule 0 and store it into the spare slot, so that no load or store
    // is conditional: under a divergent branch the compiler would wait for every load in flight.
    const uint16_t* src[GPT];
    int dst[GPT];
    bool wsrc[GPT];
#pragma unroll
    for (int i = 0; i < GPT; ++i) {
        int g = tid + i * NT;
        const bool live = g < (XR + WR) * GR;
        g = live ? g : 0;
        const int r = g / GR, c = g % GR;
        wsrc[i] = r >= XR;
        if (r < XR) {
            src[i] = x + (size_t)(r < M ? r : M - 1) * K + c * 8;
        } else {
            const int n = blk0 * 16 + (r - XR);
            src[i] = w + (size_t)(n < N ? n : N - 1) * K + c * 8;
        }
        dst[i] = live ? r * PITCH + c * 8 : SPARE;
    }
    auto load = [&](xv_u32x4 (&reg)[GPT], int part) {   // k-steps part * KSP ..; past the end re-read
        const int k0 = (part < NPARTS ? part : NPARTS - 1) * (KSP * 32);
#pragma unroll
        for (int i = 0; i < GPT; ++i)                      // W is read once, x again by every workgroup
            reg[i] = wsrc[i] ? xv_load16_nt(src[i] + k0) : xv_load16(src[i] + k0);
    };
    auto store = [&](uint16_t* sb, const xv_u32x4 (&reg)[GPT]) {
#pragma unroll
        for (int i = 0; i < GPT; ++i) *reinterpret_cast<xv_u32x4*>(sb + dst[i]) = reg[i];
    };

    const int t = wave / NBG, bg = wave % NBG;
    const bool comp = wave < MT * NBG;          // uniform per wave
    xv_f32x4 acc[BG], sum[BG];
#pragma unroll
    for (int j = 0; j < BG; ++j) { acc[j] = xv_f32x4{0.f, 0.f, 0.f, 0.f}; sum[j] = acc[j]; }

    auto consume = [&](const uint16_t* sb, int p) {    // part p from LDS buffer sb
        if (!comp) return;
        const uint16_t* ap = sb + (t * 16 + lr) * PITCH + lg * 8;
        const uint16_t* bp = sb + (XR + bg * BG * 16 + lr) * PITCH + lg * 8;
#pragma unroll
        for (int kk = 0; kk < KSP; ++kk) {
            const xv_u32x4 a = *reinterpret_cast<const xv_u32x4*>(ap + kk * 32);
#pragma unroll
            for (int j = 0; j < BG; ++j)
                if (bg * BG + j < NBW)          // uniform
                    acc[j] = xv_mfma16x16x32(a, *reinterpret_cast<const xv_u32x4*>(bp + j * 16 * PITCH + kk * 32), acc[j]);
            const int ks = p * KSP + kk + 1;    // k-steps done
            if (ks % KSW == 0) {                // a range complete (uniform): folded in order
#pragma unroll
                for (int j = 0; j < BG; ++j) {
                    sum[j] = ks == KSW ? acc[j] : sum[j] + acc[j];
                    acc[j] = xv_f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
        }
    };

    // register buffer q % NR holds part q; part p is consumed from LDS buffer p % 2
    constexpr int NR = 2;                       // parts in flight (four measured no faster)
    xv_u32x4 rb[NR][GPT];
#pragma unroll
    for (int q = 0; q < NR; ++q) load(rb[q], q);
    store(sm[0], rb[0]);
    load(rb[0], NR);
    __syncthreads();
    // whole rounds of NR parts whose successors all exist: the staging of part p + 1 and the
    // loads of part p + 1 + NR are unconditional, so that the compiler waits for part p + 1
    // alone (a conditional store or load there makes it wait for every load in flight)
    int p0 = 0;
    for (; p0 + NR < NPARTS; p0 += NR) {
#pragma unroll
        for (int u = 0; u < NR; ++u) {
            xv_u32x4 (&rn)[GPT] = rb[(u + 1) % NR];  // holds part p0 + u + 1
            store(sm[(u + 1) & 1], rn);         // its LDS buffer was freed by the last barrier
            load(rn, p0 + u + 1 + NR);
            consume(sm[u & 1], p0 + u);
            __syncthreads();                    // part p consumed, part p + 1 staged
        }
    }
    // the last round (parts p0 .. NPARTS - 1, all loaded): nothing more to load
#pragma unroll
    for (int u = 0; u < NR; ++u) {
        const int p = p0 + u;
        if (p >= NPARTS) break;                 // uniform
        if (p + 1 < NPARTS) store(sm[(u + 1) & 1], rb[(u + 1) % NR]);
        consume(sm[u & 1], p);
        __syncthreads();
    }
    if (!comp) return;
#pragma unroll
    for (int j = 0; j < BG; ++j) {
        const int bk = bg * BG + j;
        const int col = (blk0 + bk) * 16 + lr;
        if (bk >= NBW || col >= N) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = t * 16 + 4 * lg + e;
            if (row < M) {
                const size_t o = (size_t)row * N + col;
                pp.y[cur][o] = xv_f32_to_bf16(sum[j][e]);
                if (pp.y32[cur]) pp.y32[cur][o] = sum[j][e];
            }
        }
    }
}

// x fragments re-read per k-step (many row tiles or long K): U k-steps per stage.
template <int MT, int U>
__global__ __launch_bounds__(XV_GEMM_THREADS)
void xv_gemm_xstream_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                            uint16_t* __restrict__ y, float* __restrict__ y32,
                            int M, int N, int K, int mt0)
{
    __shared__ float red[XV_GEMM_WAVES][64][4];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int KS = K >> 5;
    const int ks0 = (wave * KS) / XV_GEMM_WAVES;
    const int nks = ((wave + 1) * KS) / XV_GEMM_WAVES - ks0;
    const int last = nks > 0 ? nks - 1 : 0;
    const int nblk = N >> 4;
    const int grid = gridDim.x;
    if ((int)blockIdx.x >= nblk) return;
    const xv_u32x4 zero = {0u, 0u, 0u, 0u};

    bool rvalid[MT];
    const uint16_t* xp[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        const int row = (mt0 + t) * 16 + lr;
        rvalid[t] = row < M;
        xp[t] = x + (size_t)(rvalid[t] ? row : M - 1) * K + (size_t)ks0 * 32 + lg * 8;
    }
    const uint16_t* wl = w + (size_t)lr * K + (size_t)ks0 * 32 + lg * 8;
    const int SPB = nks > 0 ? (nks + U - 1) / U : 1;              // stages per column block
    const int my_blocks = (nblk - 1 - (int)blockIdx.x) / grid + 1;
    const int nstages = my_blocks * SPB;

    auto load_stage = [&](xv_u32x4 (&wf)[U], xv_u32x4 (&xf)[U][MT], int s) {
        const int sc = s < nstages ? s : nstages - 1;
        const int blk = blockIdx.x + (sc / SPB) * grid;
        const int j0 = (sc % SPB) * U;
        const uint16_t* wb = wl + (size_t)blk * 16 * K;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int j = j0 + u;
            j = j < nks ? j : last;
            wf[u] = xv_load16(wb + (size_t)j * 32);
#pragma unroll
            for (int t = 0; t < MT; ++t) xf[u][t] = xv_load16(xp[t] + (size_t)j * 32);
        }
    };
    xv_f32x4 acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = xv_f32x4{0.f, 0.f, 0.f, 0.f};
    auto mma_stage = [&](xv_u32x4 (&wf)[U], xv_u32x4 (&xf)[U][MT], int s) {
        const int j0 = (s % SPB) * U;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (j0 + u < nks) {
#pragma unroll
                for (int t = 0; t < MT; ++t)
                    acc[t] = xv_mfma16x16x32(rvalid[t] ? xf[u][t] : zero, wf[u], acc[t]);
            }
        }
    };

    xv_u32x4 wA[U], wB[U], xA[U][MT], xB[U][MT];
    load_stage(wA, xA, 0);
    for (int s = 0; s < nstages; s += 2) {
        load_stage(wB, xB, s + 1);
        mma_stage(wA, xA, s);
        if ((s + 1) % SPB == 0)
            xv_gemm_finish<MT>(red, acc, lane, wave, blockIdx.x + (s / SPB) * grid, mt0, M, N, y, y32);
        if (s + 1 >= nstages) break;
        load_stage(wA, xA, s + 2);
        mma_stage(wB, xB, s + 1);
        if ((s + 2) % SPB == 0)
            xv_gemm_finish<MT>(red, acc, lane, wave, blockIdx.x + ((s + 1) / SPB) * grid, mt0, M, N, y, y32);
    }
}

int xv_gemm_grid(int nblk) {
    const int cus = xv_cu_count();
    return nblk < cus ? nblk : cus;
}

// Where a launch goes: the stream, and optionally events recorded at the start and
// the end of the kernel's execution (hipExtLaunchKernel).
struct XvLaunch {
    hipStream_t st;
    hipEvent_t e0, e1;
};

template <int MT, int KSW>
void xv_gemm_launch_xreg(const uint16_t* x, const uint16_t* w, uint16_t* y, float* y32,
                         int M, int N, int K, int mt0, const XvLaunch& lc)
{
    dim3 grid(xv_gemm_grid(N / 16)), block(XV_GEMM_THREADS);
    hipExtLaunchKernelGGL((xv_gemm_xreg_kernel<MT, KSW>), grid, block, 0, lc.st, lc.e0, lc.e1, 0, x, w, y, y32, M, N, K, mt0);
}

template <int KSW, int SL, int NS>
void xv_gemm_launch_wlds(const XvGemmPair& pp, int M, int K, int mt0, const XvLaunch& lc)
{
    dim3 grid(xv_gemm_grid((pp.N[0] + pp.N[1]) / 16)), block(XV_GEMM_THREADS);
    const int contig = pp.N[1] > 0 && pp.x[0] != pp.x[1];
    hipExtLaunchKernelGGL((xv_gemm_wlds_kernel<KSW, SL, NS, false>), grid, block, 0, lc.st, lc.e0, lc.e1, 0, pp, M,
                          K, mt0, contig, XvHeadGreedy{});
}

// The head with greedy acceptance: N / 16 workgroups, block i of both problems each.
template <int KSW, int SL, int NS>
void xv_gemm_launch_head_greedy(const XvGemmPair& pp, int M, int K, const XvHeadGreedy& hg, const XvLaunch& lc)
{
    hipExtLaunchKernelGGL((xv_gemm_wlds_kernel<KSW, SL, NS, true>), dim3(pp.N[0] / 16), dim3(XV_GEMM_THREADS), 0,
                          lc.st, lc.e0, lc.e1, 0, pp, M, K, 0, 0, hg);
}

// the LDS-staged variant serves one row tile and these K only
bool xv_gemm_wlds_fits(int mt, int K) { return mt == 1 && (K == 5120 || K == 6144); }

void xv_gemm_launch_wlds_k(const XvGemmPair& pp, int M, int K, int mt0, const XvLaunch& lc)
{
    if (K == 5120) xv_gemm_launch_wlds<10, 40, 4>(pp, M, K, mt0, lc);
    else xv_gemm_launch_wlds<12, 48, 4>(pp, M, K, mt0, lc);
}

template <int MT, int KC>
void xv_gemm_launch_kloop(const uint16_t* x, const uint16_t* w, uint16_t* y, float* y32,
                          int M, int N, int K, int mt0, const XvLaunch& lc)
{
    // column blocks per workgroup: as many as keep at least one workgroup per CU busy
    // (callers take this path only for N / 16 >= 2 CUs)
    const int nblk = N / 16, cus = xv_gemm_grid(1 << 30);
    const dim3 block(XV_KL_THREADS);
    if (nblk >= 4 * cus)
        hipExtLaunchKernelGGL((xv_gemm_kloop_kernel<MT, 4, KC>), dim3((nblk + 3) / 4), block, 0, lc.st, lc.e0, lc.e1, 0, x, w, y, y32, M, N, K, mt0);
    else
        hipExtLaunchKernelGGL((xv_gemm_kloop_kernel<MT, 2, KC>), dim3((nblk + 1) / 2), block, 0, lc.st, lc.e0, lc.e1, 0, x, w, y, y32, M, N, K, mt0);
}

template <int MT, int U>
void xv_gemm_launch_xstream(const uint16_t* x, const uint16_t* w, uint16_t* y, float* y32,
                            int M, int N, int K, int mt0, const XvLaunch& lc)
{
    dim3 grid(xv_gemm_grid(N / 16)), block(XV_GEMM_THREADS);
    hipExtLaunchKernelGGL((xv_gemm_xstream_kernel<MT, U>), grid, block, 0, lc.st, lc.e0, lc.e1, 0, x, w, y, y32, M, N, K, mt0);
}

// Launch of the 2..5-row-tile kernel for one or two problems (N[1] = 0: one): the fewest
// column blocks per workgroup that still fit every workgroup on the chip at once (one
// per CU), so that no CU runs a second round; at most 7 (two LDS buffers of 5 row tiles
// and 7 blocks at K = 6144 fill the 160 KB of LDS).
bool xv_gemm_mt_fits(int mt, int K) { return mt >= 2 && mt <= XV_GEMM_MT_MAX && (K == 5120 || K == 6144); }

template <int MT, int KSP>
void xv_gemm_launch_mt_n(const XvGemmPair& pp, int M, int K, const XvLaunch& lc)
{
    const int nb0 = pp.N[0] / 16, nb1 = pp.N[1] / 16;
    const int cus = xv_gemm_grid(1 << 30);
    auto wgs = [&](int nbw) { return (nb0 + nbw - 1) / nbw + (nb1 + nbw - 1) / nbw; };
    int nbw = 1;
    while (nbw < 7 && wgs(nbw) > cus) ++nbw;
#define XV_MT_LAUNCH(NBWV)                                                                                   \
    hipExtLaunchKernelGGL((xv_gemm_mt_kernel<MT, KSP, NBWV>), dim3(wgs(NBWV)), dim3(XV_GEMM_THREADS), 0,    \
                          lc.st, lc.e0, lc.e1, 0, pp, M, K, (nb0 + NBWV - 1) / NBWV)
    switch (nbw) {
        case 1: XV_MT_LAUNCH(1); break;
        case 2: XV_MT_LAUNCH(2); break;
        case 3: XV_MT_LAUNCH(3); break;
        case 4: XV_MT_LAUNCH(4); break;
        case 5: XV_MT_LAUNCH(5); break;
        case 6: XV_MT_LAUNCH(6); break;
        default: XV_MT_LAUNCH(7); break;
    }
#undef XV_MT_LAUNCH
}

void xv_gemm_launch_mt(const XvGemmPair& pp, int mt, int M, int K, const XvLaunch& lc)
{
    // parts of 4 k-steps at K = 5120 (256-byte row runs: a 5-step part of 320 bytes splits every
    // other 128-byte line between two parts, which streams measurably slower), 6 at K = 6144
    if (K == 5120) {
        switch (mt) {
            case 2: xv_gemm_launch_mt_n<2, 4>(pp, M, K, lc); break;
            case 3: xv_gemm_launch_mt_n<3, 4>(pp, M, K, lc); break;
            case 4: xv_gemm_launch_mt_n<4, 4>(pp, M, K, lc); break;
            default: xv_gemm_launch_mt_n<5, 4>(pp, M, K, lc); break;
        }
    } else {
        switch (mt) {
            case 2: xv_gemm_launch_mt_n<2, 6>(pp, M, K, lc); break;
            case 3: xv_gemm_launch_mt_n<3, 6>(pp, M, K, lc); break;
            case 4: xv_gemm_launch_mt_n<4, 6>(pp, M, K, lc); break;
            default: xv_gemm_launch_mt_n<5, 6>(pp, M, K, lc); break;
        }
    }
}

// Launch shape per row-tile count and K.  None of these choices changes any
// row's arithmetic: every variant runs the same 16-way K split, the same MFMA
// chains and the same ordered sum.
void xv_gemm_dispatch(int mt, int ksw, const uint16_t* x, const uint16_t* w, uint16_t* y,
                      float* y32, int M, int N, int K, int mt0, const XvLaunch& lc)
{
    // one row tile and the two K of the 27B-class layer: W through LDS in 1 KB contiguous wave loads
    if (xv_gemm_wlds_fits(mt, K)) {
        const XvGemmPair pp{{x, nullptr}, {w, nullptr}, {y, nullptr}, {y32, nullptr}, {N, 0}};
        xv_gemm_launch_wlds_k(pp, M, K, mt0, lc);
        return;
    }
    if (mt == 1 && ksw <= 10) {
        if (ksw <= 2) xv_gemm_launch_xreg<1, 2>(x, w, y, y32, M, N, K, mt0, lc);
        else if (ksw <= 4) xv_gemm_launch_xreg<1, 4>(x, w, y, y32, M, N, K, mt0, lc);
        else if (ksw <= 6) xv_gemm_launch_xreg<1, 6>(x, w, y, y32, M, N, K, mt0, lc);
        else if (ksw <= 8) xv_gemm_launch_xreg<1, 8>(x, w, y, y32, M, N, K, mt0, lc);
        else xv_gemm_launch_xreg<1, 10>(x, w, y, y32, M, N, K, mt0, lc);
        return;
    }
    // 2..5 row tiles and the two K of the layer: W streamed once, x from L2
    if (mt0 == 0 && M <= XV_GEMM_MT_MAX * 16 && xv_gemm_mt_fits(mt, K)) {
        const XvGemmPair pp{{x, nullptr}, {w, nullptr}, {y, nullptr}, {y32, nullptr}, {N, 0}};
        xv_gemm_launch_mt(pp, mt, M, K, lc);
        return;
    }
    // several row tiles and many column blocks: walk K per output tile (x reused over 2-4 column blocks)
    if (mt >= 2 && N / 16 >= 2 * xv_gemm_grid(1 << 30)) {
        switch (mt) {
            case 2: xv_gemm_launch_kloop<2, 4>(x, w, y, y32, M, N, K, mt0, lc); break;
            case 3: xv_gemm_launch_kloop<3, 4>(x, w, y, y32, M, N, K, mt0, lc); break;
            case 4: xv_gemm_launch_kloop<4, 4>(x, w, y, y32, M, N, K, mt0, lc); break;
            default: xv_gemm_launch_kloop<5, 4>(x, w, y, y32, M, N, K, mt0, lc); break;
        }
        return;
    }
    if (mt == 2 && ksw <= 4) {
        xv_gemm_launch_xreg<2, 4>(x, w, y, y32, M, N, K, mt0, lc);
        return;
    }
    switch (mt) {
        case 1: xv_gemm_launch_xstream<1, 4>(x, w, y, y32, M, N, K, mt0, lc); break;
        case 2: xv_gemm_launch_xstream<2, 2>(x, w, y, y32, M, N, K, mt0, lc); break;
        case 3: xv_gemm_launch_xstream<3, 1>(x, w, y, y32, M, N, K, mt0, lc); break;
        case 4: xv_gemm_launch_xstream<4, 1>(x, w, y, y32, M, N, K, mt0, lc); break;
        default: xv_gemm_launch_xstream<5, 1>(x, w, y, y32, M, N, K, mt0, lc); break;
    }
}

}  // namespace

extern "C" int xv_gemm_small_m_timed(const uint16_t* x, const uint16_t* w, uint16_t* y, float* y32,
                                     int M, int N, int K, void* stream, void* start_event,
                                     void* stop_event)
{
    XV_REQUIRE(M >= 0 && N >= 16 && N % 16 == 0 && K >= 32 && K % 32 == 0, XV_ERR_SHAPE);
    if (M == 0) return XV_OK;
    XV_REQUIRE(x && w && y, XV_ERR_NULL);
    XV_REQUIRE(xv_aligned16(x) && xv_aligned16(w) && xv_aligned(y, 2) && xv_aligned(y32, 4),
               XV_ERR_ALIGN);
    (void)hipGetLastError();
    const int KS = K / 32;
    const int ksw = (KS + XV_GEMM_WAVES - 1) / XV_GEMM_WAVES;   // k-steps of the longest range
    const int tiles = (M + 15) / 16;
    if (M >= XV_BIG_MIN_M) {                    // many rows: one launch of 128 x 128 tiles
        const int mb = (M + XV_BIG_BM - 1) / XV_BIG_BM, nb = (N + XV_BIG_BN - 1) / XV_BIG_BN;
        XV_REQUIRE((long long)mb * nb < (1LL << 31), XV_ERR_SHAPE);
        hipExtLaunchKernelGGL(xv_gemm_big_kernel, dim3(mb * nb), dim3(XV_BIG_THREADS), 0,
                              reinterpret_cast<hipStream_t>(stream), reinterpret_cast<hipEvent_t>(start_event),
                              reinterpret_cast<hipEvent_t>(stop_event), 0, x, w, y, y32, M, N, K, mb);
        return xv_launch_status();
    }
    for (int mt0 = 0; mt0 < tiles; mt0 += XV_GEMM_MT_MAX) {
        const int mt = tiles - mt0 < XV_GEMM_MT_MAX ? tiles - mt0 : XV_GEMM_MT_MAX;
        // the start event goes with the first launch, the stop event with the last
        const XvLaunch lc{reinterpret_cast<hipStream_t>(stream),
                          mt0 == 0 ? reinterpret_cast<hipEvent_t>(start_event) : nullptr,
                          mt0 + mt >= tiles ? reinterpret_cast<hipEvent_t>(stop_event) : nullptr};
        xv_gemm_dispatch(mt, ksw, x, w, y, y32, M, N, K, mt0, lc);
        int s = xv_launch_status();
        if (s != XV_OK) return s;
    }
    return XV_OK;
}

extern "C" int xv_gemm_small_m(const uint16_t* x, const uint16_t* w, uint16_t* y, float* y32,
                               int M, int N, int K, void* stream)
{
    return xv_gemm_small_m_timed(x, w, y, y32, M, N, K, stream, nullptr, nullptr);
}

extern "C" int xv_gemm_small_m_pair(const uint16_t* x0, const uint16_t* w0, uint16_t* y0, float* y32_0, int N0,
                                    const uint16_t* x1, const uint16_t* w1, uint16_t* y1, float* y32_1, int N1,
                                    int M, int K, void* stream, void* start_event, void* stop_event)
{
    XV_REQUIRE(M >= 0 && K >= 32 && K % 32 == 0, XV_ERR_SHAPE);
    XV_REQUIRE(N0 >= 16 && N0 % 16 == 0 && N1 >= 16 && N1 % 16 == 0, XV_ERR_SHAPE);
    if (M == 0) return XV_OK;
    XV_REQUIRE(x0 && w0 && y0 && x1 && w1 && y1, XV_ERR_NULL);
    XV_REQUIRE(xv_aligned16(x0) && xv_aligned16(w0) && xv_aligned(y0, 2) && xv_aligned(y32_0, 4) &&
               xv_aligned16(x1) && xv_aligned16(w1) && xv_aligned(y1, 2) && xv_aligned(y32_1, 4),
               XV_ERR_ALIGN);
    const int tiles = (M + 15) / 16;
    if (tiles >= 2 && tiles <= XV_GEMM_MT_MAX && xv_gemm_mt_fits(tiles, K)) {
        (void)hipGetLastError();
        const XvLaunch lc{reinterpret_cast<hipStream_t>(stream), reinterpret_cast<hipEvent_t>(start_event),
                          reinterpret_cast<hipEvent_t>(stop_event)};
        const XvGemmPair pp{{x0, x1}, {w0, w1}, {y0, y1}, {y32_0, y32_1}, {N0, N1}};
        xv_gemm_launch_mt(pp, tiles, M, K, lc);
        return xv_launch_status();
    }
    if (!xv_gemm_wlds_fits(tiles, K)) {
        // no fused variant for this shape: the two GEMMs one after the other (same bits)
        int s = xv_gemm_small_m_timed(x0, w0, y0, y32_0, M, N0, K, stream, start_event, nullptr);
        if (s != XV_OK) return s;
        return xv_gemm_small_m_timed(x1, w1, y1, y32_1, M, N1, K, stream, nullptr, stop_event);
    }
    (void)hipGetLastError();
    const XvLaunch lc{reinterpret_cast<hipStream_t>(stream), reinterpret_cast<hipEvent_t>(start_event),
                      reinterpret_cast<hipEvent_t>(stop_event)};
    const XvGemmPair pp{{x0, x1}, {w0, w1}, {y0, y1}, {y32_0, y32_1}, {N0, N1}};
    xv_gemm_launch_wlds_k(pp, M, K, 0, lc);
    return xv_launch_status();
}

extern "C" size_t xv_head_greedy_workspace_bytes(int B, int T, int N)
{
    const long long rows = B > 0 && T > 0 ? (long long)B * T : 0;
    const long long nb = N > 0 ? (N + 15LL) / 16 : 0;
    return (size_t)(256 + 16 * rows * nb);
}

extern "C" int xv_head_greedy_accept(const uint16_t* x_a, const uint16_t* w_a, uint16_t* y_a, float* logits_a,
                                     const uint16_t* x_b, const uint16_t* w_b, uint16_t* y_b, float* logits_b,
                                     const int32_t* draft, int32_t* ids, int32_t* n_keep, float* logprob,
                                     int32_t* kv_len, void* workspace, size_t workspace_bytes,
                                     int B, int T, int N, int K, void* stream)
{
    XV_REQUIRE(B >= 0 && B <= (1 << 20) && T >= 1 && T <= XV_TMAX, XV_ERR_SHAPE);
    XV_REQUIRE(N >= 16 && N % 16 == 0 && K >= 32 && K % 32 == 0, XV_ERR_SHAPE);
    if (B == 0) return XV_OK;
    XV_REQUIRE(x_a && w_a && y_a && logits_a && x_b && w_b && y_b && logits_b && draft && ids && n_keep &&
               workspace, XV_ERR_NULL);
    XV_REQUIRE(xv_aligned16(x_a) && xv_aligned16(w_a) && xv_aligned(y_a, 2) && xv_aligned(logits_a, 4) &&
               xv_aligned16(x_b) && xv_aligned16(w_b) && xv_aligned(y_b, 2) && xv_aligned(logits_b, 4) &&
               xv_aligned(draft, 4) && xv_aligned(ids, 4) && xv_aligned(n_keep, 4) &&
               xv_aligned(logprob, 4) && xv_aligned(kv_len, 4) && xv_aligned16(workspace), XV_ERR_ALIGN);
    XV_REQUIRE(workspace_bytes >= xv_head_greedy_workspace_bytes(B, T, N), XV_ERR_WORKSPACE);
    const int M = B * T;
    if (M <= 16 && (K == 5120 || K == 6144)) {
        // one row tile and the layer's K: the fused launch
        (void)hipGetLastError();
        const XvLaunch lc{reinterpret_cast<hipStream_t>(stream), nullptr, nullptr};
        const XvGemmPair pp{{x_a, x_b}, {w_a, w_b}, {y_a, y_b}, {logits_a, logits_b}, {N, N}};
        char* ws = static_cast<char*>(workspace);
        const XvHeadGreedy hg{draft, ids, n_keep, logprob, kv_len, reinterpret_cast<XvHeadPair*>(ws + 256),
                              reinterpret_cast<int*>(ws), B, T};
        if (K == 5120) xv_gemm_launch_head_greedy<10, 40, 4>(pp, M, K, hg, lc);
        else xv_gemm_launch_head_greedy<12, 48, 4>(pp, M, K, hg, lc);
        return xv_launch_status();
    }
    // otherwise the pair, then the argmax and acceptance in one launch with a counter per request
    // (ints 1 .. 63 of the workspace's first 256 bytes), or in two for more requests (the same bits)
    const int s = xv_gemm_small_m_pair(x_a, w_a, y_a, logits_a, N, x_b, w_b, y_b, logits_b, N, M, K, stream,
                                       nullptr, nullptr);
    if (s != XV_OK) return s;
    if (B <= 63)
        return xv_detail::xv_greedy_accept_counted(logits_a, logits_b, draft, B, T, N, ids, n_keep, logprob, kv_len,
                                                   static_cast<int*>(workspace) + 1, stream);
    return xv_greedy_accept(logits_a, logits_b, draft, B, T, N, ids, n_keep, logprob, kv_len, stream);
}
