// xv_common.h -- device helpers and host-side argument checks shared by the
// libxv kernels (gfx950 / CDNA4 only).
//
// Floating-point policy for every kernel in the library: the code is built with
// -ffp-contract=off and without fast-math, and every fused multiply-add is
// written out with __builtin_fmaf, so a given source expression always becomes
// the same instruction sequence whatever the surrounding code.  Together with a
// single code path per operation whose per-row order never depends on the row
// count, this is what makes verify rows bit-identical to decode steps.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>
#include <atomic>

#include "../../include/xv.h"

// ---------------------------------------------------------------------------
// bf16 <-> fp32
// ---------------------------------------------------------------------------
__device__ __forceinline__ float xv_bf16_to_f32(uint32_t h16) {
    return __uint_as_float(h16 << 16);
}

// low / high halves of a packed pair of bf16 values
__device__ __forceinline__ float xv_bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float xv_bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t xv_f32_to_bf16(float f) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t rne = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    const uint32_t qnan = (u >> 16) | 0x0040u;               // NaN: keep the sign, make it quiet
    return (uint16_t)((u & 0x7FFFFFFFu) > 0x7F800000u ? qnan : rne);   // a select, no branch
}

// Two fp32 values -> packed bf16 pair (low half = a), round to nearest even
// (v_cvt_pk_bf16_f32 on gfx950).
typedef float xv_f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 xv_bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t xv_pack_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(xv_f32x2{a, b}, xv_bf16x2));
}

// ---------------------------------------------------------------------------
// MFMA operand types (v_mfma_f32_16x16x32_bf16: A 16x32, B 32x16, C/D 16x16 fp32)
//   lane l supplies A[l % 16][8 * (l / 16) + e] and B[8 * (l / 16) + e][l % 16]
//   for e = 0..7, and holds D[4 * (l / 16) + i][l % 16] for i = 0..3.
// The contraction index k is matched between A and B by (l / 16, e) on both
// sides, so any fixed assignment of data to k-slots that is the same for A and
// B contracts correctly.
// ---------------------------------------------------------------------------
typedef __bf16 xv_bf16x8 __attribute__((ext_vector_type(8)));
typedef float xv_f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t xv_u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ xv_bf16x8 xv_as_bf16x8(xv_u32x4 v) {
    return __builtin_bit_cast(xv_bf16x8, v);
}

__device__ __forceinline__ xv_f32x4 xv_mfma16x16x32(xv_u32x4 a, xv_u32x4 b, xv_f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv_as_bf16x8(a), xv_as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ xv_u32x4 xv_load16(const void* p) {
    return *reinterpret_cast<const xv_u32x4*>(p);
}

// a 16-byte load of data read once per call (weights, states, KV streamed once): the
// non-temporal hint keeps it from displacing lines that are read again
__device__ __forceinline__ xv_u32x4 xv_load16_nt(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const xv_u32x4*>(p));
}

__device__ __forceinline__ void xv_store16(void* p, xv_u32x4 v) {
    *reinterpret_cast<xv_u32x4*>(p) = v;
}

// ---------------------------------------------------------------------------
// Host-side checks
// ---------------------------------------------------------------------------
static inline bool xv_aligned16(const void* p) { return (((uintptr_t)p) & 15u) == 0; }
// element alignment (2 for bf16, 4 for fp32 / int32)
static inline bool xv_aligned(const void* p, unsigned n) { return (((uintptr_t)p) & (n - 1u)) == 0; }

#define XV_REQUIRE(cond, code) do { if (!(cond)) return (code); } while (0)

static inline int xv_launch_status() {
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? XV_OK : XV_ERR_LAUNCH;
}

// The current device's compute-unit count (for grid sizes; 256 on MI355X), queried once per
// device and kept; several host threads may call it at once.
inline int xv_cu_count() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    int cus = dev < 64 ? cached[dev].load(std::memory_order_relaxed) : 0;
    if (cus > 0) return cus;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    if (dev < 64) cached[dev].store(cus, std::memory_order_relaxed);
    return cus;
}
