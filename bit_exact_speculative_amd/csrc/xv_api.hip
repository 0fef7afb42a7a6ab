// xv_api.hip -- library-wide C entry points of libxv (version, status text, and the
// streaming-read measurement helper).
#include "xv_common.h"
#include <hip/hip_ext.h>

extern "C" int xv_abi_version(void) { return XV_ABI_VERSION; }

extern "C" const char* xv_status_string(int status) {
    switch (status) {
        case XV_OK: return "ok";
        case XV_ERR_NULL: return "a required pointer is NULL";
        case XV_ERR_SHAPE: return "a size is outside the supported set";
        case XV_ERR_ALIGN: return "a pointer breaks its alignment rule";
        case XV_ERR_WORKSPACE: return "workspace too small";
        case XV_ERR_LAUNCH: return "kernel launch failed";
        case XV_ERR_ALIAS: return "an output aliases an input it must not overwrite";
        default: return "unknown status";
    }
}

// ---------------------------------------------------------------------------
// Streaming-read ceiling: two buffers read once with 16-byte loads; workgroup i
// streams its own contiguous range of their concatenation (1 KB per wave load,
// four loads in flight per thread), the fastest of the read patterns measured on
// MI355X for a cold 283 MB; each workgroup writes the XOR of the words it read to
// sink[workgroup] (so no load is dead).
// ---------------------------------------------------------------------------
namespace {

constexpr int XV_READ_THREADS = 256;
constexpr int XV_READ_UNROLL = 4;

__global__ __launch_bounds__(XV_READ_THREADS)
void xv_stream_read_kernel(const xv_u32x4* __restrict__ a, size_t na, const xv_u32x4* __restrict__ b, size_t nb,
                           uint32_t* __restrict__ sink)
{
    const size_t n = na + nb;
    const size_t per = (n + gridDim.x - 1) / gridDim.x;
    const size_t e0 = (size_t)blockIdx.x * per;
    const size_t e1 = e0 + per < n ? e0 + per : n;
    xv_u32x4 acc = {0u, 0u, 0u, 0u};
    size_t i = e0 + threadIdx.x;
    for (; i + (XV_READ_UNROLL - 1) * XV_READ_THREADS < e1; i += XV_READ_UNROLL * XV_READ_THREADS) {
        xv_u32x4 v[XV_READ_UNROLL];
#pragma unroll
        for (int u = 0; u < XV_READ_UNROLL; ++u) {
            const size_t j = i + u * XV_READ_THREADS;
            v[u] = __builtin_nontemporal_load(j < na ? &a[j] : &b[j - na]);
        }
#pragma unroll
        for (int u = 0; u < XV_READ_UNROLL; ++u) acc ^= v[u];
    }
    for (; i < e1; i += XV_READ_THREADS) acc ^= (i < na ? a[i] : b[i - na]);
    uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    for (int off = 32; off > 0; off >>= 1) x ^= (uint32_t)__shfl_xor((int)x, off);
    __shared__ uint32_t part[XV_READ_THREADS / 64];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t y = 0;
        for (int w = 0; w < XV_READ_THREADS / 64; ++w) y ^= part[w];
        sink[blockIdx.x] = y;
    }
}

}  // namespace

extern "C" int xv_stream_read(const void* src0, size_t bytes0, const void* src1, size_t bytes1,
                              uint32_t* sink, int sink_words, void* stream, void* start_event, void* stop_event)
{
    XV_REQUIRE(sink_words >= 1 && bytes0 % 16 == 0 && bytes1 % 16 == 0, XV_ERR_SHAPE);
    XV_REQUIRE((src0 || bytes0 == 0) && (src1 || bytes1 == 0) && sink, XV_ERR_NULL);
    XV_REQUIRE(xv_aligned16(src0) && xv_aligned16(src1) && xv_aligned(sink, 4), XV_ERR_ALIGN);
    if (bytes0 + bytes1 == 0) return XV_OK;
    (void)hipGetLastError();
    hipExtLaunchKernelGGL(xv_stream_read_kernel, dim3(sink_words), dim3(XV_READ_THREADS), 0,
                          reinterpret_cast<hipStream_t>(stream), reinterpret_cast<hipEvent_t>(start_event),
                          reinterpret_cast<hipEvent_t>(stop_event), 0,
                          reinterpret_cast<const xv_u32x4*>(src0), bytes0 / 16,
                          reinterpret_cast<const xv_u32x4*>(src1), bytes1 / 16, sink);
    return xv_launch_status();
}
