// abi_sanitize_main.cpp -- a host program for the sanitizer build of libxv's host code:
// every C entry point is called with arguments that break one of its checks (null,
// shape, alignment, alias, workspace, ...) and must return that check's status before
// any device call.  Built with AddressSanitizer and UndefinedBehaviorSanitizer on the host
// side, it runs on a machine without a GPU (nothing here launches).  Exit 0: every
// status as documented in xv.h and no sanitizer report.
#include <cmath>
#include <cstdint>
#include <cstdio>

#include "../../include/xv.h"

static int fails = 0;
#define EXPECT(call, want) do { const int got_ = (call); if (got_ != (want)) { \
    std::fprintf(stderr, "line %d: %s returned %d, want %d\n", __LINE__, #call, got_, (want)); ++fails; } } while (0)

int main()
{
    // fake device addresses (never dereferenced): 16-byte aligned, 4-byte only, odd
    uint16_t* A = reinterpret_cast<uint16_t*>(0x10000);
    float* F = reinterpret_cast<float*>(0x20000);
    float* G = reinterpret_cast<float*>(0x30000);
    float* H = reinterpret_cast<float*>(0x50000);
    float* J = reinterpret_cast<float*>(0x60000);
    int32_t* I = reinterpret_cast<int32_t*>(0x40000);
    uint16_t* MIS = reinterpret_cast<uint16_t*>(0x10004);
    uint16_t* ODD = reinterpret_cast<uint16_t*>(0x10001);

    EXPECT(xv_abi_version(), XV_ABI_VERSION);
    for (int s = 1; s >= -7; --s) (void)xv_status_string(s);
    EXPECT(xv_attn_chunk_tokens(), 256);
    EXPECT((int)(xv_attn_workspace_bytes(0, 9, 24, 256, 256) == 0), 1);
    EXPECT((int)(xv_attn_workspace_bytes(1, 9, 24, 256, 649) == 4096 + (size_t)9 * 24 * 3 * 258 * 4), 1);

    // GEMMs
    EXPECT(xv_gemm_small_m(A, A, A, nullptr, 0, 16, 32, nullptr), XV_OK);
    EXPECT(xv_gemm_small_m(nullptr, A, A, nullptr, 9, 16, 32, nullptr), XV_ERR_NULL);
    EXPECT(xv_gemm_small_m(A, A, A, nullptr, 9, 17, 32, nullptr), XV_ERR_SHAPE);
    EXPECT(xv_gemm_small_m(A, A, A, nullptr, 9, 16, 33, nullptr), XV_ERR_SHAPE);
    EXPECT(xv_gemm_small_m(MIS, A, A, nullptr, 9, 16, 32, nullptr), XV_ERR_ALIGN);
    EXPECT(xv_gemm_small_m_timed(A, A, A, nullptr, -1, 16, 32, nullptr, nullptr, nullptr), XV_ERR_SHAPE);
    EXPECT(xv_gemm_small_m_pair(A, A, A, nullptr, 16, A, A, nullptr, nullptr, 16, 9, 32, nullptr, nullptr, nullptr),
           XV_ERR_NULL);
    EXPECT(xv_gemm_small_m_pair(A, A, A, nullptr, 16, A, A, A, nullptr, 20, 9, 32, nullptr, nullptr, nullptr),
           XV_ERR_SHAPE);

    // GDN
    EXPECT(xv_gdn_verify(A, A, A, F, F, F, G, A, nullptr, 0, 9, 16, 48, 128, 128, nullptr), XV_OK);
    EXPECT(xv_gdn_verify(A, A, A, F, F, F, G, A, nullptr, 1, 17, 16, 48, 128, 128, nullptr), XV_ERR_SHAPE);
    EXPECT(xv_gdn_verify(A, A, A, F, F, F, G, A, nullptr, 1, 9, 16, 40, 128, 128, nullptr), XV_ERR_SHAPE);
    EXPECT(xv_gdn_verify(A, A, A, F, F, F, G, A, nullptr, 1, 9, 16, 48, 96, 128, nullptr), XV_ERR_SHAPE);
    EXPECT(xv_gdn_verify(nullptr, A, A, F, F, F, G, A, nullptr, 1, 9, 16, 48, 128, 128, nullptr), XV_ERR_NULL);
    EXPECT(xv_gdn_verify(A, MIS, A, F, F, F, G, A, nullptr, 1, 9, 16, 48, 128, 128, nullptr), XV_ERR_ALIGN);
    EXPECT(xv_gdn_verify(A, A, A, F, F, F, F, A, nullptr, 1, 9, 16, 48, 128, 128, nullptr), XV_ERR_ALIAS);
    EXPECT(xv_gdn_verify_after(A, A, A, F, F, A, A, F, F, I, 0, F, G, H, J, A, nullptr,
                               1, 9, 16, 48, 128, 128, nullptr), XV_ERR_SHAPE);
    EXPECT(xv_gdn_verify_after(A, A, A, F, F, A, A, F, F, I, 9, F, G, H, G, A, nullptr,
                               1, 9, 16, 48, 128, 128, nullptr), XV_ERR_ALIAS);
    EXPECT(xv_gdn_prefill(A, A, A, F, F, F, G, A, nullptr, 1, 0, 16, 48, 128, 128, nullptr), XV_ERR_SHAPE);
    EXPECT(xv_rollback_to_prefix(A, A, F, F, F, G, nullptr, I, 1, 9, 16, 48, 128, 128, nullptr), XV_ERR_NULL);

    // attention
    const size_t need = xv_attn_workspace_bytes(1, 9, 24, 256, 649);
    EXPECT(xv_attn_verify_rows(A, A, A, A, A, I, A, nullptr, F, need, 0, 9, 24, 4, 256, 649, 0.0625f, 0, nullptr), XV_OK);
    EXPECT(xv_attn_verify_rows(A, A, A, A, A, I, A, nullptr, F, need, 1, 17, 24, 4, 256, 649, 0.0625f, 0, nullptr),
           XV_ERR_SHAPE);
    EXPECT(xv_attn_verify_rows(A, A, A, A, A, I, A, nullptr, F, need, 1, 9, 24, 4, 256, 649, NAN, 0, nullptr),
           XV_ERR_SHAPE);
    EXPECT(xv_attn_verify_rows(A, A, A, A, A, I, A, nullptr, nullptr, need, 1, 9, 24, 4, 256, 649, 0.0625f, 0, nullptr),
           XV_ERR_NULL);
    EXPECT(xv_attn_verify_rows(A, A, A, A, A, I, A, nullptr, F, need - 4, 1, 9, 24, 4, 256, 649, 0.0625f, 0, nullptr),
           XV_ERR_WORKSPACE);
    EXPECT(xv_attn_verify_rows_noalloc(A, A, A, A, A, I, A, nullptr, 1, 9, 24, 4, 256, 127744, 0.0625f, 0, nullptr),
           XV_ERR_WORKSPACE);
    EXPECT(xv_attn_verify_rows_noalloc(MIS, A, A, A, A, I, A, nullptr, 1, 9, 24, 4, 256, 649, 0.0625f, 0, nullptr),
           XV_ERR_ALIGN);
    EXPECT(xv_attn_verify_rows(A, A, A, A, A, I, A, nullptr, F, need, 1, 9, 24, 4, 256, 649, 0.0625f, 8, nullptr),
           XV_ERR_SHAPE);                       // a length bound below T
    EXPECT(xv_attn_prefill(A, A, A, A, A, I, A, nullptr, 1, 8, 24, 4, 96, 649, 0.0625f, 1, nullptr), XV_ERR_SHAPE);
    EXPECT(xv_gdn_attn_verify(A, A, A, F, F, nullptr, nullptr, nullptr, nullptr, nullptr, 0, F, nullptr, nullptr, G,
                              A, nullptr, 16, 48, 128, 128, A, A, A, A, A, I, A, nullptr, F, need,
                              24, 4, 256, 649, 0.0625f, 1, 17, 0, nullptr), XV_ERR_SHAPE);

    // greedy, embedding, split, streaming read
    EXPECT(xv_greedy_accept(reinterpret_cast<float*>(A), nullptr, I, 1, 0, 4096, I, I, nullptr, nullptr, nullptr),
           XV_ERR_SHAPE);
    EXPECT(xv_greedy_accept(reinterpret_cast<float*>(A), reinterpret_cast<float*>(ODD), I, 1, 9, 4096, I, I,
                            nullptr, nullptr, nullptr), XV_ERR_ALIGN);
    {
        const size_t wsb = xv_head_greedy_workspace_bytes(1, 9, 4096);
        EXPECT(xv_head_greedy_accept(A, A, A, F, A, A, A, F, I, I, I, nullptr, nullptr, A, wsb, 1, 17, 4096, 6144,
                                     nullptr), XV_ERR_SHAPE);
        EXPECT(xv_head_greedy_accept(A, A, A, F, A, A, A, F, I, I, I, nullptr, nullptr, nullptr, wsb, 1, 9, 4096,
                                     6144, nullptr), XV_ERR_NULL);
        EXPECT(xv_head_greedy_accept(A, A, A, F, A, A, A, F, I, I, I, nullptr, nullptr, A, wsb - 1, 1, 9, 4096,
                                     6144, nullptr), XV_ERR_WORKSPACE);
        EXPECT(xv_head_greedy_accept(A, A, A, F, A, A, A, F, I, I, I, nullptr, nullptr, A, wsb, 0, 9, 4096, 6144,
                                     nullptr), XV_OK);
    }
    EXPECT(xv_embed_rows(A, I, 9, 4096, 5124, A, nullptr), XV_ERR_SHAPE);
    EXPECT(xv_stream_read(A, 1000, A, 1024, reinterpret_cast<uint32_t*>(I), 8, nullptr, nullptr, nullptr), XV_ERR_SHAPE);
    EXPECT(xv_stream_read(nullptr, 1024, A, 1024, reinterpret_cast<uint32_t*>(I), 8, nullptr, nullptr, nullptr),
           XV_ERR_NULL);

    if (fails) { std::fprintf(stderr, "%d checks failed\n", fails); return 1; }
    std::printf("libxv host checks under the sanitizers: ok\n");
    return 0;
}
