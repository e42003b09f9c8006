// abi_checks.cpp — the C ABI's host-side validation under AddressSanitizer /
// UndefinedBehaviorSanitizer (tests/test_sanitizers.py builds the library's host code with
// -fsanitize=address,undefined and links this driver).  Every call below fails a host-side
// check before the library's first HIP call, so nothing reaches a device: the pointers are fake
// and never dereferenced.  The workspace-size functions run on large sizes as well.
#include <stdint.h>
#include <stdio.h>

#include "csa.h"

static int fails = 0;
#define EXPECT(call, code)                                                                     \
    do {                                                                                       \
        const int rc_ = (call);                                                                \
        if (rc_ != (code)) {                                                                   \
            printf("FAIL %s:%d: %s -> %d, expected %d\n", __FILE__, __LINE__, #call, rc_, code); \
            ++fails;                                                                           \
        }                                                                                      \
    } while (0)

int main() {
    void* A = reinterpret_cast<void*>(0x10000);     // 16-byte aligned, never dereferenced
    void* MIS = reinterpret_cast<void*>(0x10004);   // misaligned
    const float* F = static_cast<const float*>(A);
    int32_t* I = static_cast<int32_t*>(A);
    float* FO = static_cast<float*>(A);
    const csa_dtype f32 = CSA_F32, bf16 = CSA_BF16, fp8 = CSA_FP8_E4M3, mx = CSA_MXFP4, mix = CSA_KV_FP8_BF16;

    // compression
    EXPECT(csa_compress(nullptr, A, A, A, F, F, 1, 64, 4, 64, f32, A, f32, nullptr), CSA_ERR_INVALID_ARG);
    EXPECT(csa_compress(A, A, MIS, A, F, F, 1, 64, 4, 64, f32, A, f32, nullptr), CSA_ERR_INVALID_ARG);
    EXPECT(csa_compress(A, A, A, A, F, F, -1, 64, 4, 64, f32, A, f32, nullptr), CSA_ERR_INVALID_ARG);
    EXPECT(csa_compress(A, A, A, A, F, F, 1, 64, 4, 60, f32, A, f32, nullptr), CSA_ERR_UNSUPPORTED);
    EXPECT(csa_compress(A, A, A, A, F, F, 1, 64, 4096, 64, f32, A, f32, nullptr), CSA_ERR_UNSUPPORTED);
    EXPECT(csa_compress(A, A, A, A, F, F, 1, 64, 4, 64, fp8, A, f32, nullptr), CSA_ERR_UNSUPPORTED);
    EXPECT(csa_compress(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 1, 3, 4, 64, f32, nullptr, fp8, nullptr),
           CSA_OK);
    EXPECT(csa_compress_step(A, A, A, A, F, F, 1, 9, 4, 64, bf16, A, 9, bf16, nullptr), CSA_ERR_INVALID_ARG);
    EXPECT(hca_compress(A, A, F, 1, 256, 0, 64, bf16, A, bf16, nullptr), CSA_ERR_INVALID_ARG);
    EXPECT(hca_compress_step(A, A, F, 1, 3, 128, 64, bf16, MIS, 8, fp8, nullptr), CSA_ERR_INVALID_ARG);
    EXPECT(hca_compress_step(A, A, F, 1, 8, 128, 64, bf16, A, 8, fp8, nullptr), CSA_ERR_INVALID_ARG);

    // indexer and top-k
    const size_t need = csa_index_topk_workspace_size(32, 1, 32768, 64, 1024);
    EXPECT(csa_index_topk(A, F, A, 32, 1, 131072, 32768, 64, 128, 4, 1024, fp8, I, FO, A, need - 1, nullptr),
           CSA_ERR_WORKSPACE);
    EXPECT(csa_index_topk(A, F, A, 32, 1, 131072, 32768, 64, 128, 4, 4096, fp8, I, FO, A, need, nullptr),
           CSA_ERR_UNSUPPORTED);
    EXPECT(csa_index_topk(A, F, A, 2, 8, 0, 64, 64, 128, 4, 8, mx, I, FO, A, need, nullptr), CSA_ERR_UNSUPPORTED);
    EXPECT(csa_index_topk(A, F, A, 32, 1, -1, 32768, 64, 128, 4, 1024, fp8, I, FO, A, need, nullptr),
           CSA_ERR_INVALID_ARG);
    EXPECT(csa_index_topk_noalloc(A, F, A, 1, 8192, 0, 2048, 64, 128, 4, 512, bf16, I, FO, nullptr),
           CSA_ERR_TOO_LARGE);
    EXPECT(csa_index_topk_noalloc(nullptr, F, A, 1, 8, 0, 64, 64, 128, 4, 8, bf16, I, FO, nullptr),
           CSA_ERR_INVALID_ARG);
    EXPECT(csa_index_scores(A, F, A, 1, 4, 0, 64, 0, 128, 4, bf16, FO, nullptr), CSA_ERR_INVALID_ARG);
    EXPECT(csa_topk(F, 62, 1, 4, 0, 64, 4, 8, I, FO, A, 1 << 20, nullptr), CSA_ERR_INVALID_ARG);
    EXPECT(csa_topk(F, 64, 1, 4, 0, 64, 4, 8, I, static_cast<float*>(MIS), A, 1 << 20, nullptr), CSA_ERR_INVALID_ARG);

    // attention
    EXPECT(csa_sparse_mqa(A, A, I, 1, 4, 64, 4, 64, 8, 0.125f, f32, nullptr, nullptr, 0, nullptr), CSA_ERR_INVALID_ARG);
    EXPECT(csa_sparse_mqa(A, A, I, 1, 4, 64, 4, 64, 8, 1.0f / 0.0f, f32, A, nullptr, 0, nullptr), CSA_ERR_INVALID_ARG);
    EXPECT(csa_sparse_mqa(A, A, I, 1, 4, 64, 4, 56, 8, 0.125f, mix, A, A, 1 << 30, nullptr), CSA_ERR_UNSUPPORTED);
    EXPECT(csa_sparse_mqa(A, A, I, 32, 1, 32768, 128, 512, 1024, 0.05f, bf16, A, nullptr, 0, nullptr),
           CSA_ERR_WORKSPACE);
    EXPECT(csa_sparse_mqa_swa(A, A, I, 1, 4, 64, 4, 64, 8, 0.125f, nullptr, nullptr, 16, 0, 0, 8, f32, A, nullptr, 0,
                              nullptr),
           CSA_ERR_INVALID_ARG);
    EXPECT(csa_sparse_mqa_sink(A, A, I, 1, 4, 64, 4, 64, 8, 0.125f, reinterpret_cast<const float*>(0x10002), f32, A,
                               nullptr, 0, nullptr),
           CSA_ERR_INVALID_ARG);
    EXPECT(hca_dense_mqa(A, A, 1, 4, 0, 8, 4, 64, 0, 0.125f, f32, A, nullptr), CSA_ERR_INVALID_ARG);
    EXPECT(hca_dense_mqa_swa(A, A, 1, 4, 0, 8, 4, 64, 128, 0.1f, nullptr, MIS, 16, 0, 8, f32, A, nullptr),
           CSA_ERR_INVALID_ARG);
    EXPECT(hca_dense_mqa_swa(A, A, 1, 4, 0, 8, 4, 64, 128, 0.1f, nullptr, A, 16, 0, 4096, f32, A, nullptr),
           CSA_ERR_UNSUPPORTED);
    EXPECT(csa_rope(A, 1, 4, 4, 64, 3, 0, 1, 10000.f, 0, f32, nullptr), CSA_ERR_INVALID_ARG);
    EXPECT(csa_rope(A, 1, 4, 4, 64, 64, 0, 1, 1.0f, 0, f32, nullptr), CSA_ERR_INVALID_ARG);

    // workspace sizes over a range of shapes, large ones included (no overflow in the arithmetic)
    size_t acc = 0;
    for (int64_t rows = 1; rows <= (int64_t(1) << 20); rows *= 8)
        for (int64_t N = 1; N < (int64_t(1) << 28); N = N * 7 + 3) {
            acc += csa_index_topk_workspace_size(rows, 1, N, 64, 2048);
            acc += csa_index_topk_workspace_size(1, rows, N, 64, 512);
            acc += csa_topk_workspace_size(rows, 1, N, 1024);
            acc += csa_sparse_mqa_workspace_size(rows, 1, 256, 512, 2048, bf16);
        }
    EXPECT(csa_index_topk_workspace_size(-1, 1, 10, 1, 1) == 0 ? 0 : 1, 0);
    printf("abi checks: %d failures (workspace sizes summed: %zu)\n", fails, acc);
    return fails != 0;
}
