// Calls every entry point of libpath_attn (include/path_attn.h) with invalid
// arguments, the workspace-size queries with valid and invalid descriptions,
// and the status helpers, so that a build of the host code (csrc/host.cpp)
// with AddressSanitizer and UndefinedBehaviorSanitizer can check the
// validation paths.  No device memory is touched: every call here must fail
// validation before anything is enqueued, which the driver also asserts.
// Test infrastructure only.
#include "path_attn.h"

#include <stdint.h>
#include <stdio.h>
#include <string.h>

static int failures = 0;

#define EXPECT(cond)                                                   \
    do {                                                               \
        if (!(cond)) {                                                 \
            fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond);  \
            ++failures;                                                \
        }                                                              \
    } while (0)

// Aligned addresses that are never dereferenced (validation fails first).
static void* const F = (void*)(uintptr_t)(1u << 20);
static float* const FF = (float*)(uintptr_t)(1u << 20);
static void* const ODD = (void*)(uintptr_t)((1u << 20) + 2);

static path_fwd_desc desc(int N, int H, int L, int d, path_dtype t, int block) {
    path_fwd_desc x;
    x.N = N; x.H = H; x.L = L; x.d = d; x.dtype = t; x.scale = 1.0f; x.block = block;
    return x;
}

int main() {
    EXPECT(path_abi_version() == PATH_ATTN_ABI_VERSION);
    for (int s = 0; s <= 9; ++s) EXPECT(path_status_str((path_status)s) != nullptr);
    EXPECT(path_status_str((path_status)-3) != nullptr);
    EXPECT(path_last_error() != nullptr);

    // workspace queries over a range of valid and invalid descriptions
    const int Ls[] = {1, 63, 64, 65, 4096, 8388608, 8388609, 0, -5};
    const int ds[] = {16, 32, 48, 64, 128};
    const int blocks[] = {0, 16, 32, 64, 8};
    for (int L : Ls)
        for (int d : ds)
            for (int b : blocks)
                for (int t = 0; t < 3; ++t) {
                    path_fwd_desc x = desc(3, 5, L, d, (path_dtype)t, b);
                    (void)path_attn_fwd_workspace(&x, 0);
                    (void)path_attn_fwd_workspace(&x, 1);
                    (void)path_attn_bwd_workspace(&x);
                    (void)path_decode_workspace(&x, L);
                    (void)path_paged_decode_workspace(&x, L);
                }
    EXPECT(path_attn_fwd_workspace(nullptr, 0) == 0);
    EXPECT(path_attn_bwd_workspace(nullptr) == 0);

    path_fwd_desc g = desc(2, 3, 200, 64, PATH_BF16, 0);
    size_t need = path_attn_fwd_workspace(&g, 1);
    EXPECT(need > 0);
    path_cache c{150, PATH_BF16, F, F, nullptr};
    EXPECT(path_attn_fwd(&g, F, F, F, F, FF, nullptr, F, nullptr, &c, F, need, nullptr) ==
           PATH_E_CAPACITY);
    EXPECT(path_attn_fwd(&g, F, F, F, F, FF, nullptr, F, nullptr, nullptr, F, 16, nullptr) ==
           PATH_E_WORKSPACE);
    EXPECT(path_attn_fwd(&g, ODD, F, F, F, FF, nullptr, F, nullptr, nullptr, F, need, nullptr) ==
           PATH_E_ALIGN);
    hipEvent_t ev[4] = {nullptr, nullptr, nullptr, nullptr};
    EXPECT(path_attn_fwd_timed(&g, F, F, F, F, FF, nullptr, F, nullptr, nullptr, F, need,
                               nullptr, ev) == PATH_E_NULL);
    EXPECT(strlen(path_last_error()) > 0);

    size_t bneed = path_attn_bwd_workspace(&g);
    EXPECT(bneed > 0);
    EXPECT(path_attn_bwd(&g, F, F, F, F, FF, FF, F, FF, F, F, F, F, F, FF, nullptr, F, bneed,
                         nullptr) == PATH_E_NULL);
    EXPECT(path_attn_bwd(&g, F, F, F, F, FF, nullptr, F, FF, F, F, F, F, F, FF, nullptr, F,
                         bneed - 1, nullptr) == PATH_E_WORKSPACE);

    path_cache small{8, PATH_BF16, F, F, nullptr};
    size_t dws = path_decode_workspace(&g, 8);
    EXPECT(dws > 0);
    EXPECT(path_kv_update(&g, &small, 9, F, FF, nullptr) == PATH_E_CAPACITY);
    EXPECT(path_kv_append(&g, &small, 8, F, F, nullptr, nullptr) == PATH_E_CAPACITY);
    EXPECT(path_decode(&g, &small, 9, F, F, nullptr, F, dws, nullptr) == PATH_E_CAPACITY);
    EXPECT(path_decode_step(&g, &small, 8, F, F, F, F, FF, nullptr, F, nullptr, F, dws,
                            nullptr) == PATH_E_CAPACITY);
    EXPECT(path_decode_step(&g, &small, 2, F, F, F, F, FF, nullptr, F, nullptr, F, 4, nullptr) ==
           PATH_E_WORKSPACE);

    // the allocation-free step: validation, then the scratch size limit
    EXPECT(path_decode_step_noalloc_limit() == ((size_t)16 << 20));
    EXPECT(path_decode_step_noalloc(&g, &small, 8, F, F, F, F, FF, nullptr, F, nullptr,
                                    nullptr) == PATH_E_CAPACITY);
    path_fwd_desc huge = desc(64, 64, 1, 64, PATH_BF16, 0);
    path_cache bigc{131072, PATH_BF16, F, F, nullptr};
    EXPECT(path_decode_step_noalloc(&huge, &bigc, 131071, F, F, F, F, FF, nullptr, F, nullptr,
                                    nullptr) == PATH_E_WORKSPACE);

    path_paged_cache pc{8, 64, PATH_BF16, F, F, nullptr};
    path_fwd_desc s3 = desc(3, 2, 1, 64, PATH_BF16, 0);
    size_t pws = path_paged_decode_workspace(&s3, 256);
    EXPECT(pws > 0);
    int* IP = (int*)F;
    EXPECT(path_paged_decode_step(&s3, &pc, IP, 4, IP, 257, F, F, F, F, FF, nullptr, F, nullptr,
                                  F, pws, nullptr) == PATH_E_SHAPE);
    EXPECT(path_paged_decode_step(&s3, &pc, IP, 4, IP, 256, F, F, F, F, FF, nullptr, F, nullptr,
                                  F, pws - 1, nullptr) == PATH_E_WORKSPACE);
    path_cache src{512, PATH_F32, F, F, nullptr};
    EXPECT(path_paged_import(&s3, &src, &pc, IP, 4, IP, 256, nullptr) == PATH_E_DTYPE);

    EXPECT(path_causal_attn_fwd(&g, nullptr, F, F, F, nullptr, nullptr) == PATH_E_NULL);
    path_fwd_desc f32 = desc(1, 1, 64, 64, PATH_F32, 0);
    EXPECT(path_causal_attn_fwd(&f32, F, F, F, F, nullptr, nullptr) == PATH_E_UNSUPPORTED);

    path_param_desc p{1, 64, 64, 16, 2, 64, PATH_BF16};
    size_t prm = path_param_workspace(&p, 1);
    EXPECT(prm > 0);
    EXPECT(path_param_fwd(&p, F, F, F, FF, F, FF, nullptr, FF, F, FF, FF, F, prm, nullptr) ==
           PATH_E_NULL);
    path_param_desc bad{1, 64, 40, 16, 2, 64, PATH_BF16};
    EXPECT(path_param_workspace(&bad, 1) == 0);

    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("abi sanitizer driver: ok\n");
    return 0;
}
