// Sanitizer driver for the host code of the C ABI (api.cpp, built with g++
// -fsanitize=address,undefined by tests/test_sanitize.py; test
// infrastructure only).  The kernel launchers are replaced by stubs that
// abort: every call made here must be settled on the host (argument checks,
// planning, the chunk and tail-split rules, the route table, knobs, status
// strings), none may reach the GPU.  Prints "ok" and returns 0 when every
// call returned the expected status.
#include <cstdio>
#include <cstdlib>

#include "drgg.h"
#include "internal.hpp"

namespace drgg {
[[noreturn]] static void no_gpu(const char* what) {
    std::fprintf(stderr, "host-only driver reached the launcher %s\n", what);
    std::abort();
}
hipError_t launch_fwd_dgrad(int, int, const GemmArgs&, bool, hipStream_t) { no_gpu("fwd/dgrad"); }
hipError_t launch_transpose_w(const uint16_t*, uint16_t*, int32_t, int64_t, int64_t, hipStream_t) {
    no_gpu("transpose");
}
hipError_t launch_wgrad_det(int, const GemmArgs&, bool, hipStream_t) { no_gpu("wgrad det"); }
hipError_t launch_wgrad_atomic(int, const GemmArgs&, int64_t, bool, hipStream_t) { no_gpu("wgrad split"); }
hipError_t launch_router(const float*, const float*, float*, int64_t, int64_t, int64_t, hipStream_t) {
    no_gpu("router");
}
hipError_t launch_router_ks(const float*, const float*, float*, float*, int64_t, int64_t, int64_t, int64_t, int64_t,
                            hipStream_t) {
    no_gpu("router ks");
}
hipError_t launch_zero(void*, size_t, hipStream_t) { no_gpu("zero"); }
hipError_t launch_hold_cus(int, uint64_t, hipStream_t) { no_gpu("hold"); }
hipError_t scratch_buffer(void**) { no_gpu("scratch"); }
}  // namespace drgg

static int fails = 0;
#define EXPECT(call, want)                                                                   \
    do {                                                                                     \
        const int got_ = (int)(call);                                                        \
        if (got_ != (int)(want)) {                                                           \
            std::fprintf(stderr, "line %d: %s returned %d, expected %d\n", __LINE__, #call, got_, \
                         (int)(want));                                                       \
            ++fails;                                                                         \
        }                                                                                    \
    } while (0)

int main() {
    void* const A = reinterpret_cast<void*>(0x10000);   // fake, aligned, never dereferenced
    const int32_t* const O = static_cast<const int32_t*>(A);
    char* const Ac = static_cast<char*>(A);
    // argument checks of the three programs
    EXPECT(grouped_gemm_fwd(A, A, O, 0, 64, 64, 64, DRGG_FP32, 1, A, nullptr, 0, nullptr), DRGG_EINVAL);
    EXPECT(grouped_gemm_fwd(A, A, O, 1025, 64, 64, 64, DRGG_FP32, 1, A, nullptr, 0, nullptr), DRGG_EINVAL);
    EXPECT(grouped_gemm_fwd(A, A, O, 2, -1, 64, 64, DRGG_FP32, 1, A, nullptr, 0, nullptr), DRGG_ESHAPE);
    EXPECT(grouped_gemm_fwd(A, A, O, 2, 64, 12, 64, DRGG_FP32, 1, A, nullptr, 0, nullptr), DRGG_EALIGN);
    EXPECT(grouped_gemm_fwd(Ac + 2, A, O, 2, 64, 64, 64, DRGG_FP32, 1, A, nullptr, 0, nullptr), DRGG_EALIGN);
    EXPECT(grouped_gemm_fwd(A, A, O, 2, int64_t(1) << 31, 64, 64, DRGG_FP32, 1, A, nullptr, 0, nullptr),
           DRGG_ESHAPE);
    EXPECT(grouped_gemm_dgrad(A, nullptr, O, 2, 64, 64, 64, DRGG_BF16, 1, A, nullptr, 0, nullptr), DRGG_EINVAL);
    EXPECT(grouped_gemm_dgrad(A, A, O, 2, 64, (int64_t(1) << 22) + 8, 64, DRGG_BF16, 1, A, nullptr, 0, nullptr),
           DRGG_ESHAPE);
    EXPECT(grouped_gemm_wgrad(A, A, O, 2, 100000, 256, 256, DRGG_FP32, 1, A, nullptr, 0, nullptr), DRGG_EWORKSPACE);
    EXPECT(grouped_gemm_wgrad(A, A, nullptr, 2, 64, 64, 64, DRGG_FP32, 1, A, A, 1 << 20, nullptr), DRGG_EINVAL);
    EXPECT(grouped_gemm_wgrad(A, A, O, 2, 64, 64, 64, (drgg_dtype)5, 1, A, A, 1 << 20, nullptr), DRGG_EINVAL);
    // the no-allocation weight gradient: refused on the host
    EXPECT(grouped_gemm_wgrad_noalloc(A, A, nullptr, 2, 64, 64, 64, DRGG_FP32, 1, A, nullptr), DRGG_EINVAL);
    EXPECT(grouped_gemm_wgrad_noalloc(A, A, O, 8, 131072, 1536, 2048, DRGG_BF16, 1, A, nullptr), DRGG_EWORKSPACE);
    EXPECT(grouped_gemm_wgrad_noalloc(A, A, O, 2, 64, 12, 64, DRGG_FP32, 1, A, nullptr), DRGG_EALIGN);
    // batched
    drgg_batched b{4, 64, 64, 64, 64, 64 * 64, 64, 64 * 64, 64, 64 * 64};
    drgg_batched bad = b;
    bad.a_row = 60;
    EXPECT(batched_gemm_fwd(A, A, &bad, DRGG_BF16, A, nullptr), DRGG_ESHAPE);
    bad = b;
    bad.o_batch = 64 * 32;
    EXPECT(batched_gemm_fwd(A, A, &bad, DRGG_BF16, A, nullptr), DRGG_ESHAPE);
    bad = b;
    bad.a_batch = int64_t(1) << 61;
    EXPECT(batched_gemm_dgrad(A, A, &bad, DRGG_BF16, A, nullptr, 0, nullptr), DRGG_EOVERFLOW);
    EXPECT(batched_gemm_wgrad(A, A, nullptr, DRGG_BF16, 1, A, nullptr, 0, nullptr), DRGG_EINVAL);
    // router
    EXPECT(router_gemm_fp32_bf16x3(nullptr, static_cast<float*>(A), 16, 16, 16, static_cast<float*>(A), nullptr),
           DRGG_EINVAL);
    EXPECT(router_gemm_fp32_bf16x3(static_cast<float*>(A), static_cast<float*>(A), 16, (1 << 22) + 4, 16,
                                   static_cast<float*>(A), nullptr),
           DRGG_ESHAPE);
    {
        size_t rw = 0;
        EXPECT(router_workspace_size(2048, 256, 4096, &rw), DRGG_OK);
        EXPECT(rw == size_t(7) * 2048 * 256 * 4 ? DRGG_OK : DRGG_EINVAL, DRGG_OK);
        EXPECT(router_workspace_size(16384, 256, 4096, &rw), DRGG_OK);
        EXPECT(rw == 0 ? DRGG_OK : DRGG_EINVAL, DRGG_OK);
        EXPECT(router_gemm_fp32_bf16x3_ws(static_cast<float*>(A), static_cast<float*>(A), 2048, 256, 4096,
                                          static_cast<float*>(A), nullptr, 0, nullptr),
               DRGG_EWORKSPACE);
        int64_t ks = 0, kq = 0;
        for (int64_t M : {1, 255, 256, 16384, 65536})
            for (int64_t K : {8, 200, 4096, 4104}) {
                EXPECT(drgg_router_split(M, 256, K, &ks, &kq), DRGG_OK);
                const bool single = ks == 0 && kq == K;
                const bool sliced = ks >= 1 && ks <= 8 && kq % 32 == 0 && (ks - 1) * kq < K && ks * kq >= K;
                EXPECT(single || sliced ? DRGG_OK : DRGG_EINVAL, DRGG_OK);
            }
    }
    // planning and the rules behind it, for a range of shapes and CU counts
    const int64_t shapes[][4] = {{8, 131072, 1536, 2048}, {32, 131072, 2048, 768}, {1, 16384, 48, 4096},
                                 {1, 16384, 4096, 4096}, {4, 512, 512, 256},     {1024, 3000, 8, 8},
                                 {3, 0, 64, 64}};
    for (const auto& s : shapes)
        for (int op = 0; op < 3; ++op)
            for (int det = 0; det < 2; ++det)
                for (int cus : {1, 80, 256, 304}) {
                    drgg_plan_info info;
                    EXPECT(drgg_plan((drgg_op)op, (int32_t)s[0], s[1], s[2], s[3], DRGG_BF16, det, cus, &info),
                           DRGG_OK);
                    size_t ws = 0;
                    EXPECT(grouped_gemm_workspace_size((drgg_op)op, (int32_t)s[0], s[1], s[2], s[3], DRGG_FP32, det,
                                                       cus, &ws),
                           DRGG_OK);
                }
    for (int64_t T = 0; T < 5000; T += 37) {
        int64_t len = 0, n = 0;
        EXPECT(drgg_wgrad_chunking(T, 512, &len, &n), DRGG_OK);
    }
    int64_t len = 0, n = 0;
    EXPECT(drgg_wgrad_chunking(100, 100, &len, &n), DRGG_EINVAL);
    int64_t t4[4];
    EXPECT(drgg_tailsplit_units(1296, 76, t4), DRGG_OK);
    if (t4[1] != 1300 || t4[3] != 2) ++fails;
    EXPECT(drgg_tailsplit_units(10, 0, t4), DRGG_EINVAL);
    // route table and knobs
    EXPECT(drgg_route_clear(), DRGG_OK);
    EXPECT(drgg_route_split(4, 512, 512, 256, DRGG_FP32), DRGG_OK);
    EXPECT(drgg_route_count(), 1);
    for (int i = 0; i < 300; ++i) drgg_route_split(2, 64 * (i + 1), 64, 64, DRGG_BF16);
    EXPECT(drgg_route_count(), 256);
    EXPECT(drgg_route_split(3, 64, 64, 64, DRGG_BF16), DRGG_EUNSUPPORTED);
    EXPECT(drgg_route_clear(), DRGG_OK);
    for (int k = 1; k <= 7; ++k) {
        EXPECT(drgg_set_knob(k, 1), DRGG_OK);
        EXPECT(drgg_set_knob(k, 0), DRGG_OK);
    }
    EXPECT(drgg_set_knob(99, 0), DRGG_EINVAL);
    EXPECT(drgg_timing_count(), 0);
    const char* name = nullptr;
    float ms = 0;
    EXPECT(drgg_timing_read(0, &name, &ms), DRGG_EINVAL);
    for (int s = 0; s < 9; ++s)
        if (!drgg_status_string((drgg_status)s)) ++fails;
    EXPECT(drgg_abi_version(), DRGG_ABI_VERSION);
    if (fails) return 1;
    std::printf("ok\n");
    return 0;
}
