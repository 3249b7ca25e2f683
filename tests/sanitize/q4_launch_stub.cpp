// q4_launch_stub.cpp -- host-only stand-ins for the launchers behind the C
// ABI, for building q4_api.cpp on the CPU under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Each launcher records its name and shape and
// returns success without touching a device; the tests read the record back
// to check that a valid call reaches the right launcher with its arguments.
// Test infrastructure only: nothing here is part of libq4.so.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "q4_internal.h"

namespace {
char g_last[256];
int g_calls = 0;

hipError_t note(const char *fmt, long long a, long long b, long long c) {
    snprintf(g_last, sizeof g_last, fmt, a, b, c);
    ++g_calls;
    return hipSuccess;
}
}  // namespace

extern "C" int q4stub_calls(void) { return g_calls; }
extern "C" const char *q4stub_last(void) { return g_last; }

namespace q4 {

hipError_t launch_pack(const float *, int64_t M, int64_t K, uint8_t *, uint16_t *, int32_t *, hipStream_t) {
    return note("pack M=%lld K=%lld%.0lld", M, K, 0);
}
bool gemv_tokens_fits(int64_t, int64_t, int64_t) { return false; }
hipError_t launch_gemv_tokens(const uint8_t *, const uint16_t *, int64_t M, int64_t K, const uint16_t *, int64_t N,
                              float *, hipStream_t) {
    return note("gemv_tokens M=%lld K=%lld N=%lld", M, K, N);
}
hipError_t launch_gemv(const uint8_t *, const uint16_t *, int64_t M, int64_t K, const uint16_t *, float *,
                       hipStream_t) {
    return note("gemv M=%lld K=%lld%.0lld", M, K, 0);
}
hipError_t launch_pack_affine(const float *, int64_t M, int64_t K, uint8_t *, uint16_t *, uint16_t *, int32_t *,
                              hipStream_t) {
    return note("pack_affine M=%lld K=%lld%.0lld", M, K, 0);
}
hipError_t launch_gemv_affine(const uint8_t *, const uint16_t *, const uint16_t *, int64_t M, int64_t K,
                              const uint16_t *, float *, hipStream_t) {
    return note("gemv_affine M=%lld K=%lld%.0lld", M, K, 0);
}
hipError_t launch_quantize_x8(const uint16_t *, int64_t K, int words, int8_t *, int8_t *, float *, hipStream_t) {
    return note("quantize_x8 K=%lld words=%lld%.0lld", K, words, 0);
}
hipError_t launch_gemv_affine_x8(const uint8_t *, const uint16_t *, const uint16_t *, int64_t M, int64_t K,
                                 const int8_t *, const int8_t *q2, const float *, float *, hipStream_t) {
    return note("gemv_affine_x8 M=%lld K=%lld words=%lld", M, K, q2 ? 2 : 1);
}
hipError_t launch_pack_nvfp4(const float *, int64_t M, int64_t K, uint8_t *, uint8_t *, float *, int32_t *,
                             hipStream_t) {
    return note("pack_nvfp4 M=%lld K=%lld%.0lld", M, K, 0);
}
hipError_t launch_gemv_nvfp4(const uint8_t *, const uint8_t *, const float *, int64_t M, int64_t K,
                             const uint16_t *, float *, hipStream_t) {
    return note("gemv_nvfp4 M=%lld K=%lld%.0lld", M, K, 0);
}
hipError_t launch_gemv_fused(int fmt, const FusedOperand *ops, int count, bool swiglu, int64_t K, const uint16_t *,
                             float *const *, const float *const *, hipStream_t) {
    long long rows = 0;
    for (int i = 0; i < count; ++i) rows += ops[i].M;
    if (fmt == kGemmAffine)
        return note(swiglu ? "gemv_fused_affine swiglu count=%lld K=%lld rows=%lld"
                           : "gemv_fused_affine count=%lld K=%lld rows=%lld",
                    count, K, rows);
    if (fmt == kGemmNvfp4)
        return note(swiglu ? "gemv_fused_nvfp4 swiglu count=%lld K=%lld rows=%lld"
                           : "gemv_fused_nvfp4 count=%lld K=%lld rows=%lld",
                    count, K, rows);
    return note(swiglu ? "gemv_fused swiglu count=%lld K=%lld rows=%lld" : "gemv_fused count=%lld K=%lld rows=%lld",
                count, K, rows);
}
hipError_t launch_gemm_smalln(const uint8_t *, const uint16_t *, int64_t M, int64_t K, const uint16_t *, int64_t N,
                              float *, hipStream_t) {
    return note("gemm_smalln M=%lld K=%lld N=%lld", M, K, N);
}
hipError_t launch_gemm_smalln_ws(const uint8_t *, const uint16_t *, int64_t M, int64_t K, const uint16_t *,
                                 int64_t N, float *, float *, hipStream_t) {
    return note("gemm_smalln_ws M=%lld K=%lld N=%lld", M, K, N);
}
hipError_t launch_gemm_smalln_affine_ws(const uint8_t *, const uint16_t *, const uint16_t *, int64_t M, int64_t K,
                                        const uint16_t *, int64_t N, float *, float *, hipStream_t) {
    return note("gemm_smalln_affine_ws M=%lld K=%lld N=%lld", M, K, N);
}
hipError_t launch_gemm_smalln_nvfp4_ws(const uint8_t *, const uint8_t *, const float *, int64_t M, int64_t K,
                                       const uint16_t *, int64_t N, float *, float *, hipStream_t) {
    return note("gemm_smalln_nvfp4_ws M=%lld K=%lld N=%lld", M, K, N);
}
hipError_t launch_gemm_smalln_noalloc(const uint8_t *, const uint16_t *, int64_t M, int64_t K, const uint16_t *,
                                      int64_t N, float *, hipStream_t) {
    return note("gemm_smalln_noalloc M=%lld K=%lld N=%lld", M, K, N);
}
hipError_t launch_gemm_smalln_affine(const uint8_t *, const uint16_t *, const uint16_t *, int64_t M, int64_t K,
                                     const uint16_t *, int64_t N, float *, hipStream_t) {
    return note("gemm_smalln_affine M=%lld K=%lld N=%lld", M, K, N);
}
hipError_t launch_gemm_smalln_nvfp4(const uint8_t *, const uint8_t *, const float *, int64_t M, int64_t K,
                                    const uint16_t *, int64_t N, float *, hipStream_t) {
    return note("gemm_smalln_nvfp4 M=%lld K=%lld N=%lld", M, K, N);
}
hipError_t launch_gather_rows(const uint8_t *, const uint16_t *, int64_t M, int64_t K, const int32_t *, int64_t n,
                              bool bf16, void *, int32_t *, hipStream_t) {
    return note(bf16 ? "gather_rows_bf16 M=%lld K=%lld n=%lld" : "gather_rows_f32 M=%lld K=%lld n=%lld", M, K, n);
}

}  // namespace q4
