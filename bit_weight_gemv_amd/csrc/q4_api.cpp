// q4_api.cpp -- the exported C ABI (declared in include/q4.h): argument
// checks on the host, then one launch on the caller's stream.
//
// Conventions (golang.design accel/tensor, Builder/Plan documentation): the
// caller owns every buffer it names; everything is validated before anything
// is launched, and a call refuses bad arguments instead of clamping them; the
// counts are passed explicitly because a buffer's size cannot give them.
#include "q4.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q4_device.h"
#include "q4_internal.h"

namespace {

// (A null pointer counts as aligned.)
bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void *p, uint64_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return {a, a + (uintptr_t)bytes};
}

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

// K must be a positive multiple of 64 up to Q4_MAX_K; M >= 0 and M*K must
// leave headroom in 64-bit byte counts.
bool shape_ok(int64_t M, int64_t K) {
    if (M < 0 || K <= 0 || K % 64 != 0 || K > Q4_MAX_K) return false;
    if (M > (INT64_C(1) << 62) / K) return false;
    return true;
}

int launch_status(hipError_t e) { return e == hipSuccess ? Q4_OK : Q4_ERR_DEVICE; }

}  // namespace

extern "C" {

size_t q4_codes_bytes(int64_t M, int64_t K) { return shape_ok(M, K) ? (size_t)(M * (K / 2)) : 0; }

size_t q4_scales_bytes(int64_t M, int64_t K) {
    return shape_ok(M, K) ? (size_t)(M * (K / 64) * 2) : 0;
}

void q4_codebook(float out[16]) {
    if (!out) return;
    for (int i = 0; i < 16; ++i) out[i] = q4::level_f32(i);
}

const char *q4_status_string(int status) {
    switch (status) {
        case Q4_OK: return "Q4_OK";
        case Q4_ERR_NULL: return "Q4_ERR_NULL: a required pointer is NULL";
        case Q4_ERR_SHAPE: return "Q4_ERR_SHAPE: bad M, K or N";
        case Q4_ERR_ALIGN: return "Q4_ERR_ALIGN: a pointer is not aligned as required";
        case Q4_ERR_OVERLAP: return "Q4_ERR_OVERLAP: an output range overlaps another range";
        case Q4_ERR_DEVICE: return "Q4_ERR_DEVICE: the HIP runtime refused the launch";
        case Q4_ERR_WORKSPACE: return "Q4_ERR_WORKSPACE: the scratch memory for partial sums is missing or too small";
        default: return "unknown q4 status";
    }
}

int q4_pack(const float *W, int64_t M, int64_t K, uint8_t *codes, uint16_t *scales, int32_t *status,
            void *stream) {
    if (!shape_ok(M, K)) return Q4_ERR_SHAPE;
    if (!W || !codes || !scales || !status) return Q4_ERR_NULL;
    if (!aligned(W, 16) || !aligned(codes, 16) || !aligned(scales, 2) || !aligned(status, 4))
        return Q4_ERR_ALIGN;
    const Range rw = range_of(W, (uint64_t)M * K * 4);
    const Range rc = range_of(codes, (uint64_t)M * (K / 2));
    const Range rs = range_of(scales, (uint64_t)M * (K / 64) * 2);
    const Range rst = range_of(status, 4);
    if (overlap(rc, rw) || overlap(rs, rw) || overlap(rst, rw) || overlap(rc, rs) || overlap(rc, rst) ||
        overlap(rs, rst))
        return Q4_ERR_OVERLAP;
    // M == 0 still clears the status word: the call's contract is that
    // *status holds the flags of this call.
    return launch_status(q4::launch_pack(W, M, K, codes, scales, status, (hipStream_t)stream));
}

int q4_unpack_canonical(const uint8_t *codes, const uint16_t *scales, int64_t M, int64_t K, uint8_t *codes_out,
                        uint16_t *scales_out, void *stream) {
    if (!shape_ok(M, K)) return Q4_ERR_SHAPE;
    if (M == 0) return Q4_OK;
    if (!codes || !scales || !codes_out || !scales_out) return Q4_ERR_NULL;
    if (!aligned(codes, 16) || !aligned(scales, 2) || !aligned(codes_out, 16) || !aligned(scales_out, 2))
        return Q4_ERR_ALIGN;
    const uint64_t cb = (uint64_t)M * (K / 2), sb = (uint64_t)M * (K / 64) * 2;
    const Range r[4] = {range_of(codes, cb), range_of(scales, sb), range_of(codes_out, cb),
                        range_of(scales_out, sb)};
    for (int i = 0; i < 4; ++i)
        for (int j = i + 1; j < 4; ++j)
            if (overlap(r[i], r[j])) return Q4_ERR_OVERLAP;
    // The device layout is the canonical layout: copy both arrays.
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = hipMemcpyAsync(codes_out, codes, cb, hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess) e = hipMemcpyAsync(scales_out, scales, sb, hipMemcpyDeviceToDevice, s);
    return launch_status(e);
}

int q4_gemv(const uint8_t *codes, const uint16_t *scales, int64_t M, int64_t K, const uint16_t *x,
            float *y, void *stream) {
    if (!shape_ok(M, K)) return Q4_ERR_SHAPE;
    if (M == 0) return Q4_OK;
    if (!codes || !scales || !x || !y) return Q4_ERR_NULL;
    if (!aligned(codes, 16) || !aligned(scales, 2) || !aligned(x, 16) || !aligned(y, 4))
        return Q4_ERR_ALIGN;
    const Range ry = range_of(y, (uint64_t)M * 4);
    if (overlap(ry, range_of(codes, (uint64_t)M * (K / 2))) ||
        overlap(ry, range_of(scales, (uint64_t)M * (K / 64) * 2)) || overlap(ry, range_of(x, (uint64_t)K * 2)))
        return Q4_ERR_OVERLAP;
    return launch_status(q4::launch_gemv(codes, scales, M, K, x, y, (hipStream_t)stream));
}

int q4_pack_affine(const float *W, int64_t M, int64_t K, uint8_t *codes, uint16_t *scales, uint16_t *zeros,
                   int32_t *status, void *stream) {
    if (!shape_ok(M, K)) return Q4_ERR_SHAPE;
    if (!W || !codes || !scales || !zeros || !status) return Q4_ERR_NULL;
    if (!aligned(W, 16) || !aligned(codes, 16) || !aligned(scales, 2) || !aligned(zeros, 2) || !aligned(status, 4))
        return Q4_ERR_ALIGN;
    const uint64_t sb = (uint64_t)M * (K / 64) * 2;
    const Range r[5] = {range_of(W, (uint64_t)M * K * 4), range_of(codes, (uint64_t)M * (K / 2)), range_of(scales, sb),
                        range_of(zeros, sb), range_of(status, 4)};
    for (int i = 0; i < 5; ++i)
        for (int j = i + 1; j < 5; ++j)
            if (overlap(r[i], r[j])) return Q4_ERR_OVERLAP;
    return launch_status(q4::launch_pack_affine(W, M, K, codes, scales, zeros, status, (hipStream_t)stream));
}

int q4_gemv_affine(const uint8_t *codes, const uint16_t *scales, const uint16_t *zeros, int64_t M, int64_t K,
                   const uint16_t *x, float *y, void *stream) {
    if (!shape_ok(M, K)) return Q4_ERR_SHAPE;
    if (M == 0) return Q4_OK;
    if (!codes || !scales || !zeros || !x || !y) return Q4_ERR_NULL;
    if (!aligned(codes, 16) || !aligned(scales, 2) || !aligned(zeros, 2) || !aligned(x, 16) || !aligned(y, 4))
        return Q4_ERR_ALIGN;
    const Range ry = range_of(y, (uint64_t)M * 4);
    const uint64_t sb = (uint64_t)M * (K / 64) * 2;
    if (overlap(ry, range_of(codes, (uint64_t)M * (K / 2))) || overlap(ry, range_of(scales, sb)) ||
        overlap(ry, range_of(zeros, sb)) || overlap(ry, range_of(x, (uint64_t)K * 2)))
        return Q4_ERR_OVERLAP;
    return launch_status(q4::launch_gemv_affine(codes, scales, zeros, M, K, x, y, (hipStream_t)stream));
}

int q4_quantize_x8(const uint16_t *x, int64_t K, int words, int8_t *q1, int8_t *q2, float *d, void *stream) {
    if (!shape_ok(0, K) || (words != 1 && words != 2)) return Q4_ERR_SHAPE;
    if (!x || !q1 || !d || (words == 2 && !q2)) return Q4_ERR_NULL;
    if (!aligned(x, 16) || !aligned(q1, 16) || !aligned(q2, 16) || !aligned(d, 4)) return Q4_ERR_ALIGN;
    const Range rx = range_of(x, (uint64_t)K * 2), r1 = range_of(q1, (uint64_t)K),
                r2 = range_of(words == 2 ? q2 : nullptr, words == 2 ? (uint64_t)K : 0), rd = range_of(d, (uint64_t)K / 8);
    if (overlap(rx, r1) || overlap(rx, r2) || overlap(rx, rd) || overlap(r1, r2) || overlap(r1, rd) || overlap(r2, rd))
        return Q4_ERR_OVERLAP;
    return launch_status(q4::launch_quantize_x8(x, K, words, q1, words == 2 ? q2 : nullptr, d, (hipStream_t)stream));
}

int q4_gemv_affine_x8(const uint8_t *codes, const uint16_t *scales, const uint16_t *zeros, int64_t M, int64_t K,
                      const int8_t *q1, const int8_t *q2, const float *d, float *y, void *stream) {
    if (!shape_ok(M, K)) return Q4_ERR_SHAPE;
    if (M == 0) return Q4_OK;
    if (!codes || !scales || !zeros || !q1 || !d || !y) return Q4_ERR_NULL;
    if (!aligned(codes, 16) || !aligned(scales, 2) || !aligned(zeros, 2) || !aligned(q1, 16) || !aligned(q2, 16) ||
        !aligned(d, 4) || !aligned(y, 4))
        return Q4_ERR_ALIGN;
    const Range ry = range_of(y, (uint64_t)M * 4);
    const uint64_t sb = (uint64_t)M * (K / 64) * 2;
    if (overlap(ry, range_of(codes, (uint64_t)M * (K / 2))) || overlap(ry, range_of(scales, sb)) ||
        overlap(ry, range_of(zeros, sb)) || overlap(ry, range_of(q1, (uint64_t)K)) ||
        overlap(ry, range_of(q2, q2 ? (uint64_t)K : 0)) || overlap(ry, range_of(d, (uint64_t)K / 8)))
        return Q4_ERR_OVERLAP;
    return launch_status(q4::launch_gemv_affine_x8(codes, scales, zeros, M, K, q1, q2, d, y, (hipStream_t)stream));
}

int q4_pack_nvfp4(const float *W, int64_t M, int64_t K, uint8_t *codes, uint8_t *scales, float *tscale,
                  int32_t *status, void *stream) {
    if (!shape_ok(M, K)) return Q4_ERR_SHAPE;
    if (!W || !codes || !scales || !tscale || !status) return Q4_ERR_NULL;
    if (!aligned(W, 16) || !aligned(codes, 16) || !aligned(scales, 2) || !aligned(tscale, 4) || !aligned(status, 4))
        return Q4_ERR_ALIGN;
    const Range r[5] = {range_of(W, (uint64_t)M * K * 4), range_of(codes, (uint64_t)M * (K / 2)),
                        range_of(scales, (uint64_t)M * (K / 16)), range_of(tscale, 4), range_of(status, 4)};
    for (int i = 0; i < 5; ++i)
        for (int j = i + 1; j < 5; ++j)
            if (overlap(r[i], r[j])) return Q4_ERR_OVERLAP;
    return launch_status(q4::launch_pack_nvfp4(W, M, K, codes, scales, tscale, status, (hipStream_t)stream));
}

int q4_gemv_nvfp4(const uint8_t *codes, const uint8_t *scales, const float *tscale, int64_t M, int64_t K,
                  const uint16_t *x, float *y, void *stream) {
    if (!shape_ok(M, K)) return Q4_ERR_SHAPE;
    if (M == 0) return Q4_OK;
    if (!codes || !scales || !tscale || !x || !y) return Q4_ERR_NULL;
    if (!aligned(codes, 16) || !aligned(scales, 2) || !aligned(tscale, 4) || !aligned(x, 16) || !aligned(y, 4))
        return Q4_ERR_ALIGN;
    const Range ry = range_of(y, (uint64_t)M * 4);
    if (overlap(ry, range_of(codes, (uint64_t)M * (K / 2))) || overlap(ry, range_of(scales, (uint64_t)M * (K / 16))) ||
        overlap(ry, range_of(tscale, 4)) || overlap(ry, range_of(x, (uint64_t)K * 2)))
        return Q4_ERR_OVERLAP;
    return launch_status(q4::launch_gemv_nvfp4(codes, scales, tscale, M, K, x, y, (hipStream_t)stream));
}

int q4_gemm_smalln(const uint8_t *codes, const uint16_t *scales, int64_t M, int64_t K, const uint16_t *X,
                   int64_t N, float *Y, void *stream) {
    if (!shape_ok(M, K) || N < 0 || N > Q4_MAX_N) return Q4_ERR_SHAPE;
    if (M == 0 || N == 0) return Q4_OK;
    if (!codes || !scales || !X || !Y) return Q4_ERR_NULL;
    if (!aligned(codes, 16) || !aligned(scales, 2) || !aligned(X, 16) || !aligned(Y, 4))
        return Q4_ERR_ALIGN;
    const Range ry = range_of(Y, (uint64_t)N * M * 4);
    if (overlap(ry, range_of(codes, (uint64_t)M * (K / 2))) ||
        overlap(ry, range_of(scales, (uint64_t)M * (K / 64) * 2)) ||
        overlap(ry, range_of(X, (uint64_t)N * K * 2)))
        return Q4_ERR_OVERLAP;
    return launch_status(q4::launch_gemm_smalln(codes, scales, M, K, X, N, Y, (hipStream_t)stream));
}

size_t q4_gemm_smalln_ws_bytes(int64_t M, int64_t K, int64_t N) {
    if (!shape_ok(M, K) || M == 0 || N < 1 || N > Q4_MAX_N || !q4::gemm_split_fits(M, K, N)) return 0;
    return q4::gemm_split_bytes(M, K, N);
}

int q4_gemm_smalln_ws(const uint8_t *codes, const uint16_t *scales, int64_t M, int64_t K, const uint16_t *X,
                      int64_t N, float *Y, void *workspace, size_t workspace_bytes, void *stream) {
    if (!shape_ok(M, K) || N < 0 || N > Q4_MAX_N) return Q4_ERR_SHAPE;
    if (M == 0 || N == 0) return Q4_OK;
    if (!codes || !scales || !X || !Y) return Q4_ERR_NULL;
    if (!aligned(codes, 16) || !aligned(scales, 2) || !aligned(X, 16) || !aligned(Y, 4))
        return Q4_ERR_ALIGN;
    const Range ry = range_of(Y, (uint64_t)N * M * 4);
    const Range rc = range_of(codes, (uint64_t)M * (K / 2)), rs = range_of(scales, (uint64_t)M * (K / 64) * 2),
                rx = range_of(X, (uint64_t)N * K * 2);
    if (overlap(ry, rc) || overlap(ry, rs) || overlap(ry, rx)) return Q4_ERR_OVERLAP;
    const size_t need = q4_gemm_smalln_ws_bytes(M, K, N);
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return Q4_ERR_WORKSPACE;
        if (!aligned(workspace, 16)) return Q4_ERR_ALIGN;
        const Range rw = range_of(workspace, need);
        if (overlap(rw, ry) || overlap(rw, rc) || overlap(rw, rs) || overlap(rw, rx)) return Q4_ERR_OVERLAP;
    }
    return launch_status(q4::launch_gemm_smalln_ws(codes, scales, M, K, X, N, Y, static_cast<float *>(workspace),
                                                   (hipStream_t)stream));
}

int q4_gemm_smalln_noalloc(const uint8_t *codes, const uint16_t *scales, int64_t M, int64_t K, const uint16_t *X,
                           int64_t N, float *Y, void *stream) {
    static_assert(q4::kNoallocScratchBytes == Q4_NOALLOC_SCRATCH_BYTES, "the header states the scratch size");
    if (!shape_ok(M, K) || N < 0 || N > Q4_MAX_N) return Q4_ERR_SHAPE;
    if (M == 0 || N == 0) return Q4_OK;
    if (!codes || !scales || !X || !Y) return Q4_ERR_NULL;
    if (!aligned(codes, 16) || !aligned(scales, 2) || !aligned(X, 16) || !aligned(Y, 4))
        return Q4_ERR_ALIGN;
    const Range ry = range_of(Y, (uint64_t)N * M * 4);
    if (overlap(ry, range_of(codes, (uint64_t)M * (K / 2))) ||
        overlap(ry, range_of(scales, (uint64_t)M * (K / 64) * 2)) ||
        overlap(ry, range_of(X, (uint64_t)N * K * 2)))
        return Q4_ERR_OVERLAP;
    if (q4_gemm_smalln_ws_bytes(M, K, N) > Q4_NOALLOC_SCRATCH_BYTES) return Q4_ERR_WORKSPACE;
    return launch_status(q4::launch_gemm_smalln_noalloc(codes, scales, M, K, X, N, Y, (hipStream_t)stream));
}

int q4_gemm_smalln_affine(const uint8_t *codes, const uint16_t *scales, const uint16_t *zeros, int64_t M, int64_t K,
                          const uint16_t *X, int64_t N, float *Y, void *stream) {
    if (!shape_ok(M, K) || N < 0 || N > Q4_MAX_N) return Q4_ERR_SHAPE;
    if (M == 0 || N == 0) return Q4_OK;
    if (!codes || !scales || !zeros || !X || !Y) return Q4_ERR_NULL;
    if (!aligned(codes, 16) || !aligned(scales, 2) || !aligned(zeros, 2) || !aligned(X, 16) || !aligned(Y, 4))
        return Q4_ERR_ALIGN;
    const Range ry = range_of(Y, (uint64_t)N * M * 4);
    const uint64_t sb = (uint64_t)M * (K / 64) * 2;
    if (overlap(ry, range_of(codes, (uint64_t)M * (K / 2))) || overlap(ry, range_of(scales, sb)) ||
        overlap(ry, range_of(zeros, sb)) || overlap(ry, range_of(X, (uint64_t)N * K * 2)))
        return Q4_ERR_OVERLAP;
    return launch_status(q4::launch_gemm_smalln_affine(codes, scales, zeros, M, K, X, N, Y, (hipStream_t)stream));
}

namespace {
// The workspace checks shared by the two formats' entry points: `in` holds
// the inputs' ranges (Y's overlap with them is checked by the caller).
int formats_ws_check(int64_t M, int64_t K, int64_t N, Range ry, const Range *in, int nin, void *workspace,
                     size_t workspace_bytes) {
    const size_t need = q4_gemm_smalln_ws_bytes(M, K, N);
    if (need == 0) return Q4_OK;
    if (!workspace || workspace_bytes < need) return Q4_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return Q4_ERR_ALIGN;
    const Range rw = range_of(workspace, need);
    if (overlap(rw, ry)) return Q4_ERR_OVERLAP;
    for (int i = 0; i < nin; ++i)
        if (overlap(rw, in[i])) return Q4_ERR_OVERLAP;
    return Q4_OK;
}
}  // namespace

int q4_gemm_smalln_affine_ws(const uint8_t *codes, const uint16_t *scales, const uint16_t *zeros, int64_t M,
                             int64_t K, const uint16_t *X, int64_t N, float *Y, void *workspace,
                             size_t workspace_bytes, void *stream) {
    if (!shape_ok(M, K) || N < 0 || N > Q4_MAX_N) return Q4_ERR_SHAPE;
    if (M == 0 || N == 0) return Q4_OK;
    if (!codes || !scales || !zeros || !X || !Y) return Q4_ERR_NULL;
    if (!aligned(codes, 16) || !aligned(scales, 2) || !aligned(zeros, 2) || !aligned(X, 16) || !aligned(Y, 4))
        return Q4_ERR_ALIGN;
    const Range ry = range_of(Y, (uint64_t)N * M * 4);
    const uint64_t sb = (uint64_t)M * (K / 64) * 2;
    const Range in[4] = {range_of(codes, (uint64_t)M * (K / 2)), range_of(scales, sb), range_of(zeros, sb),
                         range_of(X, (uint64_t)N * K * 2)};
    for (const Range &r : in)
        if (overlap(ry, r)) return Q4_ERR_OVERLAP;
    const int st = formats_ws_check(M, K, N, ry, in, 4, workspace, workspace_bytes);
    if (st != Q4_OK) return st;
    return launch_status(q4::launch_gemm_smalln_affine_ws(codes, scales, zeros, M, K, X, N, Y,
                                                          static_cast<float *>(workspace), (hipStream_t)stream));
}

int q4_gemm_smalln_nvfp4_ws(const uint8_t *codes, const uint8_t *scales, const float *tscale, int64_t M, int64_t K,
                            const uint16_t *X, int64_t N, float *Y, void *workspace, size_t workspace_bytes,
                            void *stream) {
    if (!shape_ok(M, K) || N < 0 || N > Q4_MAX_N) return Q4_ERR_SHAPE;
    if (M == 0 || N == 0) return Q4_OK;
    if (!codes || !scales || !tscale || !X || !Y) return Q4_ERR_NULL;
    if (!aligned(codes, 16) || !aligned(scales, 4) || !aligned(tscale, 4) || !aligned(X, 16) || !aligned(Y, 4))
        return Q4_ERR_ALIGN;
    const Range ry = range_of(Y, (uint64_t)N * M * 4);
    const Range in[4] = {range_of(codes, (uint64_t)M * (K / 2)), range_of(scales, (uint64_t)M * (K / 16)),
                         range_of(tscale, 4), range_of(X, (uint64_t)N * K * 2)};
    for (const Range &r : in)
        if (overlap(ry, r)) return Q4_ERR_OVERLAP;
    const int st = formats_ws_check(M, K, N, ry, in, 4, workspace, workspace_bytes);
    if (st != Q4_OK) return st;
    return launch_status(q4::launch_gemm_smalln_nvfp4_ws(codes, scales, tscale, M, K, X, N, Y,
                                                         static_cast<float *>(workspace), (hipStream_t)stream));
}

int q4_gemm_smalln_nvfp4(const uint8_t *codes, const uint8_t *scales, const float *tscale, int64_t M, int64_t K,
                         const uint16_t *X, int64_t N, float *Y, void *stream) {
    if (!shape_ok(M, K) || N < 0 || N > Q4_MAX_N) return Q4_ERR_SHAPE;
    if (M == 0 || N == 0) return Q4_OK;
    if (!codes || !scales || !tscale || !X || !Y) return Q4_ERR_NULL;
    if (!aligned(codes, 16) || !aligned(scales, 4) || !aligned(tscale, 4) || !aligned(X, 16) || !aligned(Y, 4))
        return Q4_ERR_ALIGN;
    const Range ry = range_of(Y, (uint64_t)N * M * 4);
    if (overlap(ry, range_of(codes, (uint64_t)M * (K / 2))) || overlap(ry, range_of(scales, (uint64_t)M * (K / 16))) ||
        overlap(ry, range_of(tscale, 4)) || overlap(ry, range_of(X, (uint64_t)N * K * 2)))
        return Q4_ERR_OVERLAP;
    return launch_status(q4::launch_gemm_smalln_nvfp4(codes, scales, tscale, M, K, X, N, Y, (hipStream_t)stream));
}

namespace {

// The checks of the three fused entry points, on the operands in one form:
// scales are fp16 per 64-block (K / 32 bytes a row) or, for the NVFP4-style
// format, E4M3 bytes (K / 16 a row); the affine format needs zero points,
// the NVFP4-style format a tensor scale.
int fused_call(int fmt, const q4::FusedOperand *ops, int count, int64_t K, const uint16_t *x, int mode,
               float *const *y, const float *const *residual, void *stream) {
    if (mode != Q4_FUSE_SEPARATE && mode != Q4_FUSE_SWIGLU) return Q4_ERR_SHAPE;
    if (count < 1 || count > Q4_MAX_FUSED) return Q4_ERR_SHAPE;
    if (mode == Q4_FUSE_SWIGLU && count != 2) return Q4_ERR_SHAPE;
    if (!ops) return Q4_ERR_NULL;
    if (!shape_ok(0, K) || K > Q4_MAX_FUSED_K) return Q4_ERR_SHAPE;
    for (int i = 0; i < count; ++i)
        if (!shape_ok(ops[i].M, K)) return Q4_ERR_SHAPE;
    if (mode == Q4_FUSE_SWIGLU && ops[0].M != ops[1].M) return Q4_ERR_SHAPE;
    const int nout = mode == Q4_FUSE_SWIGLU ? 1 : count;
    bool any = false;
    for (int i = 0; i < count; ++i) any = any || ops[i].M > 0;
    if (!any) return Q4_OK;
    if (!x || !y) return Q4_ERR_NULL;
    if (!aligned(x, 16)) return Q4_ERR_ALIGN;
    const uint64_t scale_row = fmt == q4::kGemmNvfp4 ? (uint64_t)K / 16 : (uint64_t)(K / 64) * 2;
    // Inputs (read only; they may overlap each other).
    Range in[5 * Q4_MAX_FUSED + 1];
    int nin = 0;
    in[nin++] = range_of(x, (uint64_t)K * 2);
    for (int i = 0; i < count; ++i) {
        if (ops[i].M == 0) continue;
        if (!ops[i].codes || !ops[i].scales) return Q4_ERR_NULL;
        if (fmt == q4::kGemmAffine && !ops[i].zeros) return Q4_ERR_NULL;
        if (fmt == q4::kGemmNvfp4 && !ops[i].tscale) return Q4_ERR_NULL;
        if (!aligned(ops[i].codes, 16) || !aligned(ops[i].scales, 2) || !aligned(ops[i].bias, 4) ||
            !aligned(ops[i].zeros, 2) || !aligned(ops[i].tscale, 4))
            return Q4_ERR_ALIGN;
        in[nin++] = range_of(ops[i].codes, (uint64_t)ops[i].M * (K / 2));
        in[nin++] = range_of(ops[i].scales, (uint64_t)ops[i].M * scale_row);
        if (ops[i].bias) in[nin++] = range_of(ops[i].bias, (uint64_t)ops[i].M * 4);
        if (ops[i].zeros) in[nin++] = range_of(ops[i].zeros, (uint64_t)ops[i].M * (K / 64) * 2);
        if (ops[i].tscale) in[nin++] = range_of(ops[i].tscale, 4);
    }
    // Output o has ops[o].M floats (for SWIGLU, the common M).
    Range out[Q4_MAX_FUSED], res[Q4_MAX_FUSED];
    for (int o = 0; o < nout; ++o) {
        const uint64_t n = (uint64_t)ops[o].M * 4;
        const float *r = residual ? residual[o] : nullptr;
        out[o] = range_of(y[o], n);
        res[o] = range_of(r, r ? n : 0);
        if (n == 0) continue;
        if (!y[o]) return Q4_ERR_NULL;
        if (!aligned(y[o], 4) || !aligned(r, 4)) return Q4_ERR_ALIGN;
    }
    for (int o = 0; o < nout; ++o) {
        if (ops[o].M == 0) continue;
        for (int i = 0; i < nin; ++i)
            if (overlap(out[o], in[i])) return Q4_ERR_OVERLAP;
        // The residual may be the output itself, exactly; nothing else may
        // overlap an output.
        if (res[o].lo != out[o].lo && overlap(res[o], out[o])) return Q4_ERR_OVERLAP;
        for (int p = 0; p < nout; ++p) {
            if (p == o || ops[p].M == 0) continue;
            if (overlap(out[o], out[p]) || overlap(out[o], res[p])) return Q4_ERR_OVERLAP;
        }
    }
    return launch_status(
        q4::launch_gemv_fused(fmt, ops, count, mode == Q4_FUSE_SWIGLU, K, x, y, residual, (hipStream_t)stream));
}

}  // namespace

int q4_gemv_fused(const q4_operand *ops, int count, int64_t K, const uint16_t *x, int mode, float *const *y,
                  const float *const *residual, void *stream) {
    q4::FusedOperand fo[Q4_MAX_FUSED] = {};
    if (ops && count >= 1 && count <= Q4_MAX_FUSED)
        for (int i = 0; i < count; ++i) fo[i] = {ops[i].codes, ops[i].scales, ops[i].M, ops[i].bias, nullptr, nullptr};
    return fused_call(q4::kGemmNf4, ops ? fo : nullptr, count, K, x, mode, y, residual, stream);
}

int q4_gemv_fused_affine(const q4_operand_affine *ops, int count, int64_t K, const uint16_t *x, int mode,
                         float *const *y, const float *const *residual, void *stream) {
    q4::FusedOperand fo[Q4_MAX_FUSED] = {};
    if (ops && count >= 1 && count <= Q4_MAX_FUSED)
        for (int i = 0; i < count; ++i)
            fo[i] = {ops[i].codes, ops[i].scales, ops[i].M, ops[i].bias, ops[i].zeros, nullptr};
    return fused_call(q4::kGemmAffine, ops ? fo : nullptr, count, K, x, mode, y, residual, stream);
}

int q4_gemv_fused_nvfp4(const q4_operand_nvfp4 *ops, int count, int64_t K, const uint16_t *x, int mode,
                        float *const *y, const float *const *residual, void *stream) {
    q4::FusedOperand fo[Q4_MAX_FUSED] = {};
    if (ops && count >= 1 && count <= Q4_MAX_FUSED)
        for (int i = 0; i < count; ++i)
            fo[i] = {ops[i].codes, reinterpret_cast<const uint16_t *>(ops[i].scales), ops[i].M, ops[i].bias, nullptr,
                     ops[i].tscale};
    return fused_call(q4::kGemmNvfp4, ops ? fo : nullptr, count, K, x, mode, y, residual, stream);
}

int q4_gather_rows(const uint8_t *codes, const uint16_t *scales, int64_t M, int64_t K, const int32_t *ids,
                   int64_t n, int out_type, void *out, int32_t *status, void *stream) {
    if (!shape_ok(M, K) || n < 0) return Q4_ERR_SHAPE;
    if (out_type != Q4_OUT_F32 && out_type != Q4_OUT_BF16) return Q4_ERR_SHAPE;
    const bool bf16 = out_type == Q4_OUT_BF16;
    const int64_t elt = bf16 ? 2 : 4;
    // The grid is n times the workgroups of one row; the output must also
    // leave headroom in 64-bit byte counts.
    if (n > (INT64_C(1) << 31) / q4::gather_blocks_per_row(K, bf16) || n > (INT64_C(1) << 62) / (K * elt))
        return Q4_ERR_SHAPE;
    if (!status) return Q4_ERR_NULL;
    if (n > 0 && (!ids || !out)) return Q4_ERR_NULL;
    if (n > 0 && M > 0 && (!codes || !scales)) return Q4_ERR_NULL;
    if (!aligned(codes, 16) || !aligned(scales, 2) || !aligned(ids, 4) || !aligned(out, 16) || !aligned(status, 4))
        return Q4_ERR_ALIGN;
    const Range ro = range_of(out, (uint64_t)n * K * elt);
    const Range rs = range_of(status, 4);
    const Range in[3] = {range_of(codes, (uint64_t)M * (K / 2)), range_of(scales, (uint64_t)M * (K / 64) * 2),
                         range_of(ids, (uint64_t)n * 4)};
    for (const Range &r : in)
        if (overlap(ro, r) || overlap(rs, r)) return Q4_ERR_OVERLAP;
    if (overlap(ro, rs)) return Q4_ERR_OVERLAP;
    return launch_status(q4::launch_gather_rows(codes, scales, M, K, ids, n, bf16, out, status,
                                                (hipStream_t)stream));
}

}  // extern "C"
