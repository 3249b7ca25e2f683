// q4_internal.h -- launchers behind the C ABI (host side, not exported).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4 {

hipError_t launch_pack(const float *W, int64_t M, int64_t K, uint8_t *codes, uint16_t *scales,
                       int32_t *status, hipStream_t stream);

// A chunk of 2 or 3 tokens on short rows (K <= 2048, at most 12 four-row
// tiles per CU): the GEMV with every table lookup serving all tokens.
bool gemv_tokens_fits(int64_t M, int64_t K, int64_t N);
hipError_t launch_gemv_tokens(const uint8_t *codes, const uint16_t *scales, int64_t M, int64_t K,
                              const uint16_t *X, int64_t N, float *Y, hipStream_t stream);
// A chunk of 2 or 3 tokens on rows of 65..768 chunks of 32 weights (4
// tokens: 256..768 chunks): the grouped long-row GEMV with every table
// lookup serving all tokens, in the three weight formats.  Each wave loads its own slice of every
// token's activations, so a token costs more on rows of fewer chunks;
// measured against the 16-row matrix-core kernel (A/B in one process, us):
// 2048 x 11008 N = 2 / 3 / 4 7.1 / 8.9 / 10.7 against 17.2 / 17.4 / 17.4;
// 27648 x 5120 N = 2 22.3 against 57.0; 5120 x 5120 N = 2 / 3 8.0 / 16.3
// against 17.7 / 17.8; 8192 x 8192 N = 4 17.0 against 23.8; 4096 x 4096
// N = 2 5.4 against 7.7 -- but N = 4 on rows of 4096 or 5120 weights:
// 4096 x 4096 8.0 against 7.8, 11008 x 4096 19.6 against 19.1, 5120 x 5120
// 19.6 against 17.8.  (Host arithmetic only: shared with the host-side
// checks of the C ABI.)
inline bool gemv_tokens_multi_fits(int64_t M, int64_t K, int64_t N) {
    const int64_t C = K / 32;  // 32-weight chunks a row
    return N >= 2 && N <= 4 && M >= 1 && C > 64 && C <= 64 * 12 && (N < 4 || C >= 256);
}
// fmt: kGemmNf4, kGemmAffine (zeros) or kGemmNvfp4 (scales: the E4M3 bytes,
// tscale); the others null.
hipError_t launch_gemv_tokens_multi(int fmt, const uint8_t *codes, const void *scales, const uint16_t *zeros,
                                    const float *tscale, int64_t M, int64_t K, const uint16_t *X, int64_t N, float *Y,
                                    hipStream_t stream);
// Weight formats of the prefill kernels.
enum { kGemmNf4 = 0, kGemmAffine = 1, kGemmNvfp4 = 2 };

// A chunk of 2..8 tokens on short rows (K <= 2048, K % 128 == 0, dword-aligned
// scale and zero-point planes, at most 12 four-row tiles per CU): one 4-row
// tile per wave on the 16-block 4x4x4 matrix-core instruction.  zeros: the
// affine format's (else null); tscale: the NVFP4-style format's (else null).
bool gemm_rows4_fits(const void *scales, const uint16_t *zeros, int64_t M, int64_t K, int64_t N);
hipError_t launch_gemm_rows4(int fmt, const uint8_t *codes, const void *scales, const uint16_t *zeros,
                             const float *tscale, int64_t M, int64_t K, const uint16_t *X, int64_t N, float *Y,
                             hipStream_t stream);
hipError_t launch_gemv(const uint8_t *codes, const uint16_t *scales, int64_t M, int64_t K,
                       const uint16_t *x, float *y, hipStream_t stream);

// The affine format ((code - z) * s per 64-block).
hipError_t launch_pack_affine(const float *W, int64_t M, int64_t K, uint8_t *codes, uint16_t *scales,
                              uint16_t *zeros, int32_t *status, hipStream_t stream);
hipError_t launch_gemv_affine(const uint8_t *codes, const uint16_t *scales, const uint16_t *zeros, int64_t M,
                              int64_t K, const uint16_t *x, float *y, hipStream_t stream);

// int8 activations (one or two words, f32 scale per 32-block) and the affine
// format's GEMV on them (q2 null: one word).
hipError_t launch_quantize_x8(const uint16_t *x, int64_t K, int words, int8_t *q1, int8_t *q2, float *d,
                              hipStream_t stream);
hipError_t launch_gemv_affine_x8(const uint8_t *codes, const uint16_t *scales, const uint16_t *zeros, int64_t M,
                                 int64_t K, const int8_t *q1, const int8_t *q2, const float *d, float *y,
                                 hipStream_t stream);

// The NVFP4-style format (E2M1 * E4M3 per 16 * f32 tensor scale).
hipError_t launch_pack_nvfp4(const float *W, int64_t M, int64_t K, uint8_t *codes, uint8_t *scales,
                             float *tscale, int32_t *status, hipStream_t stream);
hipError_t launch_gemv_nvfp4(const uint8_t *codes, const uint8_t *scales, const float *tscale, int64_t M,
                             int64_t K, const uint16_t *x, float *y, hipStream_t stream);

// One matrix of a fused GEMV launch (sharing x with the others).  scales:
// fp16 per 64-block (NF4, affine) or the E4M3 bytes (NVFP4-style, passed as
// 16-bit units); zeros: the affine format's zero points; tscale: the
// NVFP4-style tensor scale (device f32).
struct FusedOperand {
    const uint8_t *codes;
    const uint16_t *scales;
    int64_t M;
    const float *bias;  // or null
    const uint16_t *zeros;
    const float *tscale;
};

// count matrices (at most 4) into y[i] (+ residual[i]), or, with swiglu,
// silu(W0 . x + b0) * (W1 . x + b1) (+ residual[0]) into y[0] (count == 2,
// equal M), in weight format fmt (kGemmNf4, kGemmAffine, kGemmNvfp4).
// K <= 16384.  Arguments are validated by the caller.
hipError_t launch_gemv_fused(int fmt, const FusedOperand *ops, int count, bool swiglu, int64_t K, const uint16_t *x,
                             float *const *y, const float *const *residual, hipStream_t stream);

hipError_t launch_gemm_smalln(const uint8_t *codes, const uint16_t *scales, int64_t M, int64_t K,
                              const uint16_t *X, int64_t N, float *Y, hipStream_t stream);
// The prefill product with scratch memory for partial sums: where
// gemm_split_fits holds (chunks the 16-row kernel takes on rows longer than
// 2048 weights), K is split in ranges of at most 2048 weights and the
// partial planes (gemm_split_bytes: ranges x N x M fp32 at `part`) are added
// by a second launch; elsewhere launch_gemm_smalln.
// K ranges of the split: the 16-row kernel's slices of 4 64-blocks (256
// weights), at most 8 a range (one per wave of its workgroup), dealt evenly.
inline int split_kranges(int64_t K) {
    const int64_t nslices = (K / 64 + 3) / 4;
    return (int)((nslices + 7) / 8);
}
// The chunks the split serves: those the 16-row kernel takes on rows of more
// than 8 slices (the 4-row kernel and the shared-lookup GEMV of one wave a
// row take only rows of up to 2048 weights).
inline bool gemm_split_fits(int64_t M, int64_t K, int64_t N) {
    return N >= 2 && N <= 32 && M >= 1 && split_kranges(K) > 1 && !gemv_tokens_multi_fits(M, K, N);
}
inline size_t gemm_split_bytes(int64_t M, int64_t K, int64_t N) {
    return (size_t)split_kranges(K) * (size_t)N * (size_t)M * sizeof(float);
}
hipError_t launch_gemm_smalln_ws(const uint8_t *codes, const uint16_t *scales, int64_t M, int64_t K,
                                 const uint16_t *X, int64_t N, float *Y, float *part, hipStream_t stream);
// The same with the library's fixed device scratch (q4_gemm_smalln_noalloc):
// kNoallocScratchBytes per device; the caller checks gemm_split_bytes
// against it first.
constexpr size_t kNoallocScratchBytes = (size_t)16 << 20;
hipError_t launch_gemm_smalln_affine_ws(const uint8_t *codes, const uint16_t *scales, const uint16_t *zeros,
                                        int64_t M, int64_t K, const uint16_t *X, int64_t N, float *Y, float *part,
                                        hipStream_t stream);
hipError_t launch_gemm_smalln_nvfp4_ws(const uint8_t *codes, const uint8_t *scales, const float *tscale, int64_t M,
                                       int64_t K, const uint16_t *X, int64_t N, float *Y, float *part,
                                       hipStream_t stream);
hipError_t launch_gemm_smalln_noalloc(const uint8_t *codes, const uint16_t *scales, int64_t M, int64_t K,
                                      const uint16_t *X, int64_t N, float *Y, hipStream_t stream);
// The prefill product of the affine and NVFP4-style formats (N == 1: their
// GEMV).  Arguments are validated by the caller.
hipError_t launch_gemm_smalln_affine(const uint8_t *codes, const uint16_t *scales, const uint16_t *zeros, int64_t M,
                                     int64_t K, const uint16_t *X, int64_t N, float *Y, hipStream_t stream);
hipError_t launch_gemm_smalln_nvfp4(const uint8_t *codes, const uint8_t *scales, const float *tscale, int64_t M,
                                    int64_t K, const uint16_t *X, int64_t N, float *Y, hipStream_t stream);

// Rows ids[0..n) of a packed matrix into fp32 or bf16 rows; workgroup 0
// writes *status.  Arguments are validated by the caller.
hipError_t launch_gather_rows(const uint8_t *codes, const uint16_t *scales, int64_t M, int64_t K,
                              const int32_t *ids, int64_t n, bool bf16, void *out, int32_t *status,
                              hipStream_t stream);
// Workgroups one output row takes (the grid is n times this): one lane per
// 16-byte output vector (4 fp32 or 8 bf16 values), kGatherThreads lanes a
// workgroup.
constexpr int kGatherThreads = 256;
inline int64_t gather_blocks_per_row(int64_t K, bool bf16) {
    const int64_t units = K / (bf16 ? 8 : 4);
    return (units + kGatherThreads - 1) / kGatherThreads;
}

}  // namespace q4
