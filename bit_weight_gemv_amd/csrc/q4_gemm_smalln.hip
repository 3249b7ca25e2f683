// q4_gemm_smalln.hip -- Y[n][m] = sum_k level[code(m,k)] * scale[m][k/64] * X[n][k]
// for a prefill chunk of N <= 32 tokens.
//
// What is computed: the prefill form of the deep-fold "Decode V2" page
// (section 0: prompts run as chunks of up to 32 tokens through a dedicated
// matrix-core product) -- the same representation and reconstruction as the
// vector form (golang.design accel/tensor, func Int4MatMul), with the matrix
// read once per chunk of tokens and the unpacking amortised over the chunk.
//
// gfx950 design:
//  * One wave computes a 32(n) x 32(m) output tile with
//    v_mfma_f32_32x32x16_bf16: operand A is 32 tokens x 16 k of X (bf16, as
//    given), operand B is 16 k x 32 rows of dequantised weights.  Tokens
//    n >= N are zero rows of A.
//  * Dequantisation goes through an LDS table: a code byte (two weights)
//    selects the bf16 pair of their levels (hi) and the bf16 pair of the
//    levels' residuals (lo), so level = hi + lo to 2^-17 relative and two
//    MFMAs (hi, lo) reproduce the fp32 table without rounding X.  The table is
//    stored 32 times (copy = lane % 32, 8 bytes each) so every half-wave
//    reads 32 distinct 8-byte slots: no bank conflicts for random codes.
//  * Scales are per (row, 64-block): a block's four k-steps accumulate into a
//    fresh tile, which is then added into the running tile times the scale of
//    each lane's row (lane l holds column m = l % 32 of the output tile).
//  * A lane's 16 code bytes are 32 consecutive k of one block; the four
//    MFMAs of a block take k = 32h + 8t + (0..7) for lane half h and step t,
//    and X is read with the same permutation of k.
//  * The four waves of a workgroup split the blocks of K; their tiles are
//    summed through LDS at the end.
#include "q4_device.h"
#include "q4_internal.h"

namespace q4 {

constexpr int kMmaLutCopies = 32;
constexpr int kMmaLutDwords = 256 * kMmaLutCopies * 2;  // 64 KB
constexpr int kSmallnWaves = 4;

__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
    const uint32_t b = __builtin_bit_cast(uint32_t, f);
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ void level_hi_lo(int i, uint32_t &hi, uint32_t &lo) {
    const float c = level_f32(i);
    hi = bf16_rne_bits(c);
    const float rest = c - __builtin_bit_cast(float, hi << 16);  // exact
    lo = bf16_rne_bits(rest);
}

// Dword i: entry e = i / 64 (wave-uniform), copy = (i % 64) / 2, part = i % 2
// (0: hi pair, 1: lo pair).  Byte address of (e, copy) = e * 256 + copy * 8.
__device__ __forceinline__ void fill_mma_lut(uint32_t *lut) {
    for (int i = threadIdx.x; i < kMmaLutDwords; i += blockDim.x) {
        const int e = __builtin_amdgcn_readfirstlane(i >> 6);
        uint32_t h0, l0, h1, l1;
        level_hi_lo(e & 15, h0, l0);
        level_hi_lo(e >> 4, h1, l1);
        lut[i] = (i & 1) ? (l0 | (l1 << 16)) : (h0 | (h1 << 16));
    }
}

template <int B>
__device__ __forceinline__ uint2 mma_lut_pair(const uint32_t *lut, uint32_t word, uint32_t laneoff) {
    constexpr uint32_t sel = 0x0C0C0000u | ((4u + B) << 8);
    const uint32_t addr = __builtin_amdgcn_perm(word, laneoff, sel);
    return *reinterpret_cast<const uint2 *>(reinterpret_cast<const char *>(lut) + addr);
}

template <int PF>
__global__ __launch_bounds__(256) void gemm_smalln_kernel(const uint8_t *__restrict__ codes,
                                                          const uint16_t *__restrict__ scales,
                                                          int64_t M, int K,
                                                          const uint16_t *__restrict__ X, int N,
                                                          float *__restrict__ Y) {
    __shared__ uint32_t lut[kMmaLutDwords];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int col = lane & 31;   // row of W / column of the output tile
    const int half = lane >> 5;  // which 32 k of a 64-block
    const int64_t m0 = (int64_t)blockIdx.x * 32;
    const int64_t mrow = (m0 + col < M) ? m0 + col : M - 1;
    const int nsb = K >> 6;
    const int b_begin = wave * nsb / kSmallnWaves;
    const int b_end = (wave + 1) * nsb / kSmallnWaves;
    const bool xrow = col < N;  // this lane carries token n = col in operand A
    const uint8_t *crow = codes + mrow * (int64_t)(K >> 1) + half * 16;
    const uint16_t *srow = scales + mrow * nsb;
    const uint16_t *xrow_ptr = X + (int64_t)(xrow ? col : 0) * K + half * 32;

    fill_mma_lut(lut);
    __syncthreads();

    const uint32_t laneoff = (uint32_t)(lane & 31) << 3;
    float16_t acc = {};

    for (int b0 = b_begin; b0 < b_end; b0 += PF) {
        uint4 q[PF];
        uint32_t sc[PF];
        uint4 xa[PF][4];
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const int b = (b0 + p < b_end) ? b0 + p : b_end - 1;
            q[p] = *reinterpret_cast<const uint4 *>(crow + (int64_t)b * 32);
            sc[p] = srow[b];
#pragma unroll
            for (int t = 0; t < 4; ++t)
                xa[p][t] = xrow ? *reinterpret_cast<const uint4 *>(xrow_ptr + (int64_t)b * 64 + 8 * t)
                                : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            if (b0 + p < b_end) {
                float16_t tile = {};
                const uint32_t w[4] = {q[p].x, q[p].y, q[p].z, q[p].w};
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const uint2 e0 = mma_lut_pair<0>(lut, w[t], laneoff);
                    const uint2 e1 = mma_lut_pair<1>(lut, w[t], laneoff);
                    const uint2 e2 = mma_lut_pair<2>(lut, w[t], laneoff);
                    const uint2 e3 = mma_lut_pair<3>(lut, w[t], laneoff);
                    const uint4 bh = make_uint4(e0.x, e1.x, e2.x, e3.x);
                    const uint4 bl = make_uint4(e0.y, e1.y, e2.y, e3.y);
                    const bf16x8_t a = __builtin_bit_cast(bf16x8_t, xa[p][t]);
                    tile = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8_t, bh),
                                                                   tile, 0, 0, 0);
                    tile = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8_t, bl),
                                                                   tile, 0, 0, 0);
                }
                const float s = f16_bits_to_f32(sc[p]);
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[r] = fmaf(tile[r], s, acc[r]);
            }
        }
    }

    // Sum the four waves' tiles through LDS (the table is no longer needed).
    __syncthreads();
    float *red = reinterpret_cast<float *>(lut);  // [wave][reg][lane]
#pragma unroll
    for (int r = 0; r < 16; ++r) red[(wave * 16 + r) * 64 + lane] = acc[r];
    __syncthreads();
    // Wave w finishes registers 4w .. 4w+3.
    const int64_t m = m0 + col;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
        const int r = wave * 4 + rr;
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < kSmallnWaves; ++w) s += red[(w * 16 + r) * 64 + lane];
        // Output layout of the 32x32 MFMA: register r of lane l is row
        // 8 * (r / 4) + 4 * (l / 32) + r % 4, column l % 32.
        const int n = 8 * (r >> 2) + 4 * half + (r & 3);
        if (n < N && m < M) Y[(int64_t)n * M + m] = s;
    }
}

hipError_t launch_gemm_smalln(const uint8_t *codes, const uint16_t *scales, int64_t M, int64_t K,
                              const uint16_t *X, int64_t N, float *Y, hipStream_t stream) {
    const int64_t grid = (M + 31) / 32;
    int k = (int)K, n = (int)N;
    void *args[] = {&codes, &scales, &M, &k, &X, &n, &Y};
    return hipLaunchKernel(reinterpret_cast<const void *>(&gemm_smalln_kernel<4>), dim3((unsigned)grid),
                           dim3(64 * kSmallnWaves), args, 0, stream);
}

}  // namespace q4
