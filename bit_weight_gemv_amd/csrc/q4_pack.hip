// q4_pack.hip -- fp32 W[M][K] -> packed 4-bit codes + fp16 block scales.
//
// Groups of 64 weights along K share one scale (deep-fold "Decode V2",
// section 2: hidden and intermediate sizes are multiples of the NF4 group of
// 64).  The scale is the block's absolute maximum rounded to fp16 nearest-even
// (golang.design accel/tensor, func Cast: f32 -> f16 is nearest-even and an
// out-of-range value becomes infinity, which this kernel refuses rather than
// clamps).  Each code is the nearest level to w / s, an exact midpoint going
// to the lower level, decided without division: code = #{i : w > mid_i * s},
// where mid_i * s and the comparison are exact in fp64.  Codes are packed two
// to a byte, low nibble first (accel/tensor, type Int4).
//
// Work split: 16 lanes per block (one DPP row), 4 weights per lane; a lane
// writes 2 bytes of codes, so a block's 32 code bytes leave in one coalesced
// run.
#include "q4_device.h"
#include "q4_internal.h"

namespace q4 {

__global__ void clear_word_kernel(int32_t *w) { *w = 0; }

__global__ __launch_bounds__(256) void pack_kernel(const float *__restrict__ W, int64_t nblocks,
                                                   uint8_t *__restrict__ codes,
                                                   uint16_t *__restrict__ scales,
                                                   int32_t *__restrict__ status) {
    const int64_t nthreads = (int64_t)gridDim.x * blockDim.x;
    // Every lane of a 16-lane row walks the same sequence of blocks, so the
    // row reductions below always see 16 participating lanes.
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < nblocks * 16;
         t += nthreads) {
        const int64_t blk = t >> 4;
        const int j = (int)(t & 15);
        const float4 w4 = *reinterpret_cast<const float4 *>(W + blk * kBlock + 4 * j);
        const float w[4] = {w4.x, w4.y, w4.z, w4.w};

        float amax = 0.0f, bad = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (!__builtin_isfinite(w[i])) bad = 1.0f;
            amax = fmaxf(amax, fabsf(w[i]));
        }
        amax = row16_max(amax);
        bad = row16_max(bad);
        if (bad != 0.0f) {
            if (j == 0) atomicOr(status, 1);
            continue;
        }
        const _Float16 s16 = (_Float16)amax;  // v_cvt_f16_f32: nearest-even
        const uint32_t s16_bits = __builtin_bit_cast(unsigned short, s16);
        if (s16_bits == 0x7C00u) {
            if (j == 0) atomicOr(status, 2);
            continue;
        }
        const double s = (double)(float)s16;  // exact widening
        uint32_t code[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const double wd = (double)w[i];
            uint32_t c = 0;
#pragma unroll
            for (int q = 0; q < 15; ++q) c += (wd > level_mid(q) * s) ? 1u : 0u;
            code[i] = (s == 0.0) ? 7u : c;
        }
        const uint16_t two_bytes =
            (uint16_t)(code[0] | (code[1] << 4) | (code[2] << 8) | (code[3] << 12));
        *reinterpret_cast<uint16_t *>(codes + blk * (kBlock / 2) + 2 * j) = two_bytes;
        if (j == 0) scales[blk] = (uint16_t)s16_bits;
    }
}

// ---------------------------------------------------------------------------
// Affine 4-bit format (golang.design accel/tensor, type Int4 and func
// Int4MatVec: What = (code - z) * s with an fp16 scale and an fp16 zero point
// per group; the error is at most the group's range over 30).  The page does
// not print its quantiser; the steps taken:
//   range [lo, hi] of the 64-block widened to hold 0; s = fp16 nearest-even
//   of (hi - lo) / 15, the subtraction and the division in fp64 (IEEE, as
//   on any host), the fp64 -> fp16 rounding done once (below);
//   z = #{ j in 0..14 : -lo > (j + 1/2) s }: the integer nearest to -lo / s,
//   a midpoint going down;
//   code = #{ j in 0..14 : w > (j - z + 1/2) s }: the nearest level, a
//   midpoint going to the lower code.
// (j + 1/2) and (j - z + 1/2) are half-integers of at most 5 bits and s has
// 11, so every product is exact in fp32 and every comparison decides as it
// would in exact arithmetic.  s == 0: codes and z are 0.
// ---------------------------------------------------------------------------

// fp64 -> fp16 with one rounding to nearest even: round to odd into fp32
// (truncate, then set the last bit when anything was cut off), then let the
// hardware round fp32 -> fp16 to nearest even.  With 13 more bits in fp32
// than in fp16 the two steps round exactly as one would.
__device__ __forceinline__ uint32_t f64_to_f16_bits_rne(double d) {
    float f = (float)d;
    if ((double)f != d) {
        uint32_t b = __builtin_bit_cast(uint32_t, f);
        if (fabs((double)f) > fabs(d)) b -= 1;  // one step toward zero: the truncation
        f = __builtin_bit_cast(float, b | 1u);
    }
    return __builtin_bit_cast(unsigned short, (_Float16)f);
}

__global__ __launch_bounds__(256) void pack_affine_kernel(const float *__restrict__ W, int64_t nblocks,
                                                          uint8_t *__restrict__ codes,
                                                          uint16_t *__restrict__ scales,
                                                          uint16_t *__restrict__ zeros,
                                                          int32_t *__restrict__ status) {
    const int64_t nthreads = (int64_t)gridDim.x * blockDim.x;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < nblocks * 16; t += nthreads) {
        const int64_t blk = t >> 4;
        const int j = (int)(t & 15);
        const float4 w4 = *reinterpret_cast<const float4 *>(W + blk * kBlock + 4 * j);
        const float w[4] = {w4.x, w4.y, w4.z, w4.w};
        float hi = 0.0f, nlo = 0.0f, bad = 0.0f;  // nlo = -lo
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (!__builtin_isfinite(w[i])) bad = 1.0f;
            hi = fmaxf(hi, w[i]);
            nlo = fmaxf(nlo, -w[i]);
        }
        hi = row16_max(hi);
        nlo = row16_max(nlo);
        bad = row16_max(bad);
        if (bad != 0.0f) {
            if (j == 0) atomicOr(status, 1);
            continue;
        }
        const uint32_t s16_bits = f64_to_f16_bits_rne(((double)hi + (double)nlo) / 15.0);
        if (s16_bits == 0x7C00u) {
            if (j == 0) atomicOr(status, 2);
            continue;
        }
        const float s = f16_bits_to_f32(s16_bits);
        int z = 0;
        if (s > 0.0f) {
#pragma unroll
            for (int q = 0; q < 15; ++q) z += (nlo > ((float)q + 0.5f) * s) ? 1 : 0;
        }
        uint32_t code[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t c = 0;
            if (s > 0.0f) {
#pragma unroll
                for (int q = 0; q < 15; ++q) c += (w[i] > ((float)(q - z) + 0.5f) * s) ? 1u : 0u;
            }
            code[i] = c;
        }
        const uint16_t two_bytes =
            (uint16_t)(code[0] | (code[1] << 4) | (code[2] << 8) | (code[3] << 12));
        *reinterpret_cast<uint16_t *>(codes + blk * (kBlock / 2) + 2 * j) = two_bytes;
        if (j == 0) {
            scales[blk] = (uint16_t)s16_bits;
            zeros[blk] = __builtin_bit_cast(unsigned short, (_Float16)(float)z);
        }
    }
}

hipError_t launch_pack_affine(const float *W, int64_t M, int64_t K, uint8_t *codes, uint16_t *scales,
                              uint16_t *zeros, int32_t *status, hipStream_t stream) {
    hipError_t e;
    {
        void *args[] = {&status};
        e = hipLaunchKernel(reinterpret_cast<const void *>(&clear_word_kernel), dim3(1), dim3(1), args, 0, stream);
        if (e != hipSuccess) return e;
    }
    int64_t nblocks = M * (K / kBlock);
    int64_t grid = (nblocks * 16 + 255) / 256;
    if (grid > 65536) grid = 65536;
    if (grid < 1) grid = 1;
    void *args[] = {&W, &nblocks, &codes, &scales, &zeros, &status};
    return hipLaunchKernel(reinterpret_cast<const void *>(&pack_affine_kernel), dim3((unsigned)grid), dim3(256),
                           args, 0, stream);
}

// ---------------------------------------------------------------------------
// NVFP4-style format (gizai tensor/lazy, fp4Blocks: E2M1 codes, low half
// first; one E4M3 scale per 16 values along k; an f32 tensor scale
// s = max|W| / (6 * 448)).  The page leaves the rounding steps open; taken:
//   s = f32 of the fp64 quotient max|W| / 2688;
//   a block's scale: the E4M3 value nearest to amax_b / (6 s), ties to the
//   even pattern, at most 448; s == 0 gives scale 0;
//   a code: the E2M1 magnitude nearest to |w| / (scale * s), ties to the even
//   pattern, at most 6, with w's sign bit; a block of scale 0 is all code 0.
// Each decision compares against a midpoint times 6 s or scale * s, exact in
// fp64 (at most 5 + 2 + 24 or 3 + 4 + 24 significant bits).  Scales are
// stored row-major, [M][K/16].
// Four launches: clear the status and the tensor-scale word; the absolute
// maximum, gathered in that word as fp32 bits (non-negative floats order
// like their bit patterns, so an unsigned atomic max is a float max); the
// pack, each thread one 16-weight block; the tensor scale written last,
// once no thread reads the maximum any more.
// ---------------------------------------------------------------------------

__global__ void clear_two_words_kernel(int32_t *a, uint32_t *b) {
    *a = 0;
    *b = 0;
}

__global__ __launch_bounds__(256) void absmax_kernel(const float *__restrict__ W, int64_t n4, uint32_t *amax_bits,
                                                     int32_t *status) {
    const int64_t nthreads = (int64_t)gridDim.x * blockDim.x;
    float m = 0.0f;
    int bad = 0;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < n4; t += nthreads) {
        const float4 w4 = reinterpret_cast<const float4 *>(W)[t];
        const float w[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (__builtin_isfinite(w[i]))
                m = fmaxf(m, fabsf(w[i]));
            else
                bad = 1;
        }
    }
    // Non-negative floats order like their bit patterns: an integer wave max.
    const int mb = __reduce_max_sync(~0ull, (int)__builtin_bit_cast(uint32_t, m));
    bad = __any(bad);
    if ((threadIdx.x & 63) == 0) {
        atomicMax(amax_bits, (uint32_t)mb);
        if (bad) atomicOr(status, 1);
    }
}

// E4M3 (sign clear) value of pattern b, 0 <= b <= 126, from the format:
// (m/8) 2^-6 for e == 0, (1 + m/8) 2^(e-7) otherwise.
__device__ __forceinline__ double e4m3_value(int b) {
    const int e = b >> 3, m = b & 7;
    return e == 0 ? (double)m * 0x1p-9 : (double)(8 + m) * __builtin_bit_cast(double, (uint64_t)(e - 10 + 1023) << 52);
}

__device__ __forceinline__ float nvfp4_tensor_scale(uint32_t amax_bits) {
    return (float)((double)__builtin_bit_cast(float, amax_bits) / 2688.0);
}

__global__ __launch_bounds__(256) void pack_nvfp4_kernel(const float *__restrict__ W, int64_t nblocks,
                                                         const uint32_t *__restrict__ amax_bits,
                                                         uint8_t *__restrict__ codes, uint8_t *__restrict__ scales) {
    const double s = (double)nvfp4_tensor_scale(*amax_bits);
    const int64_t nthreads = (int64_t)gridDim.x * blockDim.x;
    for (int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; blk < nblocks; blk += nthreads) {
        float w[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 v = reinterpret_cast<const float4 *>(W + blk * 16)[q];
            w[4 * q] = v.x;
            w[4 * q + 1] = v.y;
            w[4 * q + 2] = v.z;
            w[4 * q + 3] = v.w;
        }
        double amax = 0.0;
        bool bad = false;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            bad = bad || !__builtin_isfinite(w[k]);
            amax = fmax(amax, fabs((double)w[k]));
        }
        if (bad) continue;  // flagged by absmax_kernel; the block's output is unspecified
        // Nearest E4M3 to amax / (6 s): step past pattern b while amax lies
        // above the midpoint to b + 1 (or on it with b odd).
        int sb = 0;
        if (s > 0.0) {
            const double u = 6.0 * s;
            while (sb < 126) {
                const double mid = (e4m3_value(sb) + e4m3_value(sb + 1)) * 0.5 * u;
                if (amax > mid || (amax == mid && (sb & 1))) ++sb;
                else break;
            }
        }
        const double unit = e4m3_value(sb) * s;
        // E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6: midpoints in units.
        constexpr double kMid[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            uint32_t c = 0;
            if (unit > 0.0) {
                const double a = fabs((double)w[k]);
                uint32_t mag = 0;
#pragma unroll
                for (int j = 0; j < 7; ++j) {
                    const double mid = kMid[j] * unit;
                    // past midpoint j when above it, or on it with j odd
                    // (then the upper neighbour j + 1 is the even pattern)
                    mag += (a > mid || (a == mid && (j & 1))) ? 1u : 0u;
                }
                c = mag | (__builtin_signbit(w[k]) ? 8u : 0u);
            }
            if (k < 8)
                lo |= c << (4 * k);
            else
                hi |= c << (4 * (k - 8));
        }
        uint32_t *dst = reinterpret_cast<uint32_t *>(codes + blk * 8);
        dst[0] = lo;
        dst[1] = hi;
        scales[blk] = (uint8_t)sb;
    }
}

__global__ void write_tensor_scale_kernel(uint32_t *word) {
    *reinterpret_cast<float *>(word) = nvfp4_tensor_scale(*word);
}

hipError_t launch_pack_nvfp4(const float *W, int64_t M, int64_t K, uint8_t *codes, uint8_t *scales,
                             float *tscale, int32_t *status, hipStream_t stream) {
    uint32_t *word = reinterpret_cast<uint32_t *>(tscale);
    hipError_t e;
    {
        void *args[] = {&status, &word};
        e = hipLaunchKernel(reinterpret_cast<const void *>(&clear_two_words_kernel), dim3(1), dim3(1), args, 0,
                            stream);
        if (e != hipSuccess) return e;
    }
    {
        int64_t n4 = M * K / 4;
        int64_t grid = (n4 + 255) / 256;
        if (grid > 4096) grid = 4096;
        if (grid < 1) grid = 1;
        void *args[] = {&W, &n4, &word, &status};
        e = hipLaunchKernel(reinterpret_cast<const void *>(&absmax_kernel), dim3((unsigned)grid), dim3(256), args,
                            0, stream);
        if (e != hipSuccess) return e;
    }
    {
        int64_t nblocks = M * (K / 16);
        int64_t grid = (nblocks + 255) / 256;
        if (grid > 65536) grid = 65536;
        if (grid < 1) grid = 1;
        const uint32_t *amax = word;
        void *args[] = {&W, &nblocks, &amax, &codes, &scales};
        e = hipLaunchKernel(reinterpret_cast<const void *>(&pack_nvfp4_kernel), dim3((unsigned)grid), dim3(256),
                            args, 0, stream);
        if (e != hipSuccess) return e;
    }
    void *args[] = {&word};
    return hipLaunchKernel(reinterpret_cast<const void *>(&write_tensor_scale_kernel), dim3(1), dim3(1), args, 0,
                           stream);
}

hipError_t launch_pack(const float *W, int64_t M, int64_t K, uint8_t *codes, uint16_t *scales,
                       int32_t *status, hipStream_t stream) {
    hipError_t e;
    {
        void *args[] = {&status};
        e = hipLaunchKernel(reinterpret_cast<const void *>(&clear_word_kernel), dim3(1), dim3(1),
                            args, 0, stream);
        if (e != hipSuccess) return e;
    }
    int64_t nblocks = M * (K / kBlock);
    int64_t threads = nblocks * 16;
    int64_t grid = (threads + 255) / 256;
    if (grid > 65536) grid = 65536;
    if (grid < 1) grid = 1;
    void *args[] = {&W, &nblocks, &codes, &scales, &status};
    return hipLaunchKernel(reinterpret_cast<const void *>(&pack_kernel), dim3((unsigned)grid),
                          dim3(256), args, 0, stream);
}

}  // namespace q4
