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
