// q4_quant.hip -- bf16 activations -> int8 words (one, or two of about 14
// bits) with an f32 scale per 32-block, for the integer-dot products.
//
// The deep-fold "Decode V2" page (the lane's knobs) lets a projection take
// its activation as f32, as two int8 words of about 14 bits (its default),
// or as one int8 word (as llama.cpp does).  Per block of 32 activations:
//   d  = the f32 rounding of the fp64 quotient max|x| / 127;
//   q1 = the integer nearest to x / d, ties to even, within +-127;
//   q2 = the integer nearest to 128 (x - q1 d) / d, same rule (two words);
// the value carried is d (q1 + q2 / 128).  Each integer is decided by
// comparing |x| (or |x - q1 d|) with (j + 1/2) d (or that over 128), all
// exact in fp64 (x has 8 significant bits, d 24, j + 1/2 at most 8), by a
// binary search over j, since the comparisons are monotone in j.
//
// One lane per activation (K <= 131072).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q4_device.h"
#include "q4_internal.h"

namespace q4 {

// #{ j in 0..126 : a > (j + 1/2) u, or a == (j + 1/2) u with j odd }: the
// nearest integer to a / u in 0..127 with ties to even.
__device__ __forceinline__ int nearest_int_127(double a, double u) {
    int lo = 0, hi = 127;  // the answer lies in [lo, hi]
    while (lo < hi) {
        const int j = (lo + hi) >> 1;
        const double mid = ((double)j + 0.5) * u;
        if (a > mid || (a == mid && (j & 1)))
            lo = j + 1;
        else
            hi = j;
    }
    return lo;
}

// One lane per activation: the 32 lanes of a half-wave hold one block, take
// its maximum by a butterfly, then each decides its own integers.
__global__ __launch_bounds__(256) void quantize_x8_kernel(const uint16_t *__restrict__ x, int K, int two,
                                                          int8_t *__restrict__ q1, int8_t *__restrict__ q2,
                                                          float *__restrict__ d) {
    const int k = blockIdx.x * blockDim.x + threadIdx.x;  // K is a multiple of 64: whole blocks per wave
    const bool live = k < K;
    const float v = live ? __builtin_bit_cast(float, (uint32_t)x[k] << 16) : 0.0f;
    float amax = fabsf(v);
#pragma unroll
    for (int m = 16; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m));  // within each 32-lane half
    if (!live) return;
    const float db = (float)((double)amax / 127.0);
    if ((k & 31) == 0) d[k >> 5] = db;
    int a1 = 0, a2 = 0;
    if (db > 0.0f) {
        const double dd = (double)db, xv = (double)v;
        a1 = nearest_int_127(fabs(xv), dd);
        if (xv < 0) a1 = -a1;
        if (two) {
            const double r = xv - (double)a1 * dd;  // exact
            a2 = nearest_int_127(fabs(r), dd / 128.0);
            if (r < 0) a2 = -a2;
        }
    }
    q1[k] = (int8_t)a1;
    if (two) q2[k] = (int8_t)a2;
}

hipError_t launch_quantize_x8(const uint16_t *x, int64_t K, int words, int8_t *q1, int8_t *q2, float *d,
                              hipStream_t stream) {
    int k = (int)K;
    int two = words == 2 ? 1 : 0;
    void *args[] = {&x, &k, &two, &q1, &q2, &d};
    return hipLaunchKernel(reinterpret_cast<const void *>(&quantize_x8_kernel), dim3((unsigned)((K + 255) / 256)),
                           dim3(256), args, 0, stream);
}

}  // namespace q4
