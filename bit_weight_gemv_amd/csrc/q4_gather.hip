// q4_gather.hip -- rows of a packed matrix, dequantised (an embedding kept in
// the packed format, or the tied embedding that shares the lm_head matrix).
//
// What is computed: the deep-fold "Decode V2" page (run notes of section 6)
// keeps the embedding as packed rows and dequantises the rows a step needs
// into its arena instead of holding a dense vocabulary table, and lets a tied
// embedding share the lm_head's packed matrix; golang.design accel/tensor
// (func QuantGatherRows) gathers rows of a quantized table.  The value of a
// weight is level[code] * scale (section 6, Linear primitive).
//
// out[i][k] = What[ids[i], k] rounded once, to nearest even, to the output
// type.  What = level * scale is a 24-bit by 11-bit product, so an fp32
// multiply rounds it exactly once (no value comes near the fp32 subnormal
// range: the smallest non-zero magnitude is about 4.7e-9).  For bf16 the
// fp32 product is rounded again, and that second rounding decides a tie
// wrongly when the first one moved the value onto the bf16 midpoint; the
// exact remainder fma(c, s, -p) tells which side of the midpoint the exact
// product lies on, so the bf16 result is one rounding of the exact value.
// An id outside [0, M) is a caller error (accel/tensor func GatherRows): its
// row is written as zeros, the table is not read, and the status word gets
// Q4_GATHER_BAD_ID.
//
// Work split: one lane writes one 16-byte vector of a row (4 fp32 or 8 bf16
// values) from 2 or 4 bytes of codes; consecutive lanes take consecutive
// pieces, so loads and stores are contiguous across the wave.  A row takes
// ceil(units / 256) workgroups.  Workgroup 0 also reads every id and writes
// the status word (the only writer, so nothing has to clear it first).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q4.h"
#include "q4_device.h"
#include "q4_internal.h"

namespace q4 {

__device__ __forceinline__ uint32_t bf16_of_product(float c, float s) {
    const float p = c * s;
    const float r = fmaf(c, s, -p);  // exact: c * s - p
    const uint32_t b = __float_as_uint(p);
    const uint32_t low = b & 0xFFFFu;
    bool up;
    if (low != 0x8000u) {
        up = low > 0x8000u;
    } else if (r != 0.0f) {
        // The exact value lies beyond p (in magnitude) when r has p's sign.
        up = (__float_as_uint(r) >> 31) == (b >> 31);
    } else {
        up = (b >> 16) & 1u;  // an exact tie: to the even pattern
    }
    return (b >> 16) + (up ? 1u : 0u);
}

template <bool BF16>
__global__ __launch_bounds__(kGatherThreads) void gather_rows_kernel(
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales, int64_t M, int K,
    const int32_t *__restrict__ ids, int64_t n, int bpr, void *__restrict__ out,
    int32_t *__restrict__ status) {
    __shared__ float lv[16];
    if (threadIdx.x < 16) lv[threadIdx.x] = level_f32((int)threadIdx.x);
    if (blockIdx.x == 0) {
        int bad = 0;
        for (int64_t i = threadIdx.x; i < n; i += kGatherThreads) {
            const int32_t id = ids[i];
            bad |= (id < 0 || (int64_t)id >= M) ? 1 : 0;
        }
        bad = __syncthreads_or(bad);
        if (threadIdx.x == 0) *status = bad ? Q4_GATHER_BAD_ID : 0;
    } else {
        __syncthreads();
    }

    const int64_t i = blockIdx.x / bpr;  // output row
    if (i >= n) return;
    const int64_t id = ids[i];
    constexpr int kPer = BF16 ? 8 : 4;    // weights per lane
    const int units = K / kPer;
    const int u = (int)(blockIdx.x % bpr) * kGatherThreads + (int)threadIdx.x;
    if (u >= units) return;
    const int k0 = u * kPer;
    if (id < 0 || id >= M) {
        // A caller error: the row comes out as zeros (the table is never
        // read outside its rows) and the status word carries the flag.
        if constexpr (BF16)
            *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(out) + i * (int64_t)K + k0) = make_uint4(0, 0, 0, 0);
        else
            *reinterpret_cast<float4 *>(static_cast<float *>(out) + i * (int64_t)K + k0) = make_float4(0, 0, 0, 0);
        return;
    }
    const uint8_t *crow = codes + id * (int64_t)(K / 2);
    const float s = f16_bits_to_f32(scales[id * (int64_t)(K / 64) + k0 / 64]);
    if constexpr (BF16) {
        const uint32_t q = *reinterpret_cast<const uint32_t *>(crow + k0 / 2);
        uint32_t h[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) h[j] = bf16_of_product(lv[(q >> (4 * j)) & 0xF], s);
        uint4 v;
        v.x = h[0] | (h[1] << 16);
        v.y = h[2] | (h[3] << 16);
        v.z = h[4] | (h[5] << 16);
        v.w = h[6] | (h[7] << 16);
        *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(out) + i * (int64_t)K + k0) = v;
    } else {
        const uint32_t q = *reinterpret_cast<const uint16_t *>(crow + k0 / 2);
        float4 v;
        v.x = lv[q & 0xF] * s;
        v.y = lv[(q >> 4) & 0xF] * s;
        v.z = lv[(q >> 8) & 0xF] * s;
        v.w = lv[(q >> 12) & 0xF] * s;
        *reinterpret_cast<float4 *>(static_cast<float *>(out) + i * (int64_t)K + k0) = v;
    }
}

hipError_t launch_gather_rows(const uint8_t *codes, const uint16_t *scales, int64_t M, int64_t K,
                              const int32_t *ids, int64_t n, bool bf16, void *out, int32_t *status,
                              hipStream_t stream) {
    int bpr = (int)gather_blocks_per_row(K, bf16);
    int64_t grid = n * bpr;
    if (grid < 1) grid = 1;  // workgroup 0 still writes the status word
    int k = (int)K;
    void *args[] = {&codes, &scales, &M, &k, &ids, &n, &bpr, &out, &status};
    const void *fn = bf16 ? reinterpret_cast<const void *>(&gather_rows_kernel<true>)
                          : reinterpret_cast<const void *>(&gather_rows_kernel<false>);
    return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(kGatherThreads), args, 0, stream);
}

}  // namespace q4
