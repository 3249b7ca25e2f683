// q4_gemv.hip -- y[m] = sum_k level[code(m,k)] * scale[m][k/64] * x[k].
//
// What is computed: the batch-1 decode projection of the deep-fold
// "Decode V2" page, section 6 ("Linear primitive"): table value times group
// scale times x, accumulated in fp32.  The page's own kernel (a 16-float
// table in shared memory, four warps splitting K, 1-4 rows per block) was
// written for a consumer NVIDIA part; what is kept here is that the table
// lives in on-chip memory that every lane can index independently (the page
// measured a constant-memory table serialising divergent lookups).  The rest
// is laid out for gfx950:
//
//  * Weight stream.  A lane owns 16-byte chunks of a row (32 weights); 64
//    lanes of a wave read 1 KB contiguous per load (global_load_dwordx4),
//    and all chunks of a tile are in flight before any is used.
//  * Lookup table.  A byte of codes (two weights) indexes a 256-entry table
//    whose entry is the pair (level[lo nibble], level[hi nibble]) as two fp16
//    in one dword, so one ds_read_b32 dequantises two weights and one
//    v_dot2_f32_f16 multiplies them with two activations.  The table is held
//    in LDS 64 times over, copy c in bank c, so lane l always reads bank
//    l % 64 and random codes never conflict (64 KB of the CU's 160 KB).  The
//    LDS address of lane l for byte b is (b << 8) | (l << 2), assembled by
//    one v_perm_b32 from the code word.
//  * Activations.  Each lane converts its own 32*CPL activations once from
//    bf16 to fp16, after scaling them by a power of two chosen from their
//    largest magnitude so that no bf16 value can overflow fp16; the lane's
//    partial sum is scaled back by the inverse power of two (exact).
//  * Scale.  The dot over a 32-weight chunk is multiplied by its block
//    scale once (fp32 FMA).
//  * Reduction.  DPP row ops + ds_swizzle + readlane inside the wave; an LDS
//    exchange across the waves of a workgroup when one row spans several
//    waves (long K).
//  * Schedule.  Rows are split into contiguous ranges, one per lane group
//    (a wave, or a whole workgroup for long K); a group walks its range NR
//    rows at a time with the next tile's loads issued before the current
//    tile is reduced.
//
// Error: the fp16 table rounds each level by at most 2^-11 relatively; every
// other step is an fp32 add or multiply.
#include "q4_device.h"
#include "q4_internal.h"

namespace q4 {

constexpr int kLutCopies = 64;
constexpr int kLutDwords = 256 * kLutCopies;  // 64 KB
constexpr int kMaxWavesPerGroup = 8;

// Dword i of the table holds entry i / 64 (a code byte) for lane slot
// i % 64.  A wave writes 64 consecutive dwords of one entry, so the entry
// index is wave-uniform.
__device__ __forceinline__ void fill_lut(uint32_t *lut) {
    for (int i = threadIdx.x; i < kLutDwords; i += blockDim.x) {
        const int e = __builtin_amdgcn_readfirstlane(i >> 6);
        lut[i] = level_f16_bits(e & 15) | (level_f16_bits(e >> 4) << 16);
    }
}

// Table value for byte `b` (0..3) of a code word.
template <int B>
__device__ __forceinline__ half2_t lut_pair(const uint32_t *lut, uint32_t word, uint32_t laneoff) {
    constexpr uint32_t sel = 0x0C0C0000u | ((4u + B) << 8);  // [laneoff, byte B, 0, 0]
    const uint32_t addr = __builtin_amdgcn_perm(word, laneoff, sel);
    const uint32_t v = *reinterpret_cast<const uint32_t *>(reinterpret_cast<const char *>(lut) + addr);
    return __builtin_bit_cast(half2_t, v);
}

// Dot of one 16-byte chunk (32 weights) with the lane's fp16 activations.
__device__ __forceinline__ float chunk_dot(const uint32_t *lut, uint4 q, const half2_t *xh,
                                           uint32_t laneoff) {
    float p = 0.0f;
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        p = __builtin_amdgcn_fdot2(lut_pair<0>(lut, w[d], laneoff), xh[4 * d + 0], p, false);
        p = __builtin_amdgcn_fdot2(lut_pair<1>(lut, w[d], laneoff), xh[4 * d + 1], p, false);
        p = __builtin_amdgcn_fdot2(lut_pair<2>(lut, w[d], laneoff), xh[4 * d + 2], p, false);
        p = __builtin_amdgcn_fdot2(lut_pair<3>(lut, w[d], laneoff), xh[4 * d + 3], p, false);
    }
    return p;
}

// Load the lane's activation chunks and convert them to fp16 scaled by a
// power of two; returns the inverse scale.
template <int CPL>
__device__ __forceinline__ float load_x(const uint16_t *__restrict__ x, const int (&cidx)[CPL],
                                        const bool (&cvalid)[CPL], half2_t (&xh)[CPL][16]) {
    uint32_t raw[CPL][16];
    u16x2_t mx = {0, 0};
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        if (cvalid[i]) {
            const uint4 *src = reinterpret_cast<const uint4 *>(x + (int64_t)cidx[i] * kChunkWeights);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const uint4 t = src[v];
                raw[i][4 * v + 0] = t.x;
                raw[i][4 * v + 1] = t.y;
                raw[i][4 * v + 2] = t.z;
                raw[i][4 * v + 3] = t.w;
            }
        } else {
#pragma unroll
            for (int v = 0; v < 16; ++v) raw[i][v] = 0;
        }
#pragma unroll
        for (int v = 0; v < 16; ++v)
            mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2_t, raw[i][v] & 0x7FFF7FFFu));
    }
    // Largest bf16 magnitude -> its biased exponent E; scale by 2^(141-E) so
    // the largest value lands in [2^14, 2^15), inside fp16's range.
    int E = (int)((mx.x > mx.y ? mx.x : mx.y) >> 7);
    if (E < 1) E = 1;
    int e = 141 - E;
    e = e > 126 ? 126 : (e < -126 ? -126 : e);
    const float up = exp2i(e);
#pragma unroll
    for (int i = 0; i < CPL; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const float lo = __builtin_bit_cast(float, raw[i][v] << 16);
            const float hi = __builtin_bit_cast(float, raw[i][v] & 0xFFFF0000u);
            half2_t h;
            h.x = (_Float16)(lo * up);
            h.y = (_Float16)(hi * up);
            xh[i][v] = h;
        }
    return exp2i(-e);
}

template <int NR, int CPL>
__global__ __launch_bounds__(512) void gemv_kernel(const uint8_t *__restrict__ codes,
                                                   const uint16_t *__restrict__ scales, int64_t M,
                                                   int K, const uint16_t *__restrict__ x,
                                                   float *__restrict__ y, int P) {
    __shared__ uint32_t lut[kLutDwords];
    __shared__ float red[kMaxWavesPerGroup][NR];

    const int C = K >> 5;        // 16-byte chunks per row
    const int nsb = K >> 6;      // scale blocks per row
    const int64_t row_bytes = K >> 1;
    const int G = blockDim.x / P;  // lane groups per workgroup
    const int lig = threadIdx.x % P;
    const int64_t ngroups = (int64_t)gridDim.x * G;
    const int64_t gid = (int64_t)blockIdx.x * G + threadIdx.x / P;
    const int64_t r_begin = gid * M / ngroups;
    const int64_t r_end = (gid + 1) * M / ngroups;

    int cidx[CPL];
    bool cvalid[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        cidx[i] = lig + i * P;
        cvalid[i] = cidx[i] < C;
    }

    uint4 q[NR][CPL];
    uint32_t sc[NR][CPL];
    auto load_tile = [&](int64_t r0) {
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const int64_t row = (r0 + r < r_end) ? r0 + r : r_end - 1;
            const uint8_t *crow = codes + row * row_bytes;
            const uint16_t *srow = scales + row * nsb;
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                if (cvalid[i]) {
                    q[r][i] = *reinterpret_cast<const uint4 *>(crow + (int64_t)cidx[i] * 16);
                    sc[r][i] = srow[cidx[i] >> 1];
                } else {
                    q[r][i] = make_uint4(0, 0, 0, 0);
                    sc[r][i] = 0;
                }
            }
        }
    };

    const bool has_rows = r_begin < r_end;
    if (has_rows) load_tile(r_begin);  // first tile in flight during set-up

    half2_t xh[CPL][16];
    const float down = load_x<CPL>(x, cidx, cvalid, xh);

    fill_lut(lut);
    __syncthreads();

    const uint32_t laneoff = (lane_id() & 63u) << 2;
    const int wave = lig >> 6;
    const int nwaves = P >> 6;

    for (int64_t r0 = r_begin; r0 < r_end; r0 += NR) {
        uint4 qc[NR][CPL];
        uint32_t scc[NR][CPL];
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                qc[r][i] = q[r][i];
                scc[r][i] = sc[r][i];
            }
        if (r0 + NR < r_end) load_tile(r0 + NR);  // prefetch the next tile

        float acc[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            acc[r] = 0.0f;
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const float p = chunk_dot(lut, qc[r][i], xh[i], laneoff);
                acc[r] = fmaf(p, f16_bits_to_f32(scc[r][i]), acc[r]);
            }
            acc[r] = wave_sum(acc[r] * down);
        }

        if (nwaves == 1) {
#pragma unroll
            for (int r = 0; r < NR; ++r)
                if (lig == r && r0 + r < r_end) y[r0 + r] = acc[r];
        } else {
            if ((lig & 63) == 0) {
#pragma unroll
                for (int r = 0; r < NR; ++r) red[wave][r] = acc[r];
            }
            __syncthreads();
            if (lig < NR && r0 + lig < r_end) {
                float s = 0.0f;
                for (int w = 0; w < nwaves; ++w) s += red[w][lig];
                y[r0 + lig] = s;
            }
            __syncthreads();
        }
    }
}

namespace {

int cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

template <int NR, int CPL>
hipError_t launch_variant(const uint8_t *codes, const uint16_t *scales, int64_t M, int K,
                          const uint16_t *x, float *y, int P, int G, hipStream_t stream) {
    // Two workgroups fit a CU (64 KB of LDS each); one pass over the grid.
    const int64_t max_wg = 2LL * cu_count();
    const int64_t tiles = (M + NR - 1) / NR;
    int64_t grid = (tiles + G - 1) / G;
    if (grid > max_wg) grid = max_wg;
    if (grid < 1) grid = 1;
    void *args[] = {&codes, &scales, &M, &K, &x, &y, &P};
    return hipLaunchKernel(reinterpret_cast<const void *>(&gemv_kernel<NR, CPL>), dim3((unsigned)grid),
                           dim3((unsigned)(P * G)), args, 0, stream);
}

}  // namespace

hipError_t launch_gemv(const uint8_t *codes, const uint16_t *scales, int64_t M, int64_t K,
                       const uint16_t *x, float *y, hipStream_t stream) {
    const int C = (int)(K / kChunkWeights);
    const int k = (int)K;
    if (C <= 64)  // one wave covers a row: 8 independent waves per workgroup
        return launch_variant<4, 1>(codes, scales, M, k, x, y, 64, 8, stream);
    if (C <= 128)
        return launch_variant<4, 2>(codes, scales, M, k, x, y, 64, 8, stream);
    // Long rows: the whole workgroup (up to 8 waves) shares a row tile.
    int cpl = 1;
    while (C > cpl * 64 * kMaxWavesPerGroup) cpl *= 2;
    const int waves = (C + cpl * 64 - 1) / (cpl * 64);
    const int P = waves * 64;
    switch (cpl) {
        case 1: return launch_variant<4, 1>(codes, scales, M, k, x, y, P, 1, stream);
        case 2: return launch_variant<4, 2>(codes, scales, M, k, x, y, P, 1, stream);
        case 4: return launch_variant<2, 4>(codes, scales, M, k, x, y, P, 1, stream);
        default: return launch_variant<1, 8>(codes, scales, M, k, x, y, P, 1, stream);
    }
}

}  // namespace q4
