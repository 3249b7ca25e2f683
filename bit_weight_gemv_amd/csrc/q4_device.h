// q4_device.h -- pieces shared by the libq4 kernels (gfx950 / CDNA4, wave64).
//
// The frozen codebook: the 16 NormalFloat-4 levels (QLoRA construction with
// an exact zero level), stored as fp32 bit patterns.  The deep-fold
// "Decode V2" page (section 6, "Linear primitive") dequantises through a
// 16-float NF4 table without printing it; this is the table the library
// commits to.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4 {

constexpr uint32_t kLevelBits[16] = {
    0xbf800000u, 0xbf3239b1u, 0xbf066b2eu, 0xbeca329eu,
    0xbe91a24bu, 0xbe3d353du, 0xbdba7869u, 0x00000000u,
    0x3da2fb01u, 0x3e24cadfu, 0x3e7c04dau, 0x3ead0336u,
    0x3ee1a4b5u, 0x3f1007a9u, 0x3f3913b0u, 0x3f800000u};

__host__ __device__ constexpr float level_f32(int i) {
    return __builtin_bit_cast(float, kLevelBits[i]);
}

// Decision midpoints between neighbouring levels, exact in fp64.
__host__ __device__ constexpr double level_mid(int i) {
    return ((double)level_f32(i) + (double)level_f32(i + 1)) * 0.5;
}

constexpr int kBlock = 64;       // weights per scale block (K direction)
constexpr int kChunkWeights = 32; // weights per 16-byte code chunk
constexpr int kWave = 64;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t lane_id() { return __lane_id(); }

// Raw buffer resource over `bytes` bytes at `base` (CDNA dword-3 format,
// no swizzle, no stride).  Loads through it take a wave-uniform base in
// SGPRs, a 32-bit per-lane offset and a uniform SGPR offset.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// Cache-policy operand of buffer loads: non-temporal (streamed once).
constexpr int kLoadNonTemporal = 2;

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

// Mark a wave-uniform 64-bit value as such (lives in SGPRs afterwards).
__device__ __forceinline__ int64_t uniform64(int64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// fp16 bit pattern of level i (round to nearest even, folded at compile
// time from the fp32 table).
__host__ __device__ constexpr uint32_t level_f16_bits_c(int i) {
    return (uint32_t)__builtin_bit_cast(unsigned short, (_Float16)level_f32(i));
}

// The same for a wave-uniform index, as a chain of scalar selects between
// literals: no memory access (a table load at kernel start would queue
// behind the first weight loads).
__device__ __forceinline__ uint32_t level_f16_bits(int i) {
    uint32_t v = level_f16_bits_c(0);
#define Q4_LEVEL_SEL(k) v = (i == k) ? level_f16_bits_c(k) : v;
    Q4_LEVEL_SEL(1) Q4_LEVEL_SEL(2) Q4_LEVEL_SEL(3) Q4_LEVEL_SEL(4) Q4_LEVEL_SEL(5)
    Q4_LEVEL_SEL(6) Q4_LEVEL_SEL(7) Q4_LEVEL_SEL(8) Q4_LEVEL_SEL(9) Q4_LEVEL_SEL(10)
    Q4_LEVEL_SEL(11) Q4_LEVEL_SEL(12) Q4_LEVEL_SEL(13) Q4_LEVEL_SEL(14) Q4_LEVEL_SEL(15)
#undef Q4_LEVEL_SEL
    return v;
}

// DPP row operations (gfx9 encodings).
constexpr int kDppQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

template <int CTRL>
__device__ __forceinline__ float dpp_add(float keep, float send) {
    return keep + dpp_f<CTRL>(send);
}

// DPP row_ror:n (rotate right by n lanes within each row of 16).
constexpr int dpp_row_ror(int n) { return 0x120 + n; }

// v + the value of lane (i ^ 16) (ds_swizzle bit mode: and 0x1f, xor 0x10).
__device__ __forceinline__ float add_xor16(float v) {
    return v + __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
}

// v + the value of lane (i ^ 32) (ds_bpermute through __shfl_xor).
__device__ __forceinline__ float add_xor32(float v) { return v + __shfl_xor(v, 32); }

template <int L>
__device__ __forceinline__ float ror_pow2(float v) {
    if constexpr (L == 0) return dpp_f<dpp_row_ror(1)>(v);
    else if constexpr (L == 1) return dpp_f<dpp_row_ror(2)>(v);
    else if constexpr (L == 2) return dpp_f<dpp_row_ror(4)>(v);
    else return dpp_f<dpp_row_ror(8)>(v);
}

// One pairing level of reduce_rows: rows 2j and 2j+1 become row j.  Lane i
// receives from lane i - 2^L (DPP row_ror, same lower bits, opposite bit L);
// a lane whose bit L is 0 keeps the sum of row 2j, otherwise of row 2j+1.
template <int L, int N>
__device__ __forceinline__ void pair_level(float (&v)[N], bool hi) {
#pragma unroll
    for (int j = 0; j < N / 2; ++j) {
        const float even = v[2 * j] + ror_pow2<L>(v[2 * j]);
        const float odd = v[2 * j + 1] + ror_pow2<L>(v[2 * j + 1]);
        v[j] = hi ? odd : even;
    }
}

// Reduce NR per-lane values (one per row) over the 64 lanes of a wave.  On
// return lane i holds the total of row i % NR.  log2(NR) pairing levels
// (three VALU operations per pair) leave each lane one row; lanes with equal
// i % NR are then summed (DPP row_ror within rows of 16, ds_swizzle across
// 16, ds_bpermute across 32).  NR = 16 costs about 50 VALU operations for 16
// rows instead of 16 full wave reductions.
template <int NR>
__device__ __forceinline__ float reduce_rows(const float (&a)[NR]) {
    static_assert(NR == 1 || NR == 2 || NR == 4 || NR == 8 || NR == 16, "NR must be a power of two <= 16");
    const unsigned lane = __lane_id();
    float v[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) v[r] = a[r];
    if constexpr (NR >= 2) pair_level<0, NR>(v, lane & 1u);
    if constexpr (NR >= 4) pair_level<1, NR>(v, (lane >> 1) & 1u);
    if constexpr (NR >= 8) pair_level<2, NR>(v, (lane >> 2) & 1u);
    if constexpr (NR >= 16) pair_level<3, NR>(v, (lane >> 3) & 1u);
    float t = v[0];
    if constexpr (NR <= 1) t += dpp_f<dpp_row_ror(1)>(t);
    if constexpr (NR <= 2) t += dpp_f<dpp_row_ror(2)>(t);
    if constexpr (NR <= 4) t += dpp_f<dpp_row_ror(4)>(t);
    if constexpr (NR <= 8) t += dpp_f<dpp_row_ror(8)>(t);
    t = add_xor16(t);
    return add_xor32(t);
}

// Sum over the 64 lanes of a wave; every lane gets the total.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_f<kDppQuadXor1>(v);
    v += dpp_f<kDppQuadXor2>(v);
    v += dpp_f<kDppRowHalfMirror>(v);  // lanes i and 7-i of each 8
    v += dpp_f<kDppRowMirror>(v);      // lanes i and 15-i of each 16
    // xor 16 within each half-wave (ds_swizzle bit mode: and 0x1f, xor 0x10)
    v += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
    float lo = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    float hi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    return lo + hi;
}

// Largest of an unsigned value over the wave, in a scalar register: DPP
// maxima over each row of 16 lanes (folded into v_max_u32 with a DPP
// operand), then the four rows' maxima read into scalar registers.  No LDS
// operation, so it does not queue behind other LDS traffic.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_max_u32(uint32_t v) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
    return o > v ? o : v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = dpp_max_u32<kDppQuadXor1>(v);
    v = dpp_max_u32<kDppQuadXor2>(v);
    v = dpp_max_u32<kDppRowHalfMirror>(v);
    v = dpp_max_u32<kDppRowMirror>(v);
    const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
    const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
    const uint32_t a0 = r0 > r1 ? r0 : r1, a1 = r2 > r3 ? r2 : r3;
    return a0 > a1 ? a0 : a1;
}

// Max over the 16 lanes of a DPP row (lanes 16r .. 16r+15); all get it.
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp_f<kDppQuadXor1>(v));
    v = fmaxf(v, dpp_f<kDppQuadXor2>(v));
    v = fmaxf(v, dpp_f<kDppRowHalfMirror>(v));
    v = fmaxf(v, dpp_f<kDppRowMirror>(v));
    return v;
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)h);
}

// Power of two 2^e as fp32 for e in [-126, 127].
__device__ __forceinline__ float exp2i(int e) {
    return __builtin_bit_cast(float, (uint32_t)(e + 127) << 23);
}

// An E4M3 scale byte (sign clear) as fp32: its 7 magnitude bits placed at
// fp32's exponent/mantissa boundary give 2^(e-127) (1 + m/8) for e > 0 and
// the denormal m 2^-129 for e == 0; times 2^120 that is exactly
// 2^(e-7) (1 + m/8), or (m/8) 2^-6 (fp32 denormals are kept).
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
    return __builtin_bit_cast(float, (b & 0x7Fu) << 20) * 0x1p120f;
}

}  // namespace q4
