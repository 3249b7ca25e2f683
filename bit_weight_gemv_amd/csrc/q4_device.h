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

// fp16 bit pattern of level i (round to nearest even), built from the fp32
// table.  Used only while filling lookup tables.
__device__ __forceinline__ uint32_t level_f16_bits(int i) {
    _Float16 h = (_Float16)level_f32(i);
    return (uint32_t)__builtin_bit_cast(unsigned short, h);
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

}  // namespace q4
