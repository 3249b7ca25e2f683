// q4_lut.h -- the LDS dequantisation table shared by the libq4 products.
//
// A byte of codes (two weights, low nibble first) indexes a 256-entry table
// whose entry is the pair (level[lo nibble], level[hi nibble]) as two fp16 in
// one dword: one ds_read_b32 dequantises two weights into an operand that a
// v_dot2 or an fp16 MFMA consumes directly.  The table is held in LDS 64
// times over, copy c in bank c, so lane l always reads bank l % 64 and random
// codes never conflict (64 KB of the CU's 160 KB).  The LDS address of lane l
// for byte b is (b << 8) | (l << 2), assembled by one v_perm_b32 from the
// code word.  On-chip placement with independent per-lane indexing follows
// the deep-fold "Decode V2" page (section 6, "Linear primitive"), which found
// a constant-memory table serialising divergent lookups.
#pragma once

#include "q4_device.h"

namespace q4 {

constexpr int kLutCopies = 64;
constexpr int kLutDwords = 256 * kLutCopies;  // 64 KB
// The 256 distinct table entries (1 KB), built at compile time: entry b is
// the fp16 pair (level[b & 15], level[b >> 4]).  Kernels read it only with
// wave-uniform scalar loads, as the source of the LDS copies; no lane ever
// indexes it.
struct PairTable {
    uint32_t v[256];
};
constexpr PairTable make_pair_table() {
    PairTable t{};
    for (int b = 0; b < 256; ++b) t.v[b] = level_f16_bits_c(b & 15) | (level_f16_bits_c(b >> 4) << 16);
    return t;
}
__device__ const PairTable kPairTable = make_pair_table();

// fp16 bits of a small integer (|v| <= 15), exact.
constexpr uint32_t small_int_f16_bits(int v) {
    if (v == 0) return 0;
    const uint32_t sign = v < 0 ? 0x8000u : 0u;
    const int a = v < 0 ? -v : v;
    int e = 0;
    while ((2 << e) <= a) ++e;  // a = 2^e * (1 + f)
    return sign | (uint32_t)(e + 15) << 10 | (uint32_t)((a - (1 << e)) << (10 - e));
}
// The affine format's table: entry b is the pair (lo - 8, hi - 8) of the
// byte's two codes (exact small integers); the product subtracts z - 8 from
// each before it multiplies, so every term is (code - z) x.
constexpr PairTable make_affine_pair_table() {
    PairTable t{};
    for (int b = 0; b < 256; ++b)
        t.v[b] = small_int_f16_bits((b & 15) - 8) | (small_int_f16_bits((b >> 4) - 8) << 16);
    return t;
}
__device__ const PairTable kAffinePairTable = make_affine_pair_table();

// fp16 bits of an E2M1 code (sign bit 3; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4,
// 6, all exact in fp16).
constexpr uint32_t e2m1_f16_bits(int c) {
    constexpr uint32_t mag[8] = {0x0000u, 0x3800u, 0x3C00u, 0x3E00u, 0x4000u, 0x4200u, 0x4400u, 0x4600u};
    return mag[c & 7] | ((c & 8) ? 0x8000u : 0u);
}
// The E2M1 format's table: entry b is the pair of the byte's two E2M1 values.
constexpr PairTable make_e2m1_pair_table() {
    PairTable t{};
    for (int b = 0; b < 256; ++b) t.v[b] = e2m1_f16_bits(b & 15) | (e2m1_f16_bits(b >> 4) << 16);
    return t;
}
__device__ const PairTable kE2m1PairTable = make_e2m1_pair_table();

// Dword e * 64 + l of the LDS table holds entry e for lane slot l.  The 256
// entries are written in 8 portions of 32; wave w writes portions w, w + nw,
// ...: two 16-dword scalar loads fetch a portion's entries, and each entry is
// written to its 64 slots by one lane each (ds_write2st64 pairs two entries
// per instruction, conflict-free).  No per-entry index arithmetic and no
// dependence on the weight loads in flight.
__device__ __forceinline__ void fill_lut_from(uint32_t *lut, const PairTable &table) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nw = blockDim.x >> 6;
    for (int p = wave; p < 8; p += nw) {
        const uint32_t *src = table.v + 32 * p;
        uint32_t *dst = lut + (32 * kLutCopies) * p + lane;
#pragma unroll
        for (int i = 0; i < 32; ++i) dst[kLutCopies * i] = src[i];
    }
}
__device__ __forceinline__ void fill_lut(uint32_t *lut) { fill_lut_from(lut, kPairTable); }

// Table value for byte `B` (0..3) of a code word.
template <int B>
__device__ __forceinline__ half2_t lut_pair(const uint32_t *lut, uint32_t word, uint32_t laneoff) {
    constexpr uint32_t sel = 0x0C0C0000u | ((4u + B) << 8);  // [laneoff, byte B, 0, 0]
    const uint32_t addr = __builtin_amdgcn_perm(word, laneoff, sel);
    const uint32_t v = *reinterpret_cast<const uint32_t *>(reinterpret_cast<const char *>(lut) + addr);
    return __builtin_bit_cast(half2_t, v);
}

}  // namespace q4
