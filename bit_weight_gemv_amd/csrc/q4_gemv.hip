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
//    lanes of a wave read 1 KB contiguous per load (non-temporal
//    buffer_load_dwordx4), and all chunks of a tile are in flight before
//    any is used.
//  * Lookup table.  A byte of codes (two weights) indexes a 256-entry table
//    whose entry is the pair (level[lo nibble], level[hi nibble]) as two fp16
//    in one dword, so one ds_read_b32 dequantises two weights and one
//    v_dot2_f32_f16 multiplies them with two activations.  The table is held
//    in LDS 64 times over, copy c in bank c, so lane l always reads bank
//    l % 64 and random codes never conflict (64 KB of the CU's 160 KB).  The
//    LDS address of lane l for byte b is (b << 8) | (l << 2), assembled by
//    one v_perm_b32 from the code word.
//  * Activations.  Each lane converts its own 32*CPL activations once from
//    bf16 to fp16, after scaling them by a power of two chosen from the
//    wave's largest magnitude so that no bf16 value can overflow fp16; the
//    partial sums are scaled back by the inverse power of two (exact).  The
//    conversion is exact while no nonzero activation of the wave lies more
//    than 2^28 below that largest one.  A wave whose activations span more
//    runs a plain loop instead (the exact loop in gemv_body) that
//    multiplies the raw bf16 activations, widened exactly to fp32, with the
//    table levels in fp32 FMAs: slower, same accuracy bound, for any finite
//    bf16 input.
//  * Scale.  The dot over a 32-weight chunk is multiplied by its block
//    scale once (fp32 FMA).
//  * Reduction.  DPP row ops, ds_swizzle and ds_bpermute inside the wave;
//    an LDS exchange across the waves of a group when one row spans several
//    waves (long K).
//  * Schedule.  Rows are split into contiguous ranges, one per lane group
//    (a wave, or a group of waves for long K), or, on large matrices of
//    short rows, tiles are dealt to the waves in turn (the strided order);
//    a group walks its tiles NR rows at a time with the next tile's loads
//    issued before the current tile is reduced.
//  * Several tokens.  A prefill chunk of 2..4 tokens (gemv_tokens_kernel,
//    gemv_tokens_multi_kernel) runs the same body with each token's
//    activations converted as above and every table lookup feeding each
//    token's dot product, so each token's arithmetic is the one-token
//    GEMV's.
//
// Error: the fp16 table rounds each level by at most 2^-11 relatively; every
// other step is an fp32 add or multiply.
#include "q4_device.h"
#include "q4_internal.h"
#include "q4_lut.h"

namespace q4 {

constexpr int kMaxWavesPerGroup = 8;
constexpr int kMaxWavesPerBlock = 16;
// Row-per-wave variants cover rows of up to 128 chunks (K <= 4096): the LDS
// copy of the activations is at most 8 KB (512 lanes x 16 bytes).
constexpr int kSharedXUnits = 512;
// Rows of the first tile whose loads are issued before the table fill:
// variants that walk a long ring of row tiles issue their first tiles whole
// (their start-up is amortised, and the early tiles keep the HBM busy);
// short row ranges issue two rows, so the set-up behind them is not held up.
constexpr int pre_rows(int nr, int s, bool multi) { return (!multi && s >= 1) ? nr : (nr < 2 ? nr : 2); }

// Dot of one 16-byte chunk (32 weights) with the lane's fp16 activations.
// All 16 lookups are issued before the first product so their LDS latencies
// overlap.  ZOFF (the affine format): `zz` (z - 8 in both halves) is taken
// from each looked-up pair of code - 8 values, one packed fp16 subtract,
// exact for these small integers, so every product is (code - z) x.
template <bool ZOFF = false>
__device__ __forceinline__ float chunk_dot(const uint32_t *lut, uint4 q, const half2_t *xh, uint32_t laneoff,
                                           half2_t zz = half2_t{(_Float16)0.0f, (_Float16)0.0f}) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    half2_t v[16];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        v[4 * d + 0] = lut_pair<0>(lut, w[d], laneoff);
        v[4 * d + 1] = lut_pair<1>(lut, w[d], laneoff);
        v[4 * d + 2] = lut_pair<2>(lut, w[d], laneoff);
        v[4 * d + 3] = lut_pair<3>(lut, w[d], laneoff);
    }
    float p = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) p = __builtin_amdgcn_fdot2(ZOFF ? v[j] - zz : v[j], xh[j], p, false);
    return p;
}

// The chunk's weights against NTOK tokens' activations: each table lookup
// serves every token.
template <int NTOK>
__device__ __forceinline__ void chunk_dot_n(const uint32_t *lut, uint4 q, const half2_t (&xh)[NTOK][1][16],
                                            uint32_t laneoff, float (&p)[NTOK]) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int t = 0; t < NTOK; ++t) p[t] = 0.0f;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        half2_t v[4];
        v[0] = lut_pair<0>(lut, w[d], laneoff);
        v[1] = lut_pair<1>(lut, w[d], laneoff);
        v[2] = lut_pair<2>(lut, w[d], laneoff);
        v[3] = lut_pair<3>(lut, w[d], laneoff);
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int t = 0; t < NTOK; ++t) p[t] = __builtin_amdgcn_fdot2(v[b], xh[t][0][4 * d + b], p[t], false);
    }
}

// The affine form of chunk_dot_n: z - 8 (`zz`) is taken from each looked-up
// pair once, and the difference serves every token (the order of each
// token's sums is chunk_dot<true>'s).
template <int NTOK>
__device__ __forceinline__ void chunk_dot_n_zoff(const uint32_t *lut, uint4 q, const half2_t (&xh)[NTOK][1][16],
                                                 uint32_t laneoff, half2_t zz, float (&p)[NTOK]) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int t = 0; t < NTOK; ++t) p[t] = 0.0f;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        half2_t v[4];
        v[0] = lut_pair<0>(lut, w[d], laneoff) - zz;
        v[1] = lut_pair<1>(lut, w[d], laneoff) - zz;
        v[2] = lut_pair<2>(lut, w[d], laneoff) - zz;
        v[3] = lut_pair<3>(lut, w[d], laneoff) - zz;
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int t = 0; t < NTOK; ++t) p[t] = __builtin_amdgcn_fdot2(v[b], xh[t][0][4 * d + b], p[t], false);
    }
}

// chunk_dot_halves for NTOK tokens sharing each lookup (each token's two sums
// in chunk_dot_halves' order).
template <int NTOK>
__device__ __forceinline__ void chunk_dot_halves_n(const uint32_t *lut, uint4 q, const half2_t (&xh)[NTOK][1][16],
                                                   uint32_t laneoff, float (&p0)[NTOK], float (&p1)[NTOK]) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    half2_t v[16];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        v[4 * d + 0] = lut_pair<0>(lut, w[d], laneoff);
        v[4 * d + 1] = lut_pair<1>(lut, w[d], laneoff);
        v[4 * d + 2] = lut_pair<2>(lut, w[d], laneoff);
        v[4 * d + 3] = lut_pair<3>(lut, w[d], laneoff);
    }
#pragma unroll
    for (int t = 0; t < NTOK; ++t) {
        p0[t] = 0.0f;
        p1[t] = 0.0f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int t = 0; t < NTOK; ++t) {
            p0[t] = __builtin_amdgcn_fdot2(v[j], xh[t][0][j], p0[t], false);
            p1[t] = __builtin_amdgcn_fdot2(v[j + 8], xh[t][0][j + 8], p1[t], false);
        }
}

// The same dot split at the chunk's middle: p0 over its first 16 weights
// (bytes 0..7), p1 over the last 16, for formats with a scale per 16 weights.
__device__ __forceinline__ void chunk_dot_halves(const uint32_t *lut, uint4 q, const half2_t *xh,
                                                 uint32_t laneoff, float &p0, float &p1) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    half2_t v[16];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        v[4 * d + 0] = lut_pair<0>(lut, w[d], laneoff);
        v[4 * d + 1] = lut_pair<1>(lut, w[d], laneoff);
        v[4 * d + 2] = lut_pair<2>(lut, w[d], laneoff);
        v[4 * d + 3] = lut_pair<3>(lut, w[d], laneoff);
    }
    p0 = 0.0f;
    p1 = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        p0 = __builtin_amdgcn_fdot2(v[j], xh[j], p0, false);
        p1 = __builtin_amdgcn_fdot2(v[j + 8], xh[j + 8], p1, false);
    }
}

// The exact forms of the dots above, for activations that span too wide a
// range for one fp16 scale.  `xw` holds the raw bf16 activations of one code
// word of the chunk (4 dwords, two each); each is widened exactly to fp32
// and multiplied with a table level (fp16, widened exactly) in an fp32 FMA:
// the product is exact (11 + 8 significant bits), only the sums round.
// ZOFF (the affine format): `zoff` = z - 8 is taken from each table value of
// code - 8 first, so each term is (code - z) x exactly.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

template <bool ZOFF>
__device__ __forceinline__ float dot_word_exact(const uint32_t *lut, uint32_t w, u32x4_t xw, uint32_t laneoff,
                                                float p, float zoff) {
    const half2_t v0 = lut_pair<0>(lut, w, laneoff);
    const half2_t v1 = lut_pair<1>(lut, w, laneoff);
    const half2_t v2 = lut_pair<2>(lut, w, laneoff);
    const half2_t v3 = lut_pair<3>(lut, w, laneoff);
    auto lv = [&](_Float16 h) { return ZOFF ? (float)h - zoff : (float)h; };
    p = fmaf(lv(v0.x), bf16_lo(xw.x), p);
    p = fmaf(lv(v0.y), bf16_hi(xw.x), p);
    p = fmaf(lv(v1.x), bf16_lo(xw.y), p);
    p = fmaf(lv(v1.y), bf16_hi(xw.y), p);
    p = fmaf(lv(v2.x), bf16_lo(xw.z), p);
    p = fmaf(lv(v2.y), bf16_hi(xw.z), p);
    p = fmaf(lv(v3.x), bf16_lo(xw.w), p);
    return fmaf(lv(v3.y), bf16_hi(xw.w), p);
}

// Raw activations of chunk c (16 dwords, two bf16 each) from global memory;
// a lane past the row's end gets zeros.
__device__ __forceinline__ void load_chunk_x(const uint16_t *__restrict__ x, int c, bool valid,
                                             uint32_t (&raw)[16]) {
    if (valid) {
        const uint4 *src = reinterpret_cast<const uint4 *>(x + (int64_t)c * kChunkWeights);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const uint4 t = src[v];
            raw[4 * v + 0] = t.x;
            raw[4 * v + 1] = t.y;
            raw[4 * v + 2] = t.z;
            raw[4 * v + 3] = t.w;
        }
    } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) raw[v] = 0;
    }
}

// The same from the workgroup's LDS copy of the activations.
__device__ __forceinline__ void load_chunk_x_lds(const uint4 *xs, int c, bool valid, uint32_t (&raw)[16]) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const uint4 t = valid ? xs[c * 4 + v] : make_uint4(0, 0, 0, 0);
        raw[4 * v + 0] = t.x;
        raw[4 * v + 1] = t.y;
        raw[4 * v + 2] = t.z;
        raw[4 * v + 3] = t.w;
    }
}

// One chunk's 32 bf16 activations to fp16 under the power of two that puts a
// magnitude of biased exponent Emax in [2^14, 2^15): a bf16 value of
// exponent E has the fp16 exponent E - Emax + 29, so the bits are rebased
// with integer operations -- `sub` = (Emax - 29) << 7 taken from the
// magnitude (saturating: zero stays zero), a shift left by 3 (7 to 10
// mantissa bits), the sign put back.  Exact for values with E >= Emax - 28.
__device__ __forceinline__ void convert_chunk_x(const uint32_t (&raw)[16], u16x2_t sub, half2_t (&xh)[16]) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const u16x2_t f = __builtin_elementwise_sub_sat(__builtin_bit_cast(u16x2_t, raw[v] & 0x7FFF7FFFu), sub)
                          << u16x2_t{3, 3};
        xh[v] = __builtin_bit_cast(half2_t, (raw[v] & 0x80008000u) | __builtin_bit_cast(uint32_t, f));
    }
}

// Activations: the lane's chunks are converted to fp16, scaled by a
// wave-uniform power of two 2^e, e = 141 - Emax, chosen from the wave's
// largest bf16 magnitude (biased exponent Emax) so that nothing can
// overflow fp16; the inverse scale (exact) is returned.  `load(i, raw)`
// fetches the raw words of the lane's chunk i.  With one chunk per lane the
// caller passes them in `raw` (loaded early, so the conversion does not wait
// behind the weight tiles); with several, the maximum is taken in a first
// pass and the chunks are fetched again (from cache or LDS) for the
// conversion, so the raw and the converted copies are never live together.
//
// `exact` is set (wave-uniform) when the conversion loses nothing: every
// nonzero magnitude has a biased exponent of at least Emax - 28 (it is then
// an fp16 normal number after scaling) and Emax is 29 .. 254; a wave of
// zeros counts as exact.  Each lane tests its smallest nonzero magnitude
// (1 + the minimum of magnitude - 1 taken modulo 2^16, so zeros drop out);
// one ballot makes the answer wave-uniform.  The wave's maximum: DPP
// maxima over rows of 16, then the four rows' read into scalar registers.
template <int CPL, bool PRELOADED, class Load>
__device__ __forceinline__ float convert_x(Load load, uint32_t (&raw)[16], half2_t (&xh)[CPL][16], bool &exact) {
    u16x2_t mx = {0, 0};
    u16x2_t mn = {0xFFFF, 0xFFFF};
    const u16x2_t one = {1, 1};
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        if (!PRELOADED || CPL > 1) load(i, raw);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const u16x2_t mag = __builtin_bit_cast(u16x2_t, raw[v] & 0x7FFF7FFFu);
            mx = __builtin_elementwise_max(mx, mag);
            mn = __builtin_elementwise_min(mn, mag - one);
        }
    }
    const int m = (int)wave_max_u32(mx.x > mx.y ? mx.x : mx.y);
    const int E = m == 0 ? 29 : m >> 7;
    const int lo = (int)(mn.x < mn.y ? mn.x : mn.y);
    const bool in_range = E >= 29 && E <= 254;
    const bool lane_ok = lo == 0xFFFF || lo + 1 >= ((E - 28) << 7);
    exact = in_range && __builtin_amdgcn_ballot_w64(!lane_ok) == 0;
    const int eb = in_range ? E - 29 : 0;
    const u16x2_t sub = {(unsigned short)(eb << 7), (unsigned short)(eb << 7)};
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        if (CPL > 1) load(i, raw);
        convert_chunk_x(raw, sub, xh[i]);
    }
    return exp2i(eb - 112);
}

// One lane group (P lanes: a wave, or a whole workgroup for long rows) owns
// a contiguous range of rows and walks it NR rows (a tile) at a time.  Tiles
// t+1 .. t+S are in flight while tile t is consumed: buffer s of the ring
// holds tile t0+s and is reloaded with tile t0+s+S+1 once it is consumed.
// Register budget: one chunk per lane keeps 4 waves per SIMD (128 VGPRs);
// longer rows trade occupancy for the extra activation registers.  Groups
// spanning several waves use workgroups of at most 512 lanes.
// The one-load-per-tile scale path (TS) asks for six (at most 80 VGPRs): the
// one-tile-per-wave launches put up to 16 waves on a CU.  Its plain
// (epilogue-free) kernels ask for eight (at most 64): their main loop fits
// in 64 without spilling, and without the bound the register budget of the
// exact-activation loop (which runs only for activations the fp16 copy
// cannot hold) would lower the occupancy the main loop is scheduled for;
// with it, that loop's few spills stay in the rarely taken branch.
constexpr int gemv_min_waves(int cpl, bool ts = false, bool plain = false) {
    return ts ? (plain ? 8 : 6) : (cpl == 1 ? 4 : 2);
}
constexpr int gemv_max_block(bool multi, int cpl) { return cpl > 1 ? 512 : 1024; }

// SiLU(z) = z * sigmoid(z) = z / (1 + e^-z) (golang.design accel/tensor,
// func SiLU), fp32.
// Lane l of each quad's value, in every lane of the quad (DPP quad_perm).
__device__ __forceinline__ uint32_t quad_bcast(uint32_t v, int l) {
    switch (l) {
        case 0: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x00, 0xF, 0xF, false);
        case 1: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x55, 0xF, 0xF, false);
        case 2: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xAA, 0xF, 0xF, false);
        default: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xFF, 0xF, 0xF, false);
    }
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + expf(-z)); }

// One output segment of a launch.  The plain and affine forms read one
// matrix (codes0/scales0); the SwiGLU form reads a gate matrix (codes0) and
// an up matrix (codes1) of the same shape and writes silu(gate . x + bias0)
// times (up . x + bias1).  Optional fp32 epilogue operands may be null.  The
// host splits the segment's rows over its own range of workgroups.
struct GemvSeg {
    const uint8_t *codes0;
    const uint16_t *scales0;
    const uint16_t *zeros0;  // affine format only: fp16 zero points [rows][K/64]
    const float *tscale;     // NVFP4-style format only: the f32 tensor scale
    const int8_t *xq1;       // int8-activation forms: first words [K]
    const int8_t *xq2;       //   second words [K] (two-word form)
    const float *xd;         //   block scales [K/32]
    const uint8_t *codes1;
    const uint16_t *scales1;
    const uint16_t *zeros1;  // affine SwiGLU form: the up matrix's zero points
    const float *tscale1;    // NVFP4-style SwiGLU form: the up matrix's tensor scale
    const float *bias0;
    const float *bias1;
    const float *residual;
    float *y;
    int64_t rows;      // outputs of the segment
    int64_t rows_q;    // rows per lane group (quotient)
    int32_t rows_rem;  // groups with one more row
    int32_t wg_begin;  // first workgroup of the segment
};
constexpr int kMaxSegs = 4;
struct GemvSegs {
    GemvSeg s[kMaxSegs];
    int32_t n;
};
enum { kModePlain = 0, kModeEpi = 1, kModeSwiglu = 2 };
// Weight formats: the NF4 codebook (level[code] * s), the affine format
// ((code - z) * s with an fp16 zero point per 64-block; golang.design
// accel/tensor, type Int4 and func Int4MatVec), or the NVFP4-style format
// (E2M1 * E4M3 scale per 16 weights * an f32 tensor scale; gizai tensor/lazy,
// fp4Blocks).
// kFmtAffineX8 / kFmtAffineX8x2: the affine format with int8 activations of
// one or two words (the deep-fold page's lane: one int8 word as llama.cpp
// does, or two of about 14 bits): integer dot products, no table.
enum { kFmtNf4 = 0, kFmtAffine = 1, kFmtNvfp4 = 2, kFmtAffineX8 = 3, kFmtAffineX8x2 = 4 };

// Host-side operands of the int8-activation forms.
struct X8Args {
    const uint16_t *zeros;
    const int8_t *q1;
    const int8_t *q2;  // null for one word
    const float *d;
};

// The GEMV of one segment by one workgroup (index `wg` within the segment).
// MODE kModePlain: y = W . x.  kModeEpi: y = W . x (+ bias0) (+ residual).
// kModeSwiglu: each tile holds NR/2 gate rows and the NR/2 up rows of the
// same outputs; after the full reduction lane pairs are brought together and
// y = silu(g (+ bias0)) * (u (+ bias1)) (+ residual) -- SiLU only ever sees
// a finished sum (deep-fold "Decode V2" page, section 6 Linear primitive).
//
// FMT kFmtAffine: the table holds code - 8 (centred, exact in fp16) and
// z - 8 is taken from each looked-up pair before its product, so every term
// is (code - z) x itself: the zero point costs one load per chunk and one
// packed subtract per code byte.  (Applying it afterwards as (z - 8) times
// the chunk's activation sum would cancel when a large activation meets a
// weight of code z, and break the per-output bound.)
//
// TS (one chunk a lane, 16-bit scales (and zero points) on dword-aligned
// planes with an even number a row, as the host checks): a tile's scales are
// one contiguous run per matrix (LPT rows of K/64 values), read with one
// dword load per lane of the group and handed to the lanes that need them by
// quad broadcasts (DPP, inside each wave): one load instruction per tile and
// plane instead of one 2-byte load per row.
//
// NTOK > 1 (plain NF4, one chunk a lane, no ring: rows of one wave, one tile
// per wave, or rows of a group of waves): x is NTOK
// tokens, [NTOK][K] bf16, and y is [NTOK][rows]; every table lookup serves
// all tokens (a prefill chunk of 2 or 3 tokens).
// ONE: every group has at most one tile (the launch guarantees it), and the
// ring refill after it is left out.
template <int NR, int CPL, int S, int RG, bool MULTI, int MODE, int FMT = kFmtNf4, bool STRIDED = false,
          bool TS = false, int NTOK = 1, bool ONE = false>
__device__ __forceinline__ void gemv_body(const GemvSeg &sg, int K, const uint16_t *__restrict__ x, int P,
                                          int64_t wg) {
    constexpr bool X8 = FMT == kFmtAffineX8 || FMT == kFmtAffineX8x2;
    constexpr bool X8TWO = FMT == kFmtAffineX8x2;
    constexpr bool ZEROS = FMT == kFmtAffine || X8;  // zero-point plane
    __shared__ uint32_t lut[X8 ? 1 : kLutDwords];
    __shared__ float red[NTOK][kMaxWavesPerBlock][RG];
    // Groups of one wave all need the whole activation vector: it is read
    // from global memory once per workgroup into LDS (raw bf16, 16 bytes per
    // lane) and every wave takes its chunks from there.
    __shared__ uint4 xs[(MULTI || X8) ? 1 : kSharedXUnits * NTOK];
    static_assert(NTOK == 1 || (MODE == kModePlain && (FMT == kFmtNf4 || FMT == kFmtAffine || FMT == kFmtNvfp4) &&
                                CPL == 1 && S == 0 && !STRIDED),
                  "several tokens: plain products of bf16 activations, one chunk a lane, no ring");

    static_assert(MODE != kModeSwiglu || NR % 2 == 0, "a SwiGLU tile pairs gate and up rows");
    constexpr int LPT = MODE == kModeSwiglu ? NR / 2 : NR;  // outputs per tile
    static_assert(!TS || (CPL == 1 && S == 0 && FMT != kFmtNvfp4 && LPT <= 4),
                  "one scale run per tile and matrix");
    constexpr int NPART = MODE == kModeSwiglu ? 2 : 1;  // matrices a tile reads
    const int64_t rows_q = sg.rows_q;
    const int rows_rem = sg.rows_rem;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // A group is one wave (MULTI == false) or P / 64 waves of the
    // workgroup (MULTI; a workgroup holds blockDim.x / P groups).
    const int wpg = MULTI ? (P >> 6) : 1;     // waves per group
    const int grp = MULTI ? wave / wpg : 0;   // group within the workgroup
    const int wig = MULTI ? wave - grp * wpg : 0;  // wave within its group
    const int lig = wig * 64 + lane;          // lane within its group
    const int64_t gid = MULTI ? wg * (int64_t)(blockDim.x / P) + grp : wg * (blockDim.x >> 6) + wave;
    const int C = K >> 5;                      // 16-byte chunks per row
    const int nsb = K >> 6;                    // 64-blocks per row
    // Scale row stride in 16-bit units: one fp16 per 64-block, or (NVFP4)
    // two E4M3 bytes per 32-weight chunk.
    const int sst = FMT == kFmtNvfp4 ? (K >> 5) : nsb;
    const int64_t row_bytes = K >> 1;
    // Rows are split evenly over the groups by the host: rows_q each, one
    // more for the first rows_rem groups (no division on the device).
    const int64_t r_begin = gid * rows_q + (gid < rows_rem ? gid : rows_rem);
    const int64_t r_end = r_begin + rows_q + (gid < rows_rem ? 1 : 0);
    // STRIDED: tiles are dealt to the groups in turn (tile t of group gid is
    // tile t * ngroups + gid of the matrix), so at any moment the grid reads
    // one contiguous stretch of the matrix instead of one stretch per group;
    // otherwise a group owns the contiguous rows [r_begin, r_end).
    const int64_t ngroups = (int64_t)gridDim.x * (MULTI ? (int64_t)(blockDim.x / P) : (int64_t)(blockDim.x >> 6));
    const int64_t all_tiles = (sg.rows + LPT - 1) / LPT;
    const int64_t ntiles = STRIDED ? (gid < all_tiles ? (all_tiles - gid + ngroups - 1) / ngroups : 0)
                                   : (r_end - r_begin + LPT - 1) / LPT;
    const int64_t r_first = STRIDED ? gid * LPT : r_begin;           // first row of the first tile
    const int64_t tile_step = STRIDED ? ngroups * LPT : (int64_t)LPT;  // rows from one tile to the next
    // Groups spanning several waves meet at workgroup barriers in every
    // reduction group, so all groups of the grid walk the same number of
    // tiles: the most any group has (a group past its own range works on
    // tiles that load nothing and store nothing).
    const int64_t nsteps = !MULTI ? ntiles
                           : STRIDED ? (all_tiles + ngroups - 1) / ngroups
                                     : (rows_q + (rows_rem > 0 ? 1 : 0) + LPT - 1) / LPT;

    // Chunk indices of this lane.  Lanes past the row's end load a valid
    // chunk (the last one) and multiply it by zero activations, so every load
    // is unconditional.
    int cidx[CPL];
    bool cvalid[CPL];
    uint32_t coff[CPL];  // byte offset of the lane's chunk in a row
    uint32_t soff[CPL];  // 16-bit offset of its scale(s) in a row
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        cidx[i] = lig + i * P;
        cvalid[i] = cidx[i] < C;
        const int c = cvalid[i] ? cidx[i] : C - 1;
        coff[i] = (uint32_t)c * 16u;
        soff[i] = FMT == kFmtNvfp4 ? (uint32_t)c : (uint32_t)c >> 1;
    }

    // TS: the four lanes of quad Q of the group hold chunks 4Q .. 4Q+3, i.e. 64-blocks 2Q
    // and 2Q+1 of each row: the low and high halves of dword Q of the row's
    // scales.  Lane 4Q+r reads that dword of tile row r (rows r % LPT of each
    // matrix when LPT < 4), so row r's scales reach the quad by a broadcast of
    // its lane r.  Quads past the row's end read past every run (zeros).
    uint32_t ts_off = 0, ts_sh = 0;
    if constexpr (TS) {
        const int quad = lig >> 2;
        ts_off = quad < (C >> 2) ? (uint32_t)((((lane & 3) % LPT) * (nsb >> 1) + quad) * 4) : 0x40000000u;
        ts_sh = (uint32_t)((lane >> 1) & 1) << 4;
    }

    uint4 q[S + 1][NR][CPL];
    uint32_t sc[TS ? 1 : S + 1][NR][CPL];
    uint32_t tsc[TS ? S + 1 : 1][NPART];  // TS: this lane's dword of each run
    uint32_t zc[ZEROS && !TS ? S + 1 : 1][NR][CPL];  // zero-point bits (affine codes only)
    uint32_t tzc[ZEROS && TS ? S + 1 : 1][NPART];    // TS: this lane's dword of each zero-point run
    // Tiles are loaded in order.  The next tile to load starts at output
    // r_begin + LPT * (tiles loaded so far); its pointers advance by one tile
    // per load.  Rows past r_end repeat the last valid row (their results are
    // not stored), so every access stays inside the matrix.  A tile past the
    // last one is loaded through a buffer resource of zero records: the loads
    // stay unconditional (no register merges in the ring) but return zeros
    // without touching memory.  In the SwiGLU form rows LPT.. of a tile are
    // the up rows of rows 0..LPT-1 and come from the up matrix.
    const uint8_t *next_codes0 = sg.codes0 + r_first * row_bytes;
    const uint16_t *next_scales0 = sg.scales0 + r_first * sst;
    const uint16_t *next_zeros0 = ZEROS ? sg.zeros0 + r_first * nsb : nullptr;
    const uint8_t *next_codes1 = MODE == kModeSwiglu ? sg.codes1 + r_first * row_bytes : nullptr;
    const uint16_t *next_scales1 = MODE == kModeSwiglu ? sg.scales1 + r_first * sst : nullptr;
    const uint16_t *next_zeros1 = ZEROS && MODE == kModeSwiglu ? sg.zeros1 + r_first * nsb : nullptr;
    // Outputs from the next tile's first row to the end of the group's rows
    // (to the end of the matrix when STRIDED).
    int64_t next_left = STRIDED ? sg.rows - r_first : r_end - r_begin;
    // Rows [r0, r1) of the next tile into ring buffer `buf`; advance() then
    // moves the pointers to the tile after it.
    auto load_rows = [&](int buf, int r0, int r1) {
        const bool real = next_left > 0;
        const int nvalid = next_left < LPT ? (int)next_left : LPT;
        const __amdgpu_buffer_rsrc_t crs0 =
            buffer_rsrc(next_codes0, real ? (uint32_t)(LPT * row_bytes) : 0u);
        const __amdgpu_buffer_rsrc_t srs0 =
            buffer_rsrc(next_scales0, real ? (uint32_t)(LPT * sst * 2) : 0u);
        __amdgpu_buffer_rsrc_t zrs0 = srs0;
        if constexpr (ZEROS)
            zrs0 = buffer_rsrc(next_zeros0, real ? (uint32_t)(LPT * nsb * 2) : 0u);
        __amdgpu_buffer_rsrc_t crs1 = crs0, srs1 = srs0, zrs1 = zrs0;
        if constexpr (MODE == kModeSwiglu) {
            crs1 = buffer_rsrc(next_codes1, real ? (uint32_t)(LPT * row_bytes) : 0u);
            srs1 = buffer_rsrc(next_scales1, real ? (uint32_t)(LPT * sst * 2) : 0u);
            if constexpr (ZEROS) zrs1 = buffer_rsrc(next_zeros1, real ? (uint32_t)(LPT * nsb * 2) : 0u);
        }
        if constexpr (TS) {
            // The run of the tile's valid rows (whole dwords: an even number
            // of scales a row); lanes past it read zeros.
            const uint32_t run = (uint32_t)((real ? nvalid : 0) * nsb * 2);
            if (r0 == 0) {
                tsc[buf][0] = __builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(next_scales0, run), (int)ts_off, 0,
                                                                   kLoadNonTemporal);
                if constexpr (ZEROS)
                    tzc[buf][0] = __builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(next_zeros0, run), (int)ts_off,
                                                                       0, kLoadNonTemporal);
            }
            if constexpr (MODE == kModeSwiglu)
                if (r0 <= LPT && LPT < r1) {
                    tsc[buf][NPART - 1] = __builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(next_scales1, run),
                                                                               (int)ts_off, 0, kLoadNonTemporal);
                    if constexpr (ZEROS)
                        tzc[buf][NPART - 1] = __builtin_amdgcn_raw_buffer_load_b32(
                            buffer_rsrc(next_zeros1, run), (int)ts_off, 0, kLoadNonTemporal);
                }
        }
#pragma unroll
        for (int r = r0; r < r1; ++r) {
            const int lr = r % LPT;
            const int rr = lr < nvalid ? lr : (nvalid > 0 ? nvalid - 1 : 0);
            const bool up = MODE == kModeSwiglu && r >= LPT;
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                // Weights are read once: non-temporal loads keep them from
                // displacing reusable lines.
                const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(
                    up ? crs1 : crs0, (int)coff[i], (int)(rr * row_bytes), kLoadNonTemporal);
                q[buf][r][i] = make_uint4(v.x, v.y, v.z, v.w);
                if constexpr (!TS)
                    sc[buf][r][i] = __builtin_amdgcn_raw_buffer_load_b16(up ? srs1 : srs0, (int)(soff[i] * 2),
                                                                          rr * sst * 2, kLoadNonTemporal);
                if constexpr (ZEROS && !TS)
                    zc[buf][r][i] = __builtin_amdgcn_raw_buffer_load_b16(up ? zrs1 : zrs0, (int)(soff[i] * 2),
                                                                          rr * nsb * 2, kLoadNonTemporal);
            }
        }
    };
    auto advance = [&]() {
        next_codes0 += tile_step * row_bytes;
        next_scales0 += tile_step * sst;
        if constexpr (ZEROS) next_zeros0 += tile_step * nsb;
        if constexpr (MODE == kModeSwiglu) {
            next_codes1 += tile_step * row_bytes;
            next_scales1 += tile_step * sst;
            if constexpr (ZEROS) next_zeros1 += tile_step * nsb;
        }
        next_left -= tile_step;
    };
    auto load_tile = [&](int buf) {
        load_rows(buf, 0, NR);
        advance();
    };

    // Set-up order: activation loads, then the first PRE rows of the first
    // tile, then the table fill (no memory dependence, so it overlaps the
    // load latency), then the activation copy or conversion (which waits
    // only for the activation loads: vector loads complete in order) and the
    // barrier, and only then the rest of the ring.  A wave that issued its
    // whole ring first would stall in the memory pipeline until the HBM
    // returned data, and the set-up behind the loads would wait with it.
    // The first tiles load unconditionally: an empty row range loads through
    // zero-record resources (no memory access), and no branch makes the
    // compiler's wait analysis assume the tile loads might be missing.
    uint32_t xrawn[MULTI ? NTOK : 1][16];
    auto &xraw = xrawn[0];
    u32x4_t xunit[NTOK];  // this lane's 16 bytes of the shared activation copy, per token
    const int xunits = K >> 3;
    if constexpr (!X8) {
        if (MULTI) {
            // (Token t's activations start t * K values further.)
            if (CPL == 1)
#pragma unroll
                for (int t = 0; t < NTOK; ++t) load_chunk_x(x + (int64_t)t * K, cidx[0], cvalid[0], xrawn[t]);
        } else {
            // Bytes past the vector's end read as zero (buffer bounds).
#pragma unroll
            for (int t = 0; t < NTOK; ++t)
                xunit[t] = __builtin_amdgcn_raw_buffer_load_b128(buffer_rsrc(x, (uint32_t)K * 2u * NTOK),
                                                                 t * K * 2 + (int)threadIdx.x * 16, 0, 0);
        }
    }
    // int8-activation forms: each lane reads the 32 words (and the block
    // scale) of its own chunks; a chunk past the row's end reads past the
    // buffer bounds and gets zeros.
    u32x4_t q1raw[X8 ? CPL : 1][2], q2raw[X8TWO ? CPL : 1][2];
    float dch[X8 ? CPL : 1];
    if constexpr (X8) {
        const __amdgpu_buffer_rsrc_t r1 = buffer_rsrc(sg.xq1, (uint32_t)K);
        const __amdgpu_buffer_rsrc_t rd = buffer_rsrc(sg.xd, (uint32_t)K / 8u);
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int off = cvalid[i] ? cidx[i] * 32 : K;
            q1raw[i][0] = __builtin_amdgcn_raw_buffer_load_b128(r1, off, 0, 0);
            q1raw[i][1] = __builtin_amdgcn_raw_buffer_load_b128(r1, off + 16, 0, 0);
            dch[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, off / 8, 0, 0));
        }
        if constexpr (X8TWO) {
            const __amdgpu_buffer_rsrc_t r2 = buffer_rsrc(sg.xq2, (uint32_t)K);
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                const int off = cvalid[i] ? cidx[i] * 32 : K;
                q2raw[i][0] = __builtin_amdgcn_raw_buffer_load_b128(r2, off, 0, 0);
                q2raw[i][1] = __builtin_amdgcn_raw_buffer_load_b128(r2, off + 16, 0, 0);
            }
        }
    }
    constexpr int PRE = pre_rows(NR, S, MULTI);
    load_rows(0, 0, PRE);
    if constexpr (FMT == kFmtAffine)
        fill_lut_from(lut, kAffinePairTable);
    else if constexpr (FMT == kFmtNvfp4)
        fill_lut_from(lut, kE2m1PairTable);
    else if constexpr (!X8)
        fill_lut(lut);
    half2_t xhn[NTOK][X8 ? 1 : CPL][16];
    float downn[NTOK];
    auto &xh = xhn[0];
    float &down = downn[0];
    down = 1.0f;
    // Whether the conversion of every token was exact (wave-uniform).  For
    // groups of waves each wave decides alone: the main loop and the exact
    // loop meet the same workgroup barriers in the same order, so waves of
    // one workgroup may take different loops.
    bool xexact = true;
    if constexpr (X8) {
        // (no table and no shared activation copy to wait for)
    } else if constexpr (MULTI) {
#pragma unroll
        for (int t = 0; t < NTOK; ++t) {
            bool ex = true;
            downn[t] = convert_x<CPL, true>(
                [&](int i, uint32_t(&r)[16]) { load_chunk_x(x + (int64_t)t * K, cidx[i], cvalid[i], r); }, xrawn[t],
                xhn[t], ex);
            xexact = xexact && ex;
        }
        __syncthreads();
    } else {
        if ((int)threadIdx.x < xunits)
#pragma unroll
            for (int t = 0; t < NTOK; ++t)
                xs[t * xunits + threadIdx.x] = make_uint4(xunit[t].x, xunit[t].y, xunit[t].z, xunit[t].w);
        __syncthreads();
    }
    load_rows(0, PRE, NR);
    advance();
#pragma unroll
    for (int s = 1; s <= S; ++s) load_tile(s);
    if constexpr (!X8 && !MULTI)
#pragma unroll
        for (int t = 0; t < NTOK; ++t) {
            bool ex = true;
            downn[t] = convert_x<CPL, false>(
                [&](int i, uint32_t(&r)[16]) { load_chunk_x_lds(xs + t * xunits, cidx[i], cvalid[i], r); }, xraw,
                xhn[t], ex);
            xexact = xexact && ex;
        }

    // int8-activation forms: the words regrouped to match the code nibbles
    // (code dword d holds weights 8d .. 8d+7, even ones in the low nibbles):
    // E[d] = words 8d, 8d+2, 8d+4, 8d+6 and O[d] = words 8d+1, ..., 8d+7;
    // the chunk's word sums (for the zero point); d / 2048 per chunk (the
    // integer dot below carries a factor 16 * 128).
    uint32_t E1[X8 ? CPL : 1][4], O1[X8 ? CPL : 1][4], E2[X8TWO ? CPL : 1][4], O2[X8TWO ? CPL : 1][4];
    int qs1[X8 ? CPL : 1], qs2[X8TWO ? CPL : 1];
    float dsc[X8 ? CPL : 1];
    if constexpr (X8) {
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const uint32_t v[8] = {q1raw[i][0].x, q1raw[i][0].y, q1raw[i][0].z, q1raw[i][0].w,
                                   q1raw[i][1].x, q1raw[i][1].y, q1raw[i][1].z, q1raw[i][1].w};
            int t = 0;
#pragma unroll
            for (int dd = 0; dd < 4; ++dd) {
                E1[i][dd] = __builtin_amdgcn_perm(v[2 * dd + 1], v[2 * dd], 0x06040200u);
                O1[i][dd] = __builtin_amdgcn_perm(v[2 * dd + 1], v[2 * dd], 0x07050301u);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) t = __builtin_amdgcn_sdot4((int)v[j], 0x01010101, t, false);
            qs1[i] = t;
            dsc[i] = dch[i] * 0x1p-11f;
            if constexpr (X8TWO) {
                const uint32_t u[8] = {q2raw[i][0].x, q2raw[i][0].y, q2raw[i][0].z, q2raw[i][0].w,
                                       q2raw[i][1].x, q2raw[i][1].y, q2raw[i][1].z, q2raw[i][1].w};
                int t2 = 0;
#pragma unroll
                for (int dd = 0; dd < 4; ++dd) {
                    E2[i][dd] = __builtin_amdgcn_perm(u[2 * dd + 1], u[2 * dd], 0x06040200u);
                    O2[i][dd] = __builtin_amdgcn_perm(u[2 * dd + 1], u[2 * dd], 0x07050301u);
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) t2 = __builtin_amdgcn_sdot4((int)u[j], 0x01010101, t2, false);
                qs2[i] = t2;
            }
        }
    }

    const uint32_t laneoff = (uint32_t)lane << 2;
    // NVFP4-style format: the tensor scale joins the activations' inverse
    // power of two (both multiply every finished sum).  In the SwiGLU form
    // the gate and up matrices carry tensor scales of their own: each
    // multiplies its finished sum in the store, before SiLU.
    if constexpr (FMT == kFmtNvfp4 && MODE != kModeSwiglu)
#pragma unroll
        for (int t = 0; t < NTOK; ++t) downn[t] *= *sg.tscale;
    float ts_gate = 1.0f, ts_up = 1.0f;
    if constexpr (FMT == kFmtNvfp4 && MODE == kModeSwiglu) {
        ts_gate = *sg.tscale;
        ts_up = *sg.tscale1;
    }

    // Rows are reduced across the wave RG at a time (RG/NR tiles): the fixed
    // cost of the cross-lane reduction and of the store is paid once per RG
    // rows.  Ring step: accumulate tile t from buffer `buf` into rows
    // [j*NR, j*NR+NR) of the group (if t exists), then refill the buffer
    // with tile t + S + 1 (past the end it reads nothing; see the refill).
    constexpr int TPG = RG / NR;  // tiles per reduction group
    static_assert(RG % NR == 0 && TPG % (S + 1) == 0, "group must hold whole ring turns");
    float accn[NTOK][RG];
    auto &acc = accn[0];
    auto step = [&](int buf, int j, int64_t t) {
        if (t < ntiles) {
            // TS: row r's scale dword, broadcast in each quad from its lane r % LPT.
            uint32_t tsb[TS ? NR : 1], tzb[TS && ZEROS ? NR : 1];
            if constexpr (TS) {
#pragma unroll
                for (int r = 0; r < NR; ++r) {
                    tsb[r] = quad_bcast(tsc[buf][r < LPT ? 0 : NPART - 1], r % LPT);
                    if constexpr (ZEROS) tzb[r] = quad_bcast(tzc[buf][r < LPT ? 0 : NPART - 1], r % LPT);
                }
            }
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                float a = 0.0f;
#pragma unroll
                for (int i = 0; i < CPL; ++i) {
                    if constexpr (X8) {
                        // Nibble c of a code byte, XOR 8, placed in a byte's
                        // high half reads as the signed byte 16 (c - 8): even
                        // weights by a shift, odd ones in place.
                        const uint32_t w[4] = {q[buf][r][i].x, q[buf][r][i].y, q[buf][r][i].z, q[buf][r][i].w};
                        int t1 = 0, t2 = 0;
#pragma unroll
                        for (int dd = 0; dd < 4; ++dd) {
                            const uint32_t f = w[dd] ^ 0x88888888u;
                            const int ev = (int)((f << 4) & 0xF0F0F0F0u), od = (int)(f & 0xF0F0F0F0u);
                            t1 = __builtin_amdgcn_sdot4(ev, (int)E1[i][dd], t1, false);
                            t1 = __builtin_amdgcn_sdot4(od, (int)O1[i][dd], t1, false);
                            if constexpr (X8TWO) {
                                t2 = __builtin_amdgcn_sdot4(ev, (int)E2[i][dd], t2, false);
                                t2 = __builtin_amdgcn_sdot4(od, (int)O2[i][dd], t2, false);
                            }
                        }
                        // 16 sum (c - z) q = 16 sum (c - 8) q - 16 (z - 8) sum q:
                        // exact integers (|.| < 2^20; times 128 < 2^27).
                        const int zi = (int)f16_bits_to_f32(TS ? tzb[r] >> ts_sh : zc[buf][r][i]) - 8;
                        int tot = 128 * (t1 - 16 * zi * qs1[i]);
                        if constexpr (X8TWO) tot += t2 - 16 * zi * qs2[i];
                        a = fmaf((float)tot, f16_bits_to_f32(TS ? tsb[r] >> ts_sh : sc[buf][r][i]) * dsc[i], a);
                    } else if constexpr (FMT == kFmtNvfp4 && NTOK > 1) {
                        // (Each token's sums as in the one-token form below.)
                        float p0n[NTOK], p1n[NTOK];
                        chunk_dot_halves_n<NTOK>(lut, q[buf][r][i], xhn, laneoff, p0n, p1n);
                        const float s0 = e4m3_to_f32(sc[buf][r][i]), s1 = e4m3_to_f32(sc[buf][r][i] >> 8);
#pragma unroll
                        for (int t = 1; t < NTOK; ++t) accn[t][j * NR + r] = fmaf(p1n[t], s1, p0n[t] * s0);
                        a = fmaf(p0n[0], s0, a);
                        a = fmaf(p1n[0], s1, a);
                    } else if constexpr (FMT == kFmtNvfp4) {
                        float p0, p1;
                        chunk_dot_halves(lut, q[buf][r][i], xh[i], laneoff, p0, p1);
                        a = fmaf(p0, e4m3_to_f32(sc[buf][r][i]), a);
                        a = fmaf(p1, e4m3_to_f32(sc[buf][r][i] >> 8), a);
                    } else if constexpr (NTOK > 1) {
                        float pn[NTOK];
                        if constexpr (FMT == kFmtAffine) {
                            const _Float16 zo =
                                (_Float16)(f16_bits_to_f32(TS ? tzb[r] >> ts_sh : zc[buf][r][i]) - 8.0f);
                            chunk_dot_n_zoff<NTOK>(lut, q[buf][r][i], xhn, laneoff, half2_t{zo, zo}, pn);
                        } else {
                            chunk_dot_n<NTOK>(lut, q[buf][r][i], xhn, laneoff, pn);
                        }
                        const float sf = f16_bits_to_f32(TS ? tsb[r] >> ts_sh : sc[buf][r][i]);
#pragma unroll
                        for (int t = 1; t < NTOK; ++t) accn[t][j * NR + r] = pn[t] * sf;
                        a = fmaf(pn[0], sf, a);
                    } else {
                        float p;
                        if constexpr (FMT == kFmtAffine) {
                            const _Float16 zo =
                                (_Float16)(f16_bits_to_f32(TS ? tzb[r] >> ts_sh : zc[buf][r][i]) - 8.0f);
                            p = chunk_dot<true>(lut, q[buf][r][i], xh[i], laneoff, half2_t{zo, zo});
                        } else {
                            p = chunk_dot(lut, q[buf][r][i], xh[i], laneoff);
                        }
                        const uint32_t sbits = TS ? tsb[r] >> ts_sh : sc[buf][r][i];
                        a = fmaf(p, f16_bits_to_f32(sbits), a);
                    }
                }
                acc[j * NR + r] = a;
            }
        } else {
#pragma unroll
            for (int t = 0; t < NTOK; ++t)
#pragma unroll
                for (int r = 0; r < NR; ++r) accn[t][j * NR + r] = 0.0f;
        }
        // Refill with tile t + S + 1.  The plain products of groups of waves
        // (MULTI) skip refills past their last tile: those would load
        // nothing, but each load instruction still costs the CU's address
        // unit (down 2048 x 11008: 5.14 -> 5.05 us; 5120 x 5120: 5.75 ->
        // 5.62).  Elsewhere the refill stays unconditional: a conditional one
        // changed the compiler's wait counts (row-per-wave lm_head 27 -> 46
        // us; the fused down + residual 5.32 -> 5.79 us).
        if constexpr (!ONE)
            if (!(MULTI && MODE == kModePlain) || t + S + 1 < ntiles) load_tile(buf);
    };

    // The epilogue operands of a reduction group (first tile g0): lane l
    // reads those of the group's output l.  They are read when the group
    // starts, behind its weight tiles and ahead of the ring's refills, so
    // their latency hides under the group's arithmetic instead of following
    // the reduction.
    const int64_t nrows = r_end - r_begin;
    // Row of output `local` of the group (local = tile * LPT + row in tile),
    // or -1 past the group's rows.
    auto out_row = [&](int64_t local) -> int64_t {
        if constexpr (STRIDED) {
            const int64_t row = ((local / LPT) * ngroups + gid) * LPT + local % LPT;
            return row < sg.rows ? row : -1;
        } else {
            return local < nrows ? r_begin + local : -1;
        }
    };
    struct Epi {
        float b0, b1, r;
    };
    auto fetch_epi = [&](int64_t g0) {
        Epi e{0.0f, 0.0f, 0.0f};
        if constexpr (MODE != kModePlain) {
            constexpr int OPG = MODE == kModeSwiglu ? RG / 2 : RG;  // outputs per group
            const int64_t row = out_row(g0 * LPT + lane);
            if ((!MULTI || wig == 0) && lane < OPG && row >= 0) {
                if (sg.bias0) e.b0 = sg.bias0[row];
                if (MODE == kModeSwiglu && sg.bias1) e.b1 = sg.bias1[row];
                if (sg.residual) e.r = sg.residual[row];
            }
        }
        return e;
    };

    // Store of a reduction group whose first tile is g0; lane l holds the
    // finished sum of group row l (l < RG).  Every lane of the wave calls it.
    auto store = [&](float tot, int64_t g0, const Epi &e, int tok = 0) {
        if constexpr (MODE == kModeSwiglu) {
            // Output o of the group: tile o / LPT, gate row o % LPT of it and
            // the up row LPT after.
            const int o = lane < RG / 2 ? lane : 0;
            const int gate_lane = (o / LPT) * NR + o % LPT;
            const float g = __shfl(tot, gate_lane) * ts_gate;
            const float u = __shfl(tot, gate_lane + LPT) * ts_up;
            const int64_t row = out_row(g0 * LPT + lane);
            if (lane < RG / 2 && row >= 0) {
                const float a = sg.bias0 ? g + e.b0 : g;
                const float b = sg.bias1 ? u + e.b1 : u;
                float v = silu_f(a) * b;
                if (sg.residual) v += e.r;
                sg.y[row] = v;
            }
        } else {
            const int64_t row = out_row(g0 * NR + lane);
            if (lane < RG && row >= 0) {
                float v = tot;
                if (MODE == kModeEpi && sg.bias0) v += e.b0;
                if (MODE == kModeEpi && sg.residual) v += e.r;
                sg.y[tok * sg.rows + row] = v;
            }
        }
    };

    // The exact loop: the same tiles, rows, reductions, barriers and stores
    // as the main loop below, for a wave whose activations the fp16
    // conversion would not hold exactly.  Each row's chunks are read
    // directly (no prefetch ring) and multiplied with the raw activations
    // (exact_row); it is kept plain so that it needs fewer registers than
    // the main loop and leaves that loop's code and register budget as they
    // are.  Rare inputs only: its speed is not a concern.
    if constexpr (!X8) {
        if (__builtin_expect(!xexact, 0)) {
            // The lane's values, derived again from an index the compiler
            // cannot trace back to the set-up, so that nothing per-lane of
            // the set-up stays live into this loop (its registers are then
            // free for the loop's own values).
            int tid = (int)threadIdx.x;
            __asm__ volatile("" : "+v"(tid));
            const int e_lig = MULTI ? tid - grp * P : (tid & 63);
            const uint32_t e_laneoff = (uint32_t)(tid & 63) << 2;
            // Raw activations of token `tok`'s chunk c (valid: c < C), code
            // word d; a chunk past the row's end has zero activations.
            auto raw_word = [&](int tok, int c, bool valid, int d) -> u32x4_t {
                if (!valid) return u32x4_t{0u, 0u, 0u, 0u};
                uint4 v;
                if constexpr (MULTI)
                    v = reinterpret_cast<const uint4 *>(x + (int64_t)tok * K)[c * 4 + d];
                else
                    v = xs[tok * xunits + c * 4 + d];
                return u32x4_t{v.x, v.y, v.z, v.w};
            };
            // The lane's part of row `row` of one matrix for token `tok`.
            auto exact_row = [&](int tok, const uint8_t *cbase, const uint16_t *sbase, const uint16_t *zbase,
                                 int64_t row) -> float {
                float a = 0.0f;
#pragma unroll
                for (int i = 0; i < CPL; ++i) {
                    const int ci = e_lig + i * P;
                    const bool valid = ci < C;
                    const int c = valid ? ci : C - 1;
                    const uint32_t so = FMT == kFmtNvfp4 ? (uint32_t)c : (uint32_t)c >> 1;
                    const uint4 qv = *reinterpret_cast<const uint4 *>(cbase + row * row_bytes + c * 16);
                    const uint32_t sbits = sbase[row * sst + so];
                    float zoff = 0.0f;
                    if constexpr (FMT == kFmtAffine) zoff = f16_bits_to_f32(zbase[row * nsb + so]) - 8.0f;
                    float p0 = 0.0f, p1 = 0.0f;
#pragma clang loop unroll(disable)
                    for (int d = 0; d < 4; ++d) {
                        const uint32_t w = d == 0 ? qv.x : (d == 1 ? qv.y : (d == 2 ? qv.z : qv.w));
                        const float t = dot_word_exact<FMT == kFmtAffine>(lut, w, raw_word(tok, c, valid, d),
                                                                          e_laneoff, 0.0f, zoff);
                        if (d < 2) p0 += t; else p1 += t;
                    }
                    if constexpr (FMT == kFmtNvfp4) {
                        a = fmaf(p0, e4m3_to_f32(sbits), a);
                        a = fmaf(p1, e4m3_to_f32(sbits >> 8), a);
                    } else {
                        a = fmaf(p0 + p1, f16_bits_to_f32(sbits), a);
                    }
                }
                return a;
            };
            const float tsc = FMT == kFmtNvfp4 && MODE != kModeSwiglu ? *sg.tscale : 1.0f;
            for (int64_t g0 = 0; g0 < nsteps; g0 += TPG) {
                const Epi epi = fetch_epi(g0);
                // Lane l gets the total of group row l % RG, as reduce_rows
                // leaves it in the main loop; the rows are taken one at a
                // time (a rolled loop) and summed over the wave at once.
                float tot[NTOK];
#pragma unroll
                for (int tk = 0; tk < NTOK; ++tk) tot[tk] = 0.0f;
#pragma clang loop unroll(disable)
                for (int gr = 0; gr < RG; ++gr) {
                    // Group row gr is row r of tile j: output (tile, r % LPT);
                    // a SwiGLU tile's rows LPT.. are the up rows of the same
                    // outputs.
                    const int j = gr / NR, r = gr % NR;
                    const int64_t row = g0 + j < ntiles ? out_row((g0 + j) * LPT + r % LPT) : -1;
                    const bool up = MODE == kModeSwiglu && r >= LPT;
#pragma unroll
                    for (int tk = 0; tk < NTOK; ++tk) {
                        const float v = row < 0 ? 0.0f
                                                : exact_row(tk, up ? sg.codes1 : sg.codes0,
                                                            up ? sg.scales1 : sg.scales0,
                                                            up ? sg.zeros1 : sg.zeros0, row);
                        const float sum = wave_sum(v);
                        if ((tid & 63) % RG == gr) tot[tk] = sum;
                    }
                }
                if (!MULTI) {
#pragma unroll
                    for (int tk = 0; tk < NTOK; ++tk) store(tot[tk] * tsc, g0, epi, tk);
                } else {
                    if (lane < RG)
#pragma unroll
                        for (int tk = 0; tk < NTOK; ++tk) red[tk][wave][lane] = tot[tk] * tsc;
                    __syncthreads();
                    if (wig == 0) {
#pragma unroll
                        for (int tk = 0; tk < NTOK; ++tk) {
                            float sum = 0.0f;
                            if (lane < RG)
                                for (int w = 0; w < wpg; ++w) sum += red[tk][grp * wpg + w][lane];
                            store(sum, g0, epi, tk);
                        }
                    }
                    __syncthreads();
                }
            }
            return;
        }
    }

    for (int64_t g0 = 0; g0 < nsteps; g0 += TPG) {
        const Epi epi = fetch_epi(g0);
#pragma unroll
        for (int j = 0; j < TPG; ++j) step(j % (S + 1), j, g0 + j);
        // Lane l now holds the wave's total of group row (l % RG).
        const float tot = reduce_rows<RG>(acc) * down;
        if (!MULTI) {
            store(tot, g0, epi);
#pragma unroll
            for (int t = 1; t < NTOK; ++t) store(reduce_rows<RG>(accn[t]) * downn[t], g0, epi, t);
        } else {
            // (Every lane takes part in each token's cross-lane reduction.)
            float totn[NTOK];
            totn[0] = tot;
#pragma unroll
            for (int t = 1; t < NTOK; ++t) totn[t] = reduce_rows<RG>(accn[t]) * downn[t];
            if (lane < RG)
#pragma unroll
                for (int t = 0; t < NTOK; ++t) red[t][wave][lane] = totn[t];
            __syncthreads();
            if (wig == 0) {
#pragma unroll
                for (int t = 0; t < NTOK; ++t) {
                    float sum = 0.0f;
                    if (lane < RG)
                        for (int w = 0; w < wpg; ++w) sum += red[t][grp * wpg + w][lane];
                    store(sum, g0, epi, t);
                }
            }
            __syncthreads();
        }
    }
}

template <int NR, int CPL, int S, int RG, bool MULTI, bool STRIDED = false, bool TS = false, bool ONE = false>
__global__ __attribute__((amdgpu_flat_work_group_size(64, gemv_max_block(MULTI, CPL)),
                          amdgpu_waves_per_eu(gemv_min_waves(CPL, TS, true), 8))) void gemv_kernel(const uint8_t *__restrict__ codes,
                                                   const uint16_t *__restrict__ scales, int64_t M,
                                                   int K, const uint16_t *__restrict__ x,
                                                   float *__restrict__ y, int P, int64_t rows_q,
                                                   int rows_rem) {
    GemvSeg sg{};
    sg.codes0 = codes;
    sg.scales0 = scales;
    sg.y = y;
    sg.rows = M;
    sg.rows_q = rows_q;
    sg.rows_rem = rows_rem;
    gemv_body<NR, CPL, S, RG, MULTI, kModePlain, kFmtNf4, STRIDED, TS, 1, ONE>(sg, K, x, P, (int64_t)blockIdx.x);
}

// A prefill chunk of NTOK = 2 or 3 tokens on rows of one wave: Y [NTOK][M] =
// W . X^T with X [NTOK][K] bf16, one 4-row tile per wave.
template <int NTOK, bool TS>
__global__ __attribute__((amdgpu_flat_work_group_size(64, 768), amdgpu_waves_per_eu(3, 8))) void gemv_tokens_kernel(
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales, int64_t M, int K,
    const uint16_t *__restrict__ X, float *__restrict__ Y, int P, int64_t rows_q, int rows_rem) {
    GemvSeg sg{};
    sg.codes0 = codes;
    sg.scales0 = scales;
    sg.y = Y;
    sg.rows = M;
    sg.rows_q = rows_q;
    sg.rows_rem = rows_rem;
    gemv_body<4, 1, 0, 4, false, kModePlain, kFmtNf4, false, TS, NTOK>(sg, K, X, P, (int64_t)blockIdx.x);
}

// The same for rows spanning a group of waves (one chunk a lane): NTOK = 2..4
// tokens, 16 VGPRs of activations each; up to 16 waves a CU for two tokens
// (at most 128 VGPRs), 12 for three or four.
constexpr int tokens_multi_waves(int ntok) { return ntok == 2 ? 16 : 12; }
// FMT: the NF4 codebook, the affine format (zeros: its zero points) or the
// NVFP4-style format (scales: its E4M3 bytes read in pairs, tscale: the
// tensor scale).
template <int NTOK, int FMT, bool TS>
__global__ __attribute__((amdgpu_flat_work_group_size(64, 64 * tokens_multi_waves(NTOK)),
                          amdgpu_waves_per_eu(tokens_multi_waves(NTOK) / 4, 8))) void
gemv_tokens_multi_kernel(const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales,
                         const uint16_t *__restrict__ zeros, const float *__restrict__ tscale, int64_t M, int K,
                         const uint16_t *__restrict__ X, float *__restrict__ Y, int P, int64_t rows_q,
                         int rows_rem) {
    GemvSeg sg{};
    sg.codes0 = codes;
    sg.scales0 = scales;
    sg.zeros0 = zeros;
    sg.tscale = tscale;
    sg.y = Y;
    sg.rows = M;
    sg.rows_q = rows_q;
    sg.rows_rem = rows_rem;
    gemv_body<4, 1, 0, 4, true, kModePlain, FMT, false, TS, NTOK>(sg, K, X, P, (int64_t)blockIdx.x);
}

// The affine format's GEMV (y = W . x with W = (code - z) * s).
template <int NR, int CPL, int S, int RG, bool MULTI, bool STRIDED = false, bool TS = false>
__global__ __attribute__((amdgpu_flat_work_group_size(64, gemv_max_block(MULTI, CPL)),
                          amdgpu_waves_per_eu(gemv_min_waves(CPL, TS, true), 8))) void gemv_affine_kernel(
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales, const uint16_t *__restrict__ zeros,
    int64_t M, int K, const uint16_t *__restrict__ x, float *__restrict__ y, int P, int64_t rows_q, int rows_rem) {
    GemvSeg sg{};
    sg.codes0 = codes;
    sg.scales0 = scales;
    sg.zeros0 = zeros;
    sg.y = y;
    sg.rows = M;
    sg.rows_q = rows_q;
    sg.rows_rem = rows_rem;
    gemv_body<NR, CPL, S, RG, MULTI, kModePlain, kFmtAffine, STRIDED, TS>(sg, K, x, P, (int64_t)blockIdx.x);
}

// The NVFP4-style format's GEMV (y = s * sum E2M1 * E4M3 * x).
template <int NR, int CPL, int S, int RG, bool MULTI, bool STRIDED = false>
__global__ __attribute__((amdgpu_flat_work_group_size(64, gemv_max_block(MULTI, CPL)),
                          amdgpu_waves_per_eu(gemv_min_waves(CPL), 8))) void gemv_nvfp4_kernel(
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales, const float *__restrict__ tscale,
    int64_t M, int K, const uint16_t *__restrict__ x, float *__restrict__ y, int P, int64_t rows_q, int rows_rem) {
    GemvSeg sg{};
    sg.codes0 = codes;
    sg.scales0 = scales;
    sg.tscale = tscale;
    sg.y = y;
    sg.rows = M;
    sg.rows_q = rows_q;
    sg.rows_rem = rows_rem;
    gemv_body<NR, CPL, S, RG, MULTI, kModePlain, kFmtNvfp4, STRIDED>(sg, K, x, P, (int64_t)blockIdx.x);
}

// The affine format's GEMV on int8 activations (one or two words).
template <int NR, int CPL, int S, int RG, bool MULTI, int FMT, bool STRIDED = false, bool TS = false>
__global__ __attribute__((amdgpu_flat_work_group_size(64, gemv_max_block(MULTI, CPL)),
                          amdgpu_waves_per_eu(gemv_min_waves(CPL, TS), 8))) void gemv_affine_x8_kernel(
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales, const uint16_t *__restrict__ zeros,
    const int8_t *__restrict__ q1, const int8_t *__restrict__ q2, const float *__restrict__ d, int64_t M, int K,
    float *__restrict__ y, int P, int64_t rows_q, int rows_rem) {
    GemvSeg sg{};
    sg.codes0 = codes;
    sg.scales0 = scales;
    sg.zeros0 = zeros;
    sg.xq1 = q1;
    sg.xq2 = q2;
    sg.xd = d;
    sg.y = y;
    sg.rows = M;
    sg.rows_q = rows_q;
    sg.rows_rem = rows_rem;
    gemv_body<NR, CPL, S, RG, MULTI, kModePlain, FMT, STRIDED, TS>(sg, K, nullptr, P, (int64_t)blockIdx.x);
}

// Several segments in one launch: workgroup b belongs to the last segment
// whose first workgroup is <= b.
template <int NR, int CPL, int S, int RG, bool MULTI, int MODE, int FMT = kFmtNf4>
__global__ __attribute__((amdgpu_flat_work_group_size(64, gemv_max_block(MULTI, CPL)),
                          amdgpu_waves_per_eu(gemv_min_waves(CPL), 8))) void gemv_fused_kernel(GemvSegs segs, int K,
                                                   const uint16_t *__restrict__ x, int P) {
    int si = 0;
#pragma unroll
    for (int i = 1; i < kMaxSegs; ++i)
        if (i < segs.n && (int)blockIdx.x >= segs.s[i].wg_begin) si = i;
    si = __builtin_amdgcn_readfirstlane(si);
    const GemvSeg &sg = segs.s[si];
    gemv_body<NR, CPL, S, RG, MULTI, MODE, FMT>(sg, K, x, P, (int64_t)blockIdx.x - sg.wg_begin);
}

// The one-segment form (a SwiGLU pair, or a single matrix): the segment is
// the kernel argument itself, so its fields arrive with the first scalar
// reads instead of after a lookup of the workgroup's segment.
template <int NR, int CPL, int S, int RG, bool MULTI, int MODE, bool STRIDED = false, bool TS = false,
          int FMT = kFmtNf4>
__global__ __attribute__((amdgpu_flat_work_group_size(64, gemv_max_block(MULTI, CPL)),
                          amdgpu_waves_per_eu(gemv_min_waves(CPL, TS), 8))) void gemv_fused1_kernel(GemvSeg sg, int K,
                                                   const uint16_t *__restrict__ x, int P) {
    gemv_body<NR, CPL, S, RG, MULTI, MODE, FMT, STRIDED, TS>(sg, K, x, P, (int64_t)blockIdx.x);
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

// Whether every tile's run of scales starts on a dword, so that the
// one-load-per-tile scale path may read whole dwords: the scale planes (the
// second is the up matrix's scales or the zero points, or null) dword-aligned
// and an even number of scales a row (a contiguous row range may start at any
// row).  Every NF4 launch with one chunk a lane takes the path when this
// holds (one tile per wave, the strided order, rows spanning several waves,
// the fused form of one matrix or a SwiGLU pair); the affine forms take it
// outside the strided order, and
// the NVFP4-style format (two scale bytes a chunk) never.  Measured against the
// 2-byte loads (lab, same run): 151936 x 2048 27.29-27.38 against
// 27.54-27.62 us, 22016 x 2048 6.24-6.29 against 6.50-6.58, 11008 x 2048
// 4.56-4.60 against 4.78-4.83, 2048 x 11008 4.98 against 5.17.  The affine
// format keeps the 2-byte loads in the strided order, where its two planes
// read this way were slower (151936 x 2048 29.30 against 28.83 us).
bool scale_runs_aligned(const uint16_t *scales0, const uint16_t *scales1, int K) {
    const bool planes = (reinterpret_cast<uintptr_t>(scales0) & 3) == 0 &&
                        (reinterpret_cast<uintptr_t>(scales1) & 3) == 0;
    return planes && (K / 64) % 2 == 0;  // K / 64 scales a row
}

template <int NR, int CPL, int S, int RG, bool MULTI, int FMT, bool STRIDED = false>
// `extra` is the format's third operand: the affine zero points, or the
// NVFP4-style tensor scale (unused for NF4).
hipError_t launch_variant(const uint8_t *codes, const uint16_t *scales, const void *extra, int64_t M, int K,
                          const uint16_t *x, float *y, int P, int G, int64_t grid, hipStream_t stream) {
    // The LDS copy of the activations of a row-per-wave variant is one
    // 16-byte unit per lane of the workgroup.
    if (!MULTI && (K / 8 > P * G || K / 8 > kSharedXUnits)) return hipErrorInvalidValue;
    const int64_t ngroups = grid * G;
    int64_t rows_q = M / ngroups;
    int rows_rem = (int)(M % ngroups);
    if constexpr (FMT == kFmtAffine) {
        const uint16_t *zeros = static_cast<const uint16_t *>(extra);
        void *args[] = {&codes, &scales, &zeros, &M, &K, &x, &y, &P, &rows_q, &rows_rem};
        // (In the strided order the affine format's two planes were slower
        // this way: lm_head 29.30 against 28.83 us; down 5.39 against 5.65.)
        const void *fn = reinterpret_cast<const void *>(&gemv_affine_kernel<NR, CPL, S, RG, MULTI, STRIDED>);
        if constexpr (CPL == 1 && S == 0 && NR <= 4 && !STRIDED)
            if (scale_runs_aligned(scales, zeros, K))
                fn = reinterpret_cast<const void *>(&gemv_affine_kernel<NR, CPL, S, RG, MULTI, STRIDED, true>);
        return hipLaunchKernel(fn, dim3((unsigned)grid), dim3((unsigned)(P * G)), args, 0, stream);
    } else if constexpr (FMT == kFmtAffineX8 || FMT == kFmtAffineX8x2) {
        const X8Args *xa = static_cast<const X8Args *>(extra);
        const uint16_t *zeros = xa->zeros;
        const int8_t *q1 = xa->q1, *q2 = xa->q2;
        const float *d = xa->d;
        void *args[] = {&codes, &scales, &zeros, &q1, &q2, &d, &M, &K, &y, &P, &rows_q, &rows_rem};
        const void *fn = reinterpret_cast<const void *>(&gemv_affine_x8_kernel<NR, CPL, S, RG, MULTI, FMT, STRIDED>);
        if constexpr (CPL == 1 && S == 0 && NR <= 4 && !STRIDED)
            if (scale_runs_aligned(scales, zeros, K))
                fn = reinterpret_cast<const void *>(&gemv_affine_x8_kernel<NR, CPL, S, RG, MULTI, FMT, STRIDED, true>);
        return hipLaunchKernel(fn, dim3((unsigned)grid), dim3((unsigned)(P * G)), args, 0, stream);
    } else if constexpr (FMT == kFmtNvfp4) {
        const float *tscale = static_cast<const float *>(extra);
        void *args[] = {&codes, &scales, &tscale, &M, &K, &x, &y, &P, &rows_q, &rows_rem};
        return hipLaunchKernel(reinterpret_cast<const void *>(&gemv_nvfp4_kernel<NR, CPL, S, RG, MULTI, STRIDED>),
                               dim3((unsigned)grid), dim3((unsigned)(P * G)), args, 0, stream);
    } else {
        (void)extra;
        void *args[] = {&codes, &scales, &M, &K, &x, &y, &P, &rows_q, &rows_rem};
        const void *fn = reinterpret_cast<const void *>(&gemv_kernel<NR, CPL, S, RG, MULTI, STRIDED>);
        if constexpr (CPL == 1 && S == 0 && NR <= 4) {
            // Small one-tile launches (every wave at most one tile, at most 4
            // tiles a CU) leave out the ring refill, which would load nothing
            // but still queue a round of loads at the wave's end: 256 x 512
            // 3.69 -> 3.38 us, 1024 x 1024 3.71 -> 3.43, 2048 x 2048 3.80 ->
            // 3.57.  (Larger one-tile launches measured slower that way:
            // 11008 x 2048 4.80 -> 4.89, 16384 x 2048 5.5 -> 5.8.)
            const int64_t tiles = (M + NR - 1) / NR;
            const bool one = !MULTI && !STRIDED && tiles <= ngroups && tiles <= 4LL * cu_count();
            if (scale_runs_aligned(scales, nullptr, K))
                fn = one ? reinterpret_cast<const void *>(&gemv_kernel<NR, CPL, S, RG, MULTI, STRIDED, true, true>)
                         : reinterpret_cast<const void *>(&gemv_kernel<NR, CPL, S, RG, MULTI, STRIDED, true>);
        }
        return hipLaunchKernel(fn, dim3((unsigned)grid), dim3((unsigned)(P * G)), args, 0, stream);
    }
}

// Workgroups for `tiles` tiles of NR rows, G groups per workgroup: two
// workgroups fit a CU (64 KB of LDS each), one pass over the grid.
int64_t gemv_grid(int64_t tiles, int G) {
    const int64_t max_wg = 2LL * cu_count();
    int64_t grid = (tiles + G - 1) / G;
    if (grid > max_wg) grid = max_wg;
    return grid < 1 ? 1 : grid;
}

// Rows of one wave (at most 64 chunks): the most tiles one pass of the
// one-tile-per-wave form covers (two workgroups of 16 waves per CU).
int64_t one_tile_limit() { return 2LL * 16 * cu_count(); }

// Rows of one wave, one matrix per launch: beyond 16 four-row tiles per CU
// the tiles are dealt to the waves in turn (the strided order), one tile at
// a time, in two workgroups of G waves per CU: G = 8 up to 32 tiles per CU,
// else 12.  Measured (lab, same run): 22016 x 2048 7.10 -> 6.45 us (against
// one tile per wave in 11-wave workgroups), 151936 x 2048 28.9 -> 27.7 us
// (against a ring of two tiles over contiguous row ranges).  A ring of two
// tiles over the strided order gained nothing (a spill-free lab kernel:
// 151936 x 2048 27.2-27.65 against 27.0-27.7 us, 22016 x 2048 7.3-8.0
// against 6.4), and up to 16 tiles per CU one tile per wave stays best
// (11008 x 2048 4.79 against 4.84-5.5 us strided).
int64_t strided_from() { return 2LL * 8 * cu_count(); }
int strided_waves(int64_t tiles) { return tiles <= one_tile_limit() ? 8 : 12; }

// Workgroup shape of the one-tile-per-wave form for `tiles` row tiles: one
// wave per tile, in one workgroup per CU while that takes at most 12 waves,
// else two; at least 4 waves and enough threads for the workgroup's copy of
// the activations (one 16-byte unit per thread).  Measured on 11008 x 2048 and
// 22016 x 2048: 4.7 and 7.0 us against 5.2 and 7.2 us for 8-wave workgroups
// at two per CU, which leave a third of the waves two tiles in sequence
// (11008 rows: 344 workgroups, two on some CUs and one on others).
struct OneTileShape {
    int G;          // lane groups per workgroup (waves, for rows of one wave)
    int64_t cap;    // most workgroups
};
OneTileShape one_tile_shape(int64_t tiles, int K) {
    const int64_t cus = cu_count();
    const int64_t per_cu = tiles <= 12 * cus ? 1 : 2;
    int64_t G = (tiles + per_cu * cus - 1) / (per_cu * cus);
    // At least 4 waves a workgroup: each workgroup fills the whole 64 KB
    // table, and one or two waves alone take longer to fill it than the rest
    // of a small launch (256 x 512: 4.61 us with 1 wave, 3.78 with 2, 3.58
    // with 4; 1024 x 1024: 3.85 with 2, 3.66 with 4; lab, same run).
    const int64_t gmin = (K / 8 + 63) / 64 > 4 ? (K / 8 + 63) / 64 : 4;
    if (G < gmin) G = gmin;
    if (G < 1) G = 1;
    if (G > 16) G = 16;
    return {(int)G, per_cu * cus};
}

// Groups per workgroup for rows spanning `wpg` waves (one chunk a lane, at
// most 512 chunks): up to about 16 waves per CU, in one workgroup per CU
// when that covers every tile once, else in two.  Each group takes one 4-row
// tile at a time.  Measured (lab sweep of the group count and the ring, same run):
// 2048 x 11008 5.50 -> 5.21 us (2 groups of 6 waves), 5120 x 5120 7.61 ->
// 5.75 (5 of 3), 27648 x 5120 18.9 -> 16.2 (2 of 3, two per CU), 8192 x 8192
// 9.28 -> 8.82 (2 of 4), 4096 x 14336 8.54 -> 8.55 (1 of 7); a ring of two
// tiles per group, or 24-32 waves per CU, was slower on every shape.
OneTileShape multi_shape(int64_t tiles, int wpg, int max_waves = 16) {
    const int64_t cus = cu_count();
    const int gmax = max_waves / wpg > 0 ? max_waves / wpg : 1;
    // Groups of more than 8 waves stay one workgroup per CU (28 waves per CU
    // measured slower than 14 on 5120 x 27648: 17.1 against 15.5 us).
    const int64_t per_cu = (tiles <= cus * gmax || 2 * wpg > 16) ? 1 : 2;
    // No more groups per workgroup than the tiles need: a small matrix keeps
    // one workgroup on every CU it can reach.
    int64_t G = gmax / per_cu;
    const int64_t need = (tiles + per_cu * cus - 1) / (per_cu * cus);
    if (G > need) G = need;
    // ... but at least 4 waves a workgroup, which share the table fill
    // (1024 x 4096: 4.22 -> 3.98 us, 300 x 4096: 4.14 -> 3.91 with two groups
    // of 2 waves instead of one; lab, same run).
    const int64_t gmin = (4 + wpg - 1) / wpg;
    if (G < gmin) G = gmin < gmax ? gmin : gmax;
    if (G < 1) G = 1;
    return {(int)G, per_cu * cus};
}

// Workgroups per segment (in proportion to its tiles of `lpt` outputs, G
// groups per workgroup, one pass over at most `cap` workgroups, by default
// two per CU) and each segment's row split.  Returns the grid; *tpg gets the
// largest number of tiles a lane group walks.
int64_t plan_segments(GemvSegs &segs, int lpt, int G, int64_t *tpg, int64_t cap = 0) {
    if (cap <= 0) cap = 2LL * cu_count();
    int64_t wg[kMaxSegs], total = 0;
    for (int i = 0; i < segs.n; ++i) {
        const int64_t tiles = (segs.s[i].rows + lpt - 1) / lpt;
        wg[i] = (tiles + G - 1) / G;
        if (wg[i] < 1) wg[i] = 1;
        total += wg[i];
    }
    if (total > cap)
        for (int i = 0; i < segs.n; ++i) {
            wg[i] = wg[i] * cap / total;
            if (wg[i] < 1) wg[i] = 1;
        }
    int64_t begin = 0, most = 0;
    for (int i = 0; i < segs.n; ++i) {
        const int64_t groups = wg[i] * G;
        segs.s[i].rows_q = segs.s[i].rows / groups;
        segs.s[i].rows_rem = (int32_t)(segs.s[i].rows % groups);
        segs.s[i].wg_begin = (int32_t)begin;
        const int64_t per = segs.s[i].rows_q + (segs.s[i].rows_rem ? 1 : 0);
        const int64_t t = (per + lpt - 1) / lpt;
        if (t > most) most = t;
        begin += wg[i];
    }
    *tpg = most;
    return begin;
}

template <int NR, int CPL, int S, int RG, bool MULTI, int MODE, bool STRIDED = false, int FMT = kFmtNf4>
hipError_t launch_fused_variant(GemvSegs segs, int K, const uint16_t *x, int P, int G, int64_t grid,
                                hipStream_t stream) {
    if (!MULTI && (K / 8 > P * G || K / 8 > kSharedXUnits)) return hipErrorInvalidValue;
    if (MODE == kModeSwiglu || segs.n == 1) {
        void *args[] = {&segs.s[0], &K, &x, &P};
        const void *fn =
            reinterpret_cast<const void *>(&gemv_fused1_kernel<NR, CPL, S, RG, MULTI, MODE, STRIDED, false, FMT>);
        // One run of scales (and zero points) a tile and matrix, for NF4 and
        // the affine format in every order (affine SwiGLU on the 11008 x 2048
        // pair in the strided order: 8.31 against 8.71 us per row); the
        // NVFP4-style scales are read per chunk.
        if constexpr (CPL == 1 && S == 0 && NR <= 4 && FMT != kFmtNvfp4)
            if (scale_runs_aligned(segs.s[0].scales0, segs.s[0].scales1, K) &&
                (FMT != kFmtAffine || scale_runs_aligned(segs.s[0].zeros0, segs.s[0].zeros1, K)))
                fn = reinterpret_cast<const void *>(
                    &gemv_fused1_kernel<NR, CPL, S, RG, MULTI, MODE, STRIDED, true, FMT>);
        return hipLaunchKernel(fn, dim3((unsigned)grid), dim3((unsigned)(P * G)), args, 0, stream);
    }
    if (STRIDED) return hipErrorInvalidValue;  // the strided order serves one matrix
    if constexpr (MODE != kModeSwiglu) {
        void *args[] = {&segs, &K, &x, &P};
        return hipLaunchKernel(reinterpret_cast<const void *>(&gemv_fused_kernel<NR, CPL, S, RG, MULTI, MODE, FMT>),
                               dim3((unsigned)grid), dim3((unsigned)(P * G)), args, 0, stream);
    }
    return hipErrorInvalidValue;
}

// The variant for the row length, as launch_gemv chooses it (rows of up to
// 512 chunks, K <= 16384).
template <int MODE, int FMT>
hipError_t launch_fused_mode(GemvSegs segs, int K, const uint16_t *x, hipStream_t stream) {
    const int C = K / kChunkWeights;
    constexpr int half = MODE == kModeSwiglu ? 2 : 1;  // rows per output
    int64_t tpg = 0;
    if (C <= 64) {
        const int lpt = 4 / half;
        int64_t tiles = 0;
        for (int i = 0; i < segs.n; ++i) tiles += (segs.s[i].rows + lpt - 1) / lpt;
        const bool one_matrix = MODE == kModeSwiglu || segs.n == 1;
        if (one_matrix && tiles > strided_from()) {
            const int G = strided_waves(tiles);
            const int64_t grid = plan_segments(segs, lpt, G, &tpg, 2LL * cu_count());
            return launch_fused_variant<4, 1, 0, 4, false, MODE, true, FMT>(segs, K, x, 64, G, grid, stream);
        }
        if (tiles <= one_tile_limit()) {
            const OneTileShape sh = one_tile_shape(tiles, K);
            const int64_t grid = plan_segments(segs, lpt, sh.G, &tpg, sh.cap);
            return launch_fused_variant<4, 1, 0, 4, false, MODE, false, FMT>(segs, K, x, 64, sh.G, grid, stream);
        }
        const int64_t grid = plan_segments(segs, lpt, 8, &tpg);
        return launch_fused_variant<4, 1, 1, 8, false, MODE, false, FMT>(segs, K, x, 64, 8, grid, stream);
    }
    if (C <= 64 * kMaxWavesPerGroup) {
        const int wpg = (C + 63) / 64;
        const int lpt = 4 / half;
        int64_t tiles = 0;
        for (int i = 0; i < segs.n; ++i) tiles += (segs.s[i].rows + lpt - 1) / lpt;
        const OneTileShape sh = multi_shape(tiles, wpg);
        const int64_t grid = plan_segments(segs, lpt, sh.G, &tpg, sh.cap);
        return launch_fused_variant<4, 1, 0, 4, true, MODE, false, FMT>(segs, K, x, wpg * 64, sh.G, grid, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

namespace {

template <int FMT>
hipError_t launch_gemv_fused_fmt(const FusedOperand *ops, int count, bool swiglu, int64_t K, const uint16_t *x,
                                 float *const *y, const float *const *residual, hipStream_t stream) {
    GemvSegs segs{};
    if (swiglu) {
        if (count != 2 || ops[0].M != ops[1].M) return hipErrorInvalidValue;
        if (ops[0].M == 0) return hipSuccess;
        GemvSeg &g = segs.s[0];
        g.codes0 = ops[0].codes;
        g.scales0 = ops[0].scales;
        g.zeros0 = ops[0].zeros;
        g.tscale = ops[0].tscale;
        g.bias0 = ops[0].bias;
        g.codes1 = ops[1].codes;
        g.scales1 = ops[1].scales;
        g.zeros1 = ops[1].zeros;
        g.tscale1 = ops[1].tscale;
        g.bias1 = ops[1].bias;
        g.residual = residual ? residual[0] : nullptr;
        g.y = y[0];
        g.rows = ops[0].M;
        segs.n = 1;
        return launch_fused_mode<kModeSwiglu, FMT>(segs, (int)K, x, stream);
    }
    if (count < 1 || count > kMaxSegs) return hipErrorInvalidValue;
    for (int i = 0; i < count; ++i) {
        if (ops[i].M == 0) continue;
        GemvSeg &g = segs.s[segs.n++];
        g.codes0 = ops[i].codes;
        g.scales0 = ops[i].scales;
        g.zeros0 = ops[i].zeros;
        g.tscale = ops[i].tscale;
        g.bias0 = ops[i].bias;
        g.residual = residual ? residual[i] : nullptr;
        g.y = y[i];
        g.rows = ops[i].M;
    }
    if (segs.n == 0) return hipSuccess;
    return launch_fused_mode<kModeEpi, FMT>(segs, (int)K, x, stream);
}

}  // namespace

hipError_t launch_gemv_fused(int fmt, const FusedOperand *ops, int count, bool swiglu, int64_t K, const uint16_t *x,
                             float *const *y, const float *const *residual, hipStream_t stream) {
    switch (fmt) {
        case kGemmNf4:
            return launch_gemv_fused_fmt<kFmtNf4>(ops, count, swiglu, K, x, y, residual, stream);
        case kGemmAffine:
            return launch_gemv_fused_fmt<kFmtAffine>(ops, count, swiglu, K, x, y, residual, stream);
        case kGemmNvfp4:
            return launch_gemv_fused_fmt<kFmtNvfp4>(ops, count, swiglu, K, x, y, residual, stream);
        default:
            return hipErrorInvalidValue;
    }
}

// Variant choice (by measurement).  Rows of one wave (K <= 2048): one 4-row
// tile per wave while the grid covers the matrix in one pass, else 4-row
// tiles dealt to the waves in turn, one at a time (the strided order: the
// grid reads one moving stretch of the matrix; the lm_head and gate/up
// shapes).  Longer rows: groups of waves share
// 4-row tiles, one tile at a time, sized by multi_shape; the longest rows
// take several chunks a lane (4-row tiles in a ring of two at 4 chunks, one
// row at a time at 8).
template <int FMT>
hipError_t launch_gemv_fmt(const uint8_t *codes, const uint16_t *scales, const void *extra, int64_t M,
                           int64_t K, const uint16_t *x, float *y, hipStream_t stream) {
    const int C = (int)(K / kChunkWeights);
    const int k = (int)K;
    const int64_t tiles4 = (M + 3) / 4;
    if (C <= 64) {  // one wave covers a row: independent waves
        if (tiles4 <= strided_from()) {
            const OneTileShape sh = one_tile_shape(tiles4, k);
            int64_t grid = (tiles4 + sh.G - 1) / sh.G;
            if (grid > sh.cap) grid = sh.cap;
            return launch_variant<4, 1, 0, 4, false, FMT>(codes, scales, extra, M, k, x, y, 64, sh.G, grid, stream);
        }
        return launch_variant<4, 1, 0, 4, false, FMT, true>(codes, scales, extra, M, k, x, y, 64,
                                                            strided_waves(tiles4), 2LL * cu_count(), stream);
    }
    // Longer rows: a group of waves shares a row tile.  One chunk a lane for
    // rows of up to 1024 chunks (groups of up to 16 waves, several groups per
    // workgroup when they are small; for rows of 65..128 chunks this measured
    // 8.4 against 11.7 us on 14336 x 4096 and 4.6 against 7.3 us on
    // 4096 x 4096 for one wave per row at two chunks a lane); longer rows take
    // 4 or 8 chunks a lane in groups of up to 8 waves.
    int cpl = 1;
    if (C > 64 * kMaxWavesPerBlock)
        while (C > cpl * 64 * kMaxWavesPerGroup) cpl *= 2;
    const int waves = (C + cpl * 64 - 1) / (cpl * 64);
    const int P = waves * 64;
    switch (cpl) {
        case 1: {
            const OneTileShape sh = multi_shape(tiles4, waves);
            int64_t grid = (tiles4 + sh.G - 1) / sh.G;
            if (grid > sh.cap) grid = sh.cap;
            return launch_variant<4, 1, 0, 4, true, FMT>(codes, scales, extra, M, k, x, y, P, sh.G, grid, stream);
        }
        case 4: {
            const int64_t tiles2 = (M + 1) / 2;
            return launch_variant<2, 4, 1, 4, true, FMT>(codes, scales, extra, M, k, x, y, P, 1, gemv_grid(tiles2, 1), stream);
        }
        default:
            return launch_variant<1, 8, 0, 2, true, FMT>(codes, scales, extra, M, k, x, y, P, 1, gemv_grid(M, 1), stream);
    }
}

// Chunks of 2 or 3 tokens on rows of one wave, in one workgroup of at most
// 12 waves per CU (the table and the activations take up to 88 KB of LDS;
// a wave holds 16 VGPRs of activations per token; 4 tokens spill).
bool gemv_tokens_fits(int64_t M, int64_t K, int64_t N) {
    return N >= 2 && N <= 3 && K <= 64 * kChunkWeights && (M + 3) / 4 <= 12LL * cu_count();
}

namespace {
template <int NTOK>
const void *gemv_tokens_fn(bool ts) {
    return ts ? reinterpret_cast<const void *>(&gemv_tokens_kernel<NTOK, true>)
              : reinterpret_cast<const void *>(&gemv_tokens_kernel<NTOK, false>);
}
template <int NTOK, int FMT>
const void *gemv_tokens_multi_fn(bool ts) {
    if constexpr (FMT == kFmtNvfp4)  // (no one-load scale runs for E4M3 bytes)
        return reinterpret_cast<const void *>(&gemv_tokens_multi_kernel<NTOK, FMT, false>);
    else
        return ts ? reinterpret_cast<const void *>(&gemv_tokens_multi_kernel<NTOK, FMT, true>)
                  : reinterpret_cast<const void *>(&gemv_tokens_multi_kernel<NTOK, FMT, false>);
}
template <int FMT>
const void *gemv_tokens_multi_fn(int64_t N, bool ts) {
    return N == 2 ? gemv_tokens_multi_fn<2, FMT>(ts) : N == 3 ? gemv_tokens_multi_fn<3, FMT>(ts)
                                                            : gemv_tokens_multi_fn<4, FMT>(ts);
}
}  // namespace

hipError_t launch_gemv_tokens_multi(int fmt, const uint8_t *codes, const void *scales_v, const uint16_t *zeros,
                                    const float *tscale, int64_t M, int64_t K, const uint16_t *X, int64_t N, float *Y,
                                    hipStream_t stream) {
    // (The E4M3 bytes of the NVFP4-style format are read two at a time, as
    // one 16-bit value per 32-weight chunk.)
    const uint16_t *scales = static_cast<const uint16_t *>(scales_v);
    if (!gemv_tokens_multi_fits(M, K, N)) return hipErrorInvalidValue;
    int k = (int)K;
    const int C = k / kChunkWeights;
    const int waves = (C + 63) / 64;
    int P = waves * 64;
    const int64_t tiles4 = (M + 3) / 4;
    const int max_waves = N == 2 ? tokens_multi_waves(2) : tokens_multi_waves(3);
    const OneTileShape sh = multi_shape(tiles4, waves, max_waves);
    if (sh.G * waves > max_waves) return hipErrorInvalidValue;
    int64_t grid = (tiles4 + sh.G - 1) / sh.G;
    if (grid > sh.cap) grid = sh.cap;
    const int64_t ngroups = grid * sh.G;
    int64_t rows_q = M / ngroups;
    int rows_rem = (int)(M % ngroups);
    const bool ts = scale_runs_aligned(scales, fmt == kGemmAffine ? zeros : nullptr, k);
    const void *fn = fmt == kGemmAffine ? gemv_tokens_multi_fn<kFmtAffine>(N, ts)
                     : fmt == kGemmNvfp4 ? gemv_tokens_multi_fn<kFmtNvfp4>(N, ts)
                                         : gemv_tokens_multi_fn<kFmtNf4>(N, ts);
    void *args[] = {&codes, &scales, &zeros, &tscale, &M, &k, &X, &Y, &P, &rows_q, &rows_rem};
    return hipLaunchKernel(fn, dim3((unsigned)grid), dim3((unsigned)(P * sh.G)), args, 0, stream);
}

hipError_t launch_gemv_tokens(const uint8_t *codes, const uint16_t *scales, int64_t M, int64_t K,
                              const uint16_t *X, int64_t N, float *Y, hipStream_t stream) {
    if (!gemv_tokens_fits(M, K, N)) return hipErrorInvalidValue;
    int k = (int)K;
    const int64_t tiles4 = (M + 3) / 4;
    const OneTileShape sh = one_tile_shape(tiles4, k);
    int64_t grid = (tiles4 + sh.G - 1) / sh.G;
    if (grid > sh.cap) grid = sh.cap;
    int P = 64;
    if (k / 8 > P * sh.G || sh.G > 12) return hipErrorInvalidValue;  // at most 768 threads
    const int64_t ngroups = grid * sh.G;
    int64_t rows_q = M / ngroups;
    int rows_rem = (int)(M % ngroups);
    const bool ts = scale_runs_aligned(scales, nullptr, k);
    const void *fn = N == 2 ? gemv_tokens_fn<2>(ts) : gemv_tokens_fn<3>(ts);
    void *args[] = {&codes, &scales, &M, &k, &X, &Y, &P, &rows_q, &rows_rem};
    return hipLaunchKernel(fn, dim3((unsigned)grid), dim3((unsigned)(P * sh.G)), args, 0, stream);
}

hipError_t launch_gemv(const uint8_t *codes, const uint16_t *scales, int64_t M, int64_t K, const uint16_t *x,
                       float *y, hipStream_t stream) {
    return launch_gemv_fmt<kFmtNf4>(codes, scales, nullptr, M, K, x, y, stream);
}

hipError_t launch_gemv_affine(const uint8_t *codes, const uint16_t *scales, const uint16_t *zeros, int64_t M,
                              int64_t K, const uint16_t *x, float *y, hipStream_t stream) {
    return launch_gemv_fmt<kFmtAffine>(codes, scales, zeros, M, K, x, y, stream);
}

hipError_t launch_gemv_affine_x8(const uint8_t *codes, const uint16_t *scales, const uint16_t *zeros, int64_t M,
                                 int64_t K, const int8_t *q1, const int8_t *q2, const float *d, float *y,
                                 hipStream_t stream) {
    const X8Args xa{zeros, q1, q2, d};
    if (q2) return launch_gemv_fmt<kFmtAffineX8x2>(codes, scales, &xa, M, K, nullptr, y, stream);
    return launch_gemv_fmt<kFmtAffineX8>(codes, scales, &xa, M, K, nullptr, y, stream);
}

hipError_t launch_gemv_nvfp4(const uint8_t *codes, const uint8_t *scales, const float *tscale, int64_t M,
                             int64_t K, const uint16_t *x, float *y, hipStream_t stream) {
    // Two E4M3 bytes per 32-weight chunk are read as one 16-bit value.
    return launch_gemv_fmt<kFmtNvfp4>(codes, reinterpret_cast<const uint16_t *>(scales), tscale, M, K, x, y,
                                      stream);
}

}  // namespace q4
