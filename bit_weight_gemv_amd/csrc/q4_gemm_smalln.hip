// q4_gemm_smalln.hip -- Y[n][m] = sum_k What[m,k] * X[n][k] for a prefill chunk of N <= 32 tokens,
// for the NF4 codebook format and the affine and NVFP4-style formats.
//
// What is computed: the prefill form of the deep-fold "Decode V2" page
// (section 0: prompts run as chunks of up to 32 tokens through a dedicated
// matrix-core product) -- the same representation and reconstruction as the
// vector form (golang.design accel/tensor, func Int4MatMul), with the matrix
// read once per chunk of tokens and the unpacking amortised over the chunk.
// The affine format is accel/tensor's type Int4 (What = (code - z) * s per
// 64-block); the NVFP4-style format is gizai tensor/lazy's fp4Blocks (E2M1
// codes, one E4M3 scale per 16 values, an f32 tensor scale).
//
// gfx950 design:
//  * Matrix cores.  v_mfma_f32_16x16x32_f16 multiplies a 16-token x 32-k
//    slab of X (operand A) by a 32-k x 16-row slab of dequantised weights
//    (operand B) into a 16 x 16 fp32 tile; chunks of 17..32 tokens take two
//    MFMAs per slab of weights, so each dequantised weight feeds every token.
//    Lane l of an operand holds row/token l % 16 and eight k of group l / 16;
//    within a 64-block, k-group g of MFMA step s is k = 16g + 8s + (0..7)
//    (a fixed permutation of k, the same for X and W), so a lane's codes for
//    one block are 8 contiguous bytes.
//  * Dequantisation.  The LDS byte -> fp16-pair table (one ds_read_b32 per
//    two weights; the 64-copy layout keeps random codes conflict-free).
//    NF4: the fp32 result of a block's two MFMAs is multiplied by the block
//    scale of the lane's weight row (fp32 FMA): levels round to fp16 (2^-11
//    relative) and nothing else is rounded below fp32.  Affine: the table
//    holds code - 8 and z - 8 is subtracted from every pair before the MFMA
//    (a packed fp16 subtract of small integers, exact), so each term is
//    (code - z) x; then the block scale as for NF4.  NVFP4: each E2M1 pair
//    is multiplied by its 16-block's E4M3 scale in fp16 before the MFMA
//    (E2M1 has at most 2 and E4M3 at most 4 significant bits, so the
//    product is exact and within fp16's normal range), the tiles accumulate
//    across blocks, and the tensor scale multiplies the finished sums.
//  * Activations.  The workgroup's waves split K into slices of 256 (four
//    blocks); a wave converts its slice of X to fp16 once, each token scaled
//    by a power of two chosen from that token's largest magnitude in the
//    slice, and keeps it in registers for every row tile it visits.  The
//    inverse scale is applied to the wave's partial sums.  The conversion is
//    exact while no nonzero value of a token's slice lies more than 2^28
//    below that token's largest (each lane tests its own values; one ballot
//    decides for the wave).  A wave whose slice is not held exactly keeps
//    the raw bf16 values instead and multiplies them with
//    v_mfma_f32_16x16x4_f32 (fp32 operands, exact products): eight such
//    MFMAs per 32-k slab, the same accumulator layout.  Slower, and only for
//    inputs that need it.
//  * Schedule.  Row tiles of 16 rows are split into contiguous ranges, one
//    per workgroup (one workgroup per CU); the waves walk the range in step
//    with a ring of prefetched tiles (codes and scales of tile t+1 .. t+S are
//    in flight while tile t is multiplied).  The waves' partial tiles are
//    summed through LDS, once per group of tiles.
//  * Long rows with scratch memory (the *_ws entry points).  K is cut into
//    ranges of at most 8 slices (2048 weights); each workgroup takes one
//    range of one row range, keeps that range's activations in registers
//    for all its tiles, and writes a partial plane; a second launch adds the
//    planes in range order.  Without scratch, rows longer than 8 slices
//    reload each slice of the activations for every tile.
#include <mutex>
#include <type_traits>

#include "q4_device.h"
#include "q4_internal.h"
#include "q4_lut.h"

namespace q4 {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));


constexpr int kGemmMaxWaves = 8;   // workgroup: up to 8 waves, one K slice each
constexpr int kSliceBlocks = 4;    // 64-blocks per K slice (256 k)
constexpr int kTileRows = 16;

// Loads are laid out for the memory pipeline, not for the MFMA: a load
// instruction whose neighbouring lanes read neighbouring 16-byte pieces of
// one row is served at full rate, while the operand layout (neighbouring
// lanes on different rows) costs about one request per lane.  Activations
// and codes are therefore loaded row-contiguously and regrouped into operand
// order through a per-wave LDS area.

// Per-wave LDS staging, in 16-byte units.  Activations: 16 tokens x 512 bytes
// (one token half of a slice), row pitch 33 units; codes: 16 rows x 128
// bytes (one tile of a slice), row pitch 9 units.  Pitches are odd so the
// 16 rows of an operand read fall in different banks.
constexpr int kXPitch = 33;
constexpr int kXStageUnits = 16 * kXPitch;
constexpr int kCPitch = 9;
constexpr int kCStageUnits = 16 * kCPitch;

// This wave's slice of X, row-contiguously: piece p = 64 i + lane (16 bytes)
// is token p / 32, bytes 16 (p % 32) of the slice.  Tokens past N and blocks
// past the row's end read as zero (offsets past the buffer).  Only the first
// XP token pairs are loaded (XP covers N, fixed at compile time so the wait
// counts stay static); the rest are zero without a load, so a small chunk
// does not queue dead requests in the memory pipeline.
template <int NT, int XP>
__device__ __forceinline__ void load_x_linear(__amdgpu_buffer_rsrc_t xrs, int K, int nsb, int slice,
                                              u32x4_t (&lin)[NT * 8]) {
    static_assert(XP >= 1 && XP <= NT * 8, "token pairs loaded");
    const int lane = threadIdx.x & 63;
    const int within = lane & 31;
    const int blk = slice * kSliceBlocks + (within >> 3);
    // All ones for a block past the row's end: the offset then lies past the
    // buffer (arithmetic, so the loads stay unconditional).
    const int past = (nsb - 1 - blk) >> 31;
#pragma unroll
    for (int i = 0; i < NT * 8; ++i) {
        const int tok = 2 * i + (lane >> 5);
        const int off = ((tok * K + 256 * slice + 8 * within) * 2) | (past & 0x7FFFFFF0);
        lin[i] = i < XP ? __builtin_amdgcn_raw_buffer_load_b128(xrs, off, 0, 0) : u32x4_t{0u, 0u, 0u, 0u};
    }
}

// Regroup through the wave's staging area into operand order: lane (j, g)
// gets token 16t + j, k = 64b + 16g + 8s + (0..7) of the slice for block b,
// step s.  One token half at a time; LDS operations of a wave complete in
// order, so each half's reads finish before the next half's writes.
template <int NT>
__device__ __forceinline__ void regroup_x(uint4 *xs, const u32x4_t (&lin)[NT * 8],
                                          u32x4_t (&raw)[NT][kSliceBlocks][2]) {
    const int lane = threadIdx.x & 63;
    const int j = lane & 15, g = lane >> 4;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int tok = 2 * i + (lane >> 5);
            const u32x4_t v = lin[8 * t + i];
            xs[tok * kXPitch + (lane & 31)] = make_uint4(v.x, v.y, v.z, v.w);
        }
#pragma unroll
        for (int b = 0; b < kSliceBlocks; ++b)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const uint4 v = xs[j * kXPitch + 8 * b + 2 * g + s];
                raw[t][b][s] = u32x4_t{v.x, v.y, v.z, v.w};
            }
    }
}

// Prepare the slice's activations per token: lanes j, j+16, j+32, j+48 hold
// token j's values; the biased exponent Emax of their largest bf16
// magnitude fixes the power of two 2^e, e = 141 - Emax, that puts it in
// [2^14, 2^15).  A bf16 value of exponent E then has the fp16 exponent
// E - Emax + 29, so the conversion is integer arithmetic on the bits:
// subtract (Emax - 29) << 7 from the magnitude (saturating: zero stays
// zero), shift left by 3 (7 to 10 mantissa bits), restore the sign.  It is
// exact when every nonzero value is an fp16 normal number after scaling
// (E >= Emax - 28: each lane tests its smallest nonzero magnitude, found as
// 1 + the minimum of magnitude - 1 taken modulo 2^16 so that zeros drop
// out) and Emax is 29 .. 254 (a slice of zeros counts as exact); one
// ballot makes the decision for the wave.
// Exact: xa holds the fp16 values and inv[t][r] the inverse power of two of
// the token of output register r (token 4g + r of half t), times `post`.
// Otherwise xa keeps the raw bf16 bits and inv[t][r] = post.  Returns
// whether the fp16 form is exact.  (Against an fp32 multiply and round per
// value this is ~20% fewer instructions in a set-up every wave runs before
// the workgroup barrier.)
template <int NT>
__device__ __forceinline__ bool prepare_x_slice(const u32x4_t (&raw)[NT][kSliceBlocks][2],
                                                half8_t (&xa)[NT][kSliceBlocks][2], float (&inv)[NT][4],
                                                float post) {
    const int lane = threadIdx.x & 63;
    int emax[NT];
    bool ok = true;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        u16x2_t mx = {0, 0};
        u16x2_t mn = {0xFFFF, 0xFFFF};
#pragma unroll
        for (int b = 0; b < kSliceBlocks; ++b)
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const u16x2_t mag = __builtin_bit_cast(u16x2_t, raw[t][b][s][c] & 0x7FFF7FFFu);
                    mx = __builtin_elementwise_max(mx, mag);
                    mn = __builtin_elementwise_min(mn, mag - u16x2_t{1, 1});
                }
        int m = (int)(mx.x > mx.y ? mx.x : mx.y);
        m = max(m, __shfl_xor(m, 16));
        m = max(m, __shfl_xor(m, 32));
        // (A token whose slice is all zeros, such as the padding tokens
        // past N, is held exactly by any scale: Emax 29 stands in.)
        const int E = m == 0 ? 29 : m >> 7;
        emax[t] = E;
        const uint32_t lo = mn.x < mn.y ? mn.x : mn.y;
        ok = ok && E >= 29 && E <= 254 && (lo == 0xFFFFu || lo + 1u >= ((uint32_t)(E - 28) << 7));
    }
    const bool exact = __builtin_amdgcn_ballot_w64(!ok) == 0;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        float down = post;
        if (exact) {
            down *= exp2i(emax[t] - 141);
            const unsigned short sb = (unsigned short)((emax[t] - 29) << 7);
            const u16x2_t sub = {sb, sb};
#pragma unroll
            for (int b = 0; b < kSliceBlocks; ++b)
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    u32x4_t h;
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const uint32_t w = raw[t][b][s][c];
                        const u16x2_t f =
                            __builtin_elementwise_sub_sat(__builtin_bit_cast(u16x2_t, w & 0x7FFF7FFFu), sub)
                            << u16x2_t{3, 3};
                        h[c] = (w & 0x80008000u) | __builtin_bit_cast(uint32_t, f);
                    }
                    xa[t][b][s] = __builtin_bit_cast(half8_t, h);
                }
        } else {
#pragma unroll
            for (int b = 0; b < kSliceBlocks; ++b)
#pragma unroll
                for (int s = 0; s < 2; ++s) xa[t][b][s] = __builtin_bit_cast(half8_t, raw[t][b][s]);
        }
        // Output register r of lane l belongs to token 4 (l / 16) + r, whose
        // scale lane 4 (l / 16) + r computed.
#pragma unroll
        for (int r = 0; r < 4; ++r) inv[t][r] = __shfl(down, 4 * (lane >> 4) + r);
    }
    return exact;
}

// One 32-k slab: acc + X (16 tokens x 32 k) . W (32 k x 16 rows).  EXACT:
// the fp16 MFMA.  Otherwise x holds raw bf16 bits: element e of every lane
// (k = 8 (l / 16) + e of the slab) is widened to fp32, as is the weight, and
// v_mfma_f32_16x16x4_f32 adds the products over the four k groups; the
// eight such products cover the slab (exact: 8 x 11 significant bits).
template <bool EXACT>
__device__ __forceinline__ float4_t slab_mfma(const half8_t &x, const half8_t &w, float4_t acc) {
    if constexpr (EXACT) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(x, w, acc, 0, 0, 0);
    } else {
        // (Each dword is passed through an empty asm so that its widening is
        // redone per use: the activations are loop-invariant, and widening
        // them all once would hold 8 registers per slab across the loop.)
        const u32x4_t xr = __builtin_bit_cast(u32x4_t, x);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            uint32_t d = xr[c];
            __asm__ volatile("" : "+v"(d));
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__builtin_bit_cast(float, d << 16), (float)w[2 * c], acc, 0,
                                                       0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__builtin_bit_cast(float, d & 0xFFFF0000u), (float)w[2 * c + 1],
                                                       acc, 0, 0, 0);
        }
        return acc;
    }
}

template <int NT, int S, bool XFIXED, int XP, int FMT>
__global__ __launch_bounds__(64 * kGemmMaxWaves) void gemm_smalln_kernel(
    const uint8_t *__restrict__ codes, const void *__restrict__ scales, const uint16_t *__restrict__ zeros,
    const float *__restrict__ tscale, int64_t M, int K, const uint16_t *__restrict__ X, int N,
    float *__restrict__ Y, int64_t tiles_q, int tiles_rem, int kranges, float *__restrict__ part) {
    // One block of LDS with the table at address 0, so a lookup address
    // built by v_perm needs no base added (the 16-bit offset field of a DS
    // instruction cannot hold a base past 64 KB).  Activation staging is
    // used during set-up only (and per unit on the long-row path); the same
    // bytes hold the partial tiles of the cross-wave sum.
    struct Smem {
        uint32_t lut[kLutDwords];
        uint4 xstage[kGemmMaxWaves * kXStageUnits];
        uint4 cstage[kGemmMaxWaves * kCStageUnits];
    };
    __shared__ Smem sm;
    uint32_t *lut = sm.lut;
    // Partial tiles of the cross-wave sum.  Activations kept in registers
    // (XFIXED): each wave writes the partial tiles of up to kGroupTiles
    // consecutive tiles into its own staging area, [tile][lane][register],
    // and the workgroup sums them once per group (one barrier per group, not
    // per tile, so the waves run through a group's tiles independently).
    // Long rows restage activations per tile in that area, so they use a
    // double-buffered [buffer][wave][lane][register] sum per tile instead.
    constexpr int kGroupTiles = XFIXED ? (NT == 1 ? 8 : 4) : 1;
    typedef float WavePart[kGroupTiles][64][NT * 4];
    static_assert(sizeof(WavePart) <= kXStageUnits * sizeof(uint4), "partial tiles must fit a wave's staging area");
    typedef float RedBuf[2][kGemmMaxWaves][64][NT * 4];
    static_assert(sizeof(RedBuf) <= sizeof(sm.xstage), "reduction buffer must fit the staging area");
    RedBuf &red = *reinterpret_cast<RedBuf *>(sm.xstage);
    auto wave_part = [&](int w) -> WavePart & {
        return *reinterpret_cast<WavePart *>(sm.xstage + w * kXStageUnits);
    };

    // Always kGemmMaxWaves waves; waves past the last K slice load nothing
    // (zero-record resources, zero activations) and add exact zeros.
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    constexpr int nw = kGemmMaxWaves;
    const int j = lane & 15;  // token (operand A) / weight row (operand B) of this lane
    const int g = lane >> 4;  // k group
    const int nsb = K >> 6;
    const int nslices = (nsb + kSliceBlocks - 1) / kSliceBlocks;
    // Slices per wave: one when the waves cover K (XFIXED: the activations
    // stay in registers), else several, reloaded per unit.
    const int spw = XFIXED ? 1 : (nslices + nw - 1) / nw;
    // K split in `kranges` ranges of at most kGemmMaxWaves slices (rows
    // longer than that, activations in registers): workgroup b takes range
    // b % kranges of row range b / kranges and writes its sums into partial
    // plane b % kranges of `part` ([kranges][N][M]); a second pass adds the
    // planes.  With one range the sums go to Y.
    const int krange = kranges > 1 ? (int)(blockIdx.x % (unsigned)kranges) : 0;
    const int spr = kranges > 1 ? (nslices + kranges - 1) / kranges : nslices;  // slices per range
    const int slice0 = krange * spr;
    const int slice_end = min(nslices, slice0 + spr);
    const int row_bytes = K >> 1;
    // Scale plane: fp16 per 64-block (NF4, affine: also the zero points), or
    // one E4M3 byte per 16-block (NVFP4).
    const int sc_row_bytes = FMT == kGemmNvfp4 ? (K >> 4) : (nsb * 2);
    const int64_t wg = kranges > 1 ? (int64_t)(blockIdx.x / (unsigned)kranges) : (int64_t)blockIdx.x;  // row range
    const int64_t t_begin = wg * tiles_q + (wg < tiles_rem ? wg : tiles_rem);
    const int ntiles = (int)tiles_q + (wg < tiles_rem ? 1 : 0);
    const int nunits = ntiles * spw;  // (tile, slice) pairs of this wave
    uint4 *xs = sm.xstage + wave * kXStageUnits;
    uint4 *cs = sm.cstage + wave * kCStageUnits;
    // NVFP4: the tensor scale multiplies every finished sum (with the
    // activations' inverse power of two).
    const float post = FMT == kGemmNvfp4 ? *tscale : 1.0f;
    // Where the finished sums go: Y, or this range's partial plane.
    float *const dst = kranges > 1 ? part + (int64_t)krange * N * M : Y;

    const __amdgpu_buffer_rsrc_t xrs = buffer_rsrc(X, (uint32_t)N * (uint32_t)K * 2u);

    // Ring of prefetched units: the scales (and zero points) and codes of
    // one tile over one K slice, issued in that order.  Codes: 16 rows x 128
    // bytes, lane l takes row l / 8 (+ 8 for the second load), bytes
    // 16 (l % 8) of the slice.  Scales: one load per lane (the address
    // unit's cost is per instruction, so the unit's scales come in a single
    // one and lane shuffles hand them out): lane l takes row l / 4, 64-block
    // 4 slice + l % 4 -- its fp16 scale (NF4, affine; likewise the zero
    // point), or the dword of that block's four E4M3 bytes (NVFP4, one per
    // 16 k).  A block past the row's end reads past the buffer and gets 0.
    // The buffer resource of a unit starts at its tile and ends at the last
    // row of the matrix, so rows past M read as zero (their results are not
    // stored); units of the set-up's first S + 1 past the last load through
    // zero-record resources (no memory access, unconditional loads), and the
    // ring's refills stop at the last unit.
    const int c_off = (lane >> 3) * row_bytes + 16 * (lane & 7);
    const int s_row_off = (lane >> 2) * sc_row_bytes + (FMT == kGemmNvfp4 ? 4 : 2) * (lane & 3);
    u32x4_t qv[S + 1][2];
    uint32_t sc[S + 1];
    uint32_t zc[FMT == kGemmAffine ? S + 1 : 1];
    const uint8_t *ld_codes = codes + t_begin * kTileRows * row_bytes;
    const uint8_t *ld_scales = static_cast<const uint8_t *>(scales) + t_begin * kTileRows * sc_row_bytes;
    const uint8_t *ld_zeros = reinterpret_cast<const uint8_t *>(zeros) + t_begin * kTileRows * sc_row_bytes;
    int64_t ld_rows = M - t_begin * kTileRows;  // rows from the next tile to load to M
    int ld_unit = 0, ld_si = 0;
    auto load_unit = [&](int buf) {
        const bool real = ld_unit < nunits;
        const int slice = slice0 + wave + nw * ld_si;
        const int rows = ld_rows < kTileRows ? (int)ld_rows : kTileRows;
        const bool live = real && slice < slice_end;
        const uint32_t sbytes = live ? (uint32_t)(rows * sc_row_bytes) : 0u;
        const int sblk = kSliceBlocks * slice + (lane & 3);
        const int past = (nsb - 1 - sblk) >> 31;  // all ones past the row's end
        const int s_off = (s_row_off + (FMT == kGemmNvfp4 ? 16 : 8) * slice) | (past & 0x7FFFFFF0);
        if constexpr (FMT == kGemmNvfp4) {
            sc[buf] = __builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(ld_scales, sbytes), s_off, 0, kLoadNonTemporal);
        } else {
            sc[buf] = __builtin_amdgcn_raw_buffer_load_b16(buffer_rsrc(ld_scales, sbytes), s_off, 0, kLoadNonTemporal);
            if constexpr (FMT == kGemmAffine)
                zc[buf] = __builtin_amdgcn_raw_buffer_load_b16(buffer_rsrc(ld_zeros, sbytes), s_off, 0,
                                                               kLoadNonTemporal);
        }
        const __amdgpu_buffer_rsrc_t crs =
            buffer_rsrc(ld_codes + 128 * slice, live ? (uint32_t)(rows * row_bytes - 128 * slice) : 0u);
        qv[buf][0] = __builtin_amdgcn_raw_buffer_load_b128(crs, c_off, 0, kLoadNonTemporal);
        qv[buf][1] = __builtin_amdgcn_raw_buffer_load_b128(crs, c_off + 8 * row_bytes, 0, kLoadNonTemporal);
        // Keep the unit's loads together and in this order: the wait for a
        // unit's codes then covers its scales, and never a later unit's.
        __builtin_amdgcn_sched_barrier(0);
        ++ld_unit;
        if (XFIXED || ++ld_si == spw) {
            ld_si = 0;
            ld_codes += kTileRows * row_bytes;
            ld_scales += kTileRows * sc_row_bytes;
            ld_zeros += kTileRows * sc_row_bytes;
            ld_rows -= kTileRows;
        }
    };

    // Set-up: this wave's activations (when it keeps one slice for the whole
    // run), the first units, the table fill, then the activation regrouping
    // and preparation (which waits only for the activation loads: vector
    // loads complete in order) and the barrier that publishes the table.
    // (Measured on the 11008 x 2048 shape: issuing weight units ahead of the
    // activations, or the barrier before the conversion, is slower.)
    u32x4_t lin[NT * 8];
    u32x4_t raw[NT][kSliceBlocks][2];
    // (A wave past its range's last slice loads zeros: the slice index then
    // points past the row's end.)
    if (XFIXED) load_x_linear<NT, XP>(xrs, K, nsb, slice0 + wave < slice_end ? slice0 + wave : nslices, lin);
#pragma unroll
    for (int s = 0; s <= S; ++s) load_unit(s);
    if constexpr (FMT == kGemmAffine)
        fill_lut_from(lut, kAffinePairTable);
    else if constexpr (FMT == kGemmNvfp4)
        fill_lut_from(lut, kE2m1PairTable);
    else
        fill_lut(lut);
    half8_t xa[NT][kSliceBlocks][2];
    float inv[NT][4];
    bool xexact = true;
    if (XFIXED) {
        regroup_x<NT>(xs, lin, raw);
        xexact = prepare_x_slice<NT>(raw, xa, inv, post);
    }
    __syncthreads();

    const uint32_t laneoff = (uint32_t)lane << 2;
    float acc[NT][4];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[t][r] = 0.0f;
    int rbuf = 0;
    // Output of this thread in a tile's sum: token n = tid / 16, row
    // tid % 16; it is register 4 (n / 16) + n % 4 of lane
    // 16 ((n % 16) / 4) + row of every wave.
    static_assert(NT * 256 <= 64 * nw, "one output per thread");
    const int out_n = threadIdx.x >> 4, out_mm = threadIdx.x & 15;
    const int out_v = 4 * (out_n >> 4) + (out_n & 3);
    const int out_l = ((out_n & 15) >> 2) * 16 + out_mm;
    const int64_t out_base = (int64_t)out_n * M + out_mm;
    int cu_si = 0;               // slice index of the unit being consumed
    int64_t cu_m0 = t_begin * kTileRows;  // first row of its tile
    int gslot = 0;               // XFIXED: tile slot within the current group
    int tiles_done = 0;

    // XFIXED: the sums of the group's `nslot` tiles, whose first row is m0.
    // Thread (n, row) adds the eight waves' partials of its output in each
    // tile; every wave has written its partials before the barrier.
    auto sum_group = [&](int nslot, int64_t m0) {
        __syncthreads();
        if (out_n < N) {
            for (int t = 0; t < nslot; ++t) {
                float sum = 0.0f;
#pragma unroll
                for (int w = 0; w < nw; ++w) sum += wave_part(w)[t][out_l][out_v];
                const int64_t m = m0 + (int64_t)t * kTileRows + out_mm;
                if (m < M) dst[(int64_t)out_n * M + m] = sum;
            }
        }
    };

    // The unit's dequantised weights, then its MFMAs: EXACT selects the fp16
    // product or the exact fp32 one (activations held as raw bf16).
    auto multiply = [&](auto exact_tag, int buf, float (&part)[NT][4]) {
        constexpr bool EXACT = decltype(exact_tag)::value;
        // Regroup the codes: lane (j, g) takes bytes 32b + 8g (8 bytes) of
        // row j for block b.  All lookups of the unit are issued before the
        // first MFMA so the LDS latencies overlap.
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const u32x4_t v = qv[buf][q];
            cs[((lane >> 3) + 8 * q) * kCPitch + (lane & 7)] = make_uint4(v.x, v.y, v.z, v.w);
        }
        const char *crow = reinterpret_cast<const char *>(cs + j * kCPitch);
        uint2 qw[kSliceBlocks];
#pragma unroll
        for (int b = 0; b < kSliceBlocks; ++b) qw[b] = *reinterpret_cast<const uint2 *>(crow + 32 * b + 8 * g);
        half8_t bop[kSliceBlocks][2];
#pragma unroll
        for (int b = 0; b < kSliceBlocks; ++b) {
            // Per-block adjustment of the table pairs: affine subtracts
            // z - 8, NVFP4 multiplies by the lane's E4M3 scale (both exact
            // in fp16).
            // (The values of row j, block b sit in lane 4j + b.)
            half2_t adj = {0, 0};
            if constexpr (FMT == kGemmAffine) {
                const _Float16 z = (_Float16)(f16_bits_to_f32(__shfl(zc[buf], 4 * j + b) & 0xFFFFu) - 8.0f);
                adj = half2_t{z, z};
            } else if constexpr (FMT == kGemmNvfp4) {
                const uint32_t d = __shfl(sc[buf], 4 * j + b);
                const _Float16 v = (_Float16)e4m3_to_f32(d >> (8 * g));
                adj = half2_t{v, v};
            }
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const uint32_t w = s ? qw[b].y : qw[b].x;
                half2_t p0 = lut_pair<0>(lut, w, laneoff);
                half2_t p1 = lut_pair<1>(lut, w, laneoff);
                half2_t p2 = lut_pair<2>(lut, w, laneoff);
                half2_t p3 = lut_pair<3>(lut, w, laneoff);
                if constexpr (FMT == kGemmAffine) {
                    p0 -= adj; p1 -= adj; p2 -= adj; p3 -= adj;
                } else if constexpr (FMT == kGemmNvfp4) {
                    p0 *= adj; p1 *= adj; p2 *= adj; p3 *= adj;
                }
                bop[b][s] = half8_t{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
            }
        }
        if constexpr (FMT == kGemmNvfp4) {
            // Scales already in the weights: one accumulation over the slice.
            float4_t tile[NT];
#pragma unroll
            for (int t = 0; t < NT; ++t) tile[t] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int b = 0; b < kSliceBlocks; ++b)
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    tile[t] = slab_mfma<EXACT>(xa[t][b][0], bop[b][0], tile[t]);
                    tile[t] = slab_mfma<EXACT>(xa[t][b][1], bop[b][1], tile[t]);
                }
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) part[t][r] = tile[t][r];
        } else {
            float sb[kSliceBlocks];
#pragma unroll
            for (int b = 0; b < kSliceBlocks; ++b) sb[b] = f16_bits_to_f32(__shfl(sc[buf], 4 * j + b) & 0xFFFFu);
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) part[t][r] = 0.0f;
#pragma unroll
            for (int b = 0; b < kSliceBlocks; ++b) {
                float4_t tile[NT];
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    tile[t] = slab_mfma<EXACT>(xa[t][b][0], bop[b][0], float4_t{0.0f, 0.0f, 0.0f, 0.0f});
                    tile[t] = slab_mfma<EXACT>(xa[t][b][1], bop[b][1], tile[t]);
                }
#pragma unroll
                for (int t = 0; t < NT; ++t)
#pragma unroll
                    for (int r = 0; r < 4; ++r) part[t][r] = fmaf(tile[t][r], sb[b], part[t][r]);
            }
        }
    };

    auto consume = [&](int buf) {
        if (!XFIXED) {
            // Long rows: this slice's activations, regrouped through the
            // staging area's share of this wave; the reduction buffer shares
            // those bytes, so the workgroup first leaves the previous tile's
            // sum.
            load_x_linear<NT, XP>(xrs, K, nsb, wave + nw * cu_si, lin);
            __syncthreads();
            regroup_x<NT>(xs, lin, raw);
            xexact = prepare_x_slice<NT>(raw, xa, inv, post);
            __syncthreads();
        }
        float part[NT][4];
        if (__builtin_expect(xexact, 1))
            multiply(std::true_type{}, buf, part);
        else
            multiply(std::false_type{}, buf, part);
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[t][r] = fmaf(part[t][r], inv[t][r], acc[t][r]);

        if (XFIXED) {
            // Tile complete for this wave: its partial goes to the group's
            // next slot; the group is summed when full or at the last tile.
            float4_t *mine = reinterpret_cast<float4_t *>(&wave_part(wave)[gslot][lane][0]);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                mine[t] = float4_t{acc[t][0], acc[t][1], acc[t][2], acc[t][3]};
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[t][r] = 0.0f;
            }
            ++gslot;
            ++tiles_done;
            if (gslot == kGroupTiles || tiles_done == ntiles) {
                sum_group(gslot, cu_m0 - (int64_t)(gslot - 1) * kTileRows);
                // The slots are rewritten by the next group only after
                // every thread has read them.
                if (tiles_done < ntiles) __syncthreads();
                gslot = 0;
            }
            cu_m0 += kTileRows;
        } else if (++cu_si == spw) {
            cu_si = 0;
            // Tile complete for this wave: sum the waves' partial tiles.
            float4_t *mine = reinterpret_cast<float4_t *>(&red[rbuf][wave][lane][0]);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                mine[t] = float4_t{acc[t][0], acc[t][1], acc[t][2], acc[t][3]};
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[t][r] = 0.0f;
            }
            __syncthreads();
            if (out_n < N) {
                float sum = 0.0f;
#pragma unroll
                for (int w = 0; w < nw; ++w) sum += red[rbuf][w][out_l][out_v];
                if (cu_m0 + out_mm < M) Y[out_base + cu_m0] = sum;
            }
            rbuf ^= 1;
            cu_m0 += kTileRows;
        }
    };

    for (int u0 = 0; u0 < nunits; u0 += S + 1) {
#pragma unroll
        for (int s = 0; s <= S; ++s) {
            if (u0 + s < nunits) consume(s);
            // Unit u0 + s + S + 1, if there is one: a load past the last unit
            // would read nothing but still cost the address unit (12 / 16 /
            // 32 tokens on 11008 x 2048: 7.45 / 7.59 / 10.23 -> 7.29 / 7.38 /
            // 10.13 us).
            if (u0 + s + S + 1 < nunits) load_unit(s);
        }
    }
}

namespace {

// The kernel for a chunk of N tokens (2 <= N <= 32).  Token pairs loaded:
// the smallest of 1, 2, 4, 8 (one 16-token half) or 12, 16 (two halves)
// that covers N for the NF4 format; the extra formats take 4, 8 or 16.
template <int FMT, bool XF>
const void *smalln_kernel_for(int64_t N) {
    if constexpr (FMT == kGemmNf4) {
        if (N <= 2) return reinterpret_cast<const void *>(&gemm_smalln_kernel<1, XF ? 2 : 0, XF, 1, FMT>);
        if (N <= 4) return reinterpret_cast<const void *>(&gemm_smalln_kernel<1, XF ? 2 : 0, XF, 2, FMT>);
        if (N <= 8) return reinterpret_cast<const void *>(&gemm_smalln_kernel<1, XF ? 2 : 0, XF, 4, FMT>);
        if (N <= 16) return reinterpret_cast<const void *>(&gemm_smalln_kernel<1, XF ? 2 : 0, XF, 8, FMT>);
        if (N <= 24) return reinterpret_cast<const void *>(&gemm_smalln_kernel<2, XF ? 2 : 0, XF, 12, FMT>);
        return reinterpret_cast<const void *>(&gemm_smalln_kernel<2, XF ? 2 : 0, XF, 16, FMT>);
    } else {
        if (N <= 8) return reinterpret_cast<const void *>(&gemm_smalln_kernel<1, XF ? 2 : 0, XF, 4, FMT>);
        if (N <= 16) return reinterpret_cast<const void *>(&gemm_smalln_kernel<1, XF ? 2 : 0, XF, 8, FMT>);
        return reinterpret_cast<const void *>(&gemm_smalln_kernel<2, XF ? 2 : 0, XF, 16, FMT>);
    }
}

static_assert(kSliceBlocks == 4 && kGemmMaxWaves == 8, "split_kranges (q4_internal.h) assumes these");

int device_cus() {
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

// One workgroup of 8 waves per CU (the table and the staging areas take
// 148 KB of LDS).  Chunks of up to 16 tokens take one MFMA per slab of
// weights, larger ones two.  Rows of up to 8 slices (K <= 2048) keep the
// activations in registers; longer rows reload them per tile.
template <int FMT>
hipError_t launch_matrix_core(const uint8_t *codes, const void *scales, const uint16_t *zeros,
                              const float *tscale, int64_t M, int64_t K, const uint16_t *X, int64_t N, float *Y,
                              hipStream_t stream) {
    const int64_t tiles = (M + kTileRows - 1) / kTileRows;
    const int cus = device_cus();
    int64_t grid = tiles < cus ? tiles : cus;
    if (grid < 1) grid = 1;
    int64_t tiles_q = tiles / grid;
    int tiles_rem = (int)(tiles % grid);
    const int nslices = (int)((K / 64 + kSliceBlocks - 1) / kSliceBlocks);
    int k = (int)K, n = (int)N;
    int kranges = 1;
    float *part = nullptr;
    void *args[] = {&codes, &scales, &zeros, &tscale, &M, &k, &X, &n, &Y, &tiles_q, &tiles_rem, &kranges, &part};
    const void *fn = nslices <= kGemmMaxWaves ? smalln_kernel_for<FMT, true>(N) : smalln_kernel_for<FMT, false>(N);
    return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(64 * kGemmMaxWaves), args, 0, stream);
}

// Y[i] = part[0][i] + part[1][i] + ... + part[planes - 1][i], in that order.
__global__ __launch_bounds__(256) void sum_planes_kernel(const float *__restrict__ part, int planes, int64_t n,
                                                         float *__restrict__ Y) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        float s = part[i];
        for (int p = 1; p < planes; ++p) s += part[(int64_t)p * n + i];
        Y[i] = s;
    }
}

// Long rows with scratch memory: K in ranges of at most 8 slices (2048
// weights), so that every workgroup keeps its range's activations in
// registers across all its tiles instead of restaging each slice per tile;
// workgroup b takes range b % R of row range b / R (about CUs / R row
// ranges), writes partial plane b % R of `part`, and a second launch adds
// the R planes into Y.
template <int FMT>
hipError_t launch_matrix_core_split(const uint8_t *codes, const void *scales, const uint16_t *zeros,
                                    const float *tscale, int64_t M, int64_t K, const uint16_t *X, int64_t N,
                                    float *Y, float *part, hipStream_t stream) {
    const int64_t tiles = (M + kTileRows - 1) / kTileRows;
    int kranges = split_kranges(K);
    int64_t groups = device_cus() / kranges;
    if (groups < 1) groups = 1;
    if (groups > tiles) groups = tiles;
    const int64_t grid = groups * kranges;
    int64_t tiles_q = tiles / groups;
    int tiles_rem = (int)(tiles % groups);
    int k = (int)K, n = (int)N;
    void *args[] = {&codes, &scales, &zeros, &tscale, &M, &k, &X, &n, &Y, &tiles_q, &tiles_rem, &kranges, &part};
    hipError_t e = hipLaunchKernel(smalln_kernel_for<FMT, true>(N), dim3((unsigned)grid),
                                   dim3(64 * kGemmMaxWaves), args, 0, stream);
    if (e != hipSuccess) return e;
    const int64_t total = N * M;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 2048) blocks = 2048;
    hipLaunchKernelGGL(sum_planes_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (const float *)part, kranges,
                       total, Y);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_smalln(const uint8_t *codes, const uint16_t *scales, int64_t M, int64_t K,
                              const uint16_t *X, int64_t N, float *Y, hipStream_t stream) {
    // A chunk of one token is the GEMV (measured on the 11008 x 2048 prefill
    // shape: 5.3 us against 7.1 us for the matrix-core kernel, whose set-up
    // and 16-token tiles do not pay for one token).  Two to eight tokens on
    // short rows take one 4-row tile per wave (q4_gemm_rows4.hip); where
    // that kernel's layout conditions fail, two or three tokens share each
    // table lookup in the GEMV kernels.
    if (N == 1) return launch_gemv(codes, scales, M, K, X, Y, stream);
    if (gemm_rows4_fits(scales, nullptr, M, K, N))
        return launch_gemm_rows4(kGemmNf4, codes, scales, nullptr, nullptr, M, K, X, N, Y, stream);
    if (gemv_tokens_fits(M, K, N)) return launch_gemv_tokens(codes, scales, M, K, X, N, Y, stream);
    if (gemv_tokens_multi_fits(M, K, N))
        return launch_gemv_tokens_multi(kGemmNf4, codes, scales, nullptr, nullptr, M, K, X, N, Y, stream);
    return launch_matrix_core<kGemmNf4>(codes, scales, nullptr, nullptr, M, K, X, N, Y, stream);
}

// The library's own scratch for q4_gemm_smalln_noalloc (callers that cannot
// allocate): partial planes of the long-row split, kNoallocScratchBytes on
// each device the library runs on, held until the process ends.  Its name
// is a host-side stand-in: host code uses only the device address that
// hipGetSymbolAddress returns for it (noalloc_scratch below).
static __device__ __align__(256) float scratch[kNoallocScratchBytes / sizeof(float)];

namespace {
// Device address of `scratch` on each device, looked up on the first call
// made with that device current.
constexpr int kMaxDevices = 64;
void *g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mu;

hipError_t noalloc_scratch(float **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = static_cast<float *>(g_scratch_ptr[dev]);
    return hipSuccess;
}
}  // namespace

hipError_t launch_gemm_smalln_noalloc(const uint8_t *codes, const uint16_t *scales, int64_t M, int64_t K,
                                      const uint16_t *X, int64_t N, float *Y, hipStream_t stream) {
    if (!gemm_split_fits(M, K, N)) return launch_gemm_smalln(codes, scales, M, K, X, N, Y, stream);
    if (gemm_split_bytes(M, K, N) > kNoallocScratchBytes) return hipErrorInvalidValue;
    float *part = nullptr;
    const hipError_t e = noalloc_scratch(&part);
    if (e != hipSuccess) return e;
    return launch_matrix_core_split<kGemmNf4>(codes, scales, nullptr, nullptr, M, K, X, N, Y, part, stream);
}

hipError_t launch_gemm_smalln_ws(const uint8_t *codes, const uint16_t *scales, int64_t M, int64_t K,
                                 const uint16_t *X, int64_t N, float *Y, float *part, hipStream_t stream) {
    if (!gemm_split_fits(M, K, N)) return launch_gemm_smalln(codes, scales, M, K, X, N, Y, stream);
    return launch_matrix_core_split<kGemmNf4>(codes, scales, nullptr, nullptr, M, K, X, N, Y, part, stream);
}

hipError_t launch_gemm_smalln_affine_ws(const uint8_t *codes, const uint16_t *scales, const uint16_t *zeros,
                                        int64_t M, int64_t K, const uint16_t *X, int64_t N, float *Y, float *part,
                                        hipStream_t stream) {
    if (!gemm_split_fits(M, K, N)) return launch_gemm_smalln_affine(codes, scales, zeros, M, K, X, N, Y, stream);
    return launch_matrix_core_split<kGemmAffine>(codes, scales, zeros, nullptr, M, K, X, N, Y, part, stream);
}

hipError_t launch_gemm_smalln_nvfp4_ws(const uint8_t *codes, const uint8_t *scales, const float *tscale, int64_t M,
                                       int64_t K, const uint16_t *X, int64_t N, float *Y, float *part,
                                       hipStream_t stream) {
    if (!gemm_split_fits(M, K, N)) return launch_gemm_smalln_nvfp4(codes, scales, tscale, M, K, X, N, Y, stream);
    return launch_matrix_core_split<kGemmNvfp4>(codes, scales, nullptr, tscale, M, K, X, N, Y, part, stream);
}

hipError_t launch_gemm_smalln_affine(const uint8_t *codes, const uint16_t *scales, const uint16_t *zeros, int64_t M,
                                     int64_t K, const uint16_t *X, int64_t N, float *Y, hipStream_t stream) {
    if (N == 1) return launch_gemv_affine(codes, scales, zeros, M, K, X, Y, stream);
    if (gemm_rows4_fits(scales, zeros, M, K, N))
        return launch_gemm_rows4(kGemmAffine, codes, scales, zeros, nullptr, M, K, X, N, Y, stream);
    if (gemv_tokens_multi_fits(M, K, N))
        return launch_gemv_tokens_multi(kGemmAffine, codes, scales, zeros, nullptr, M, K, X, N, Y, stream);
    return launch_matrix_core<kGemmAffine>(codes, scales, zeros, nullptr, M, K, X, N, Y, stream);
}

hipError_t launch_gemm_smalln_nvfp4(const uint8_t *codes, const uint8_t *scales, const float *tscale, int64_t M,
                                    int64_t K, const uint16_t *X, int64_t N, float *Y, hipStream_t stream) {
    if (N == 1) return launch_gemv_nvfp4(codes, scales, tscale, M, K, X, Y, stream);
    if (gemm_rows4_fits(scales, nullptr, M, K, N))
        return launch_gemm_rows4(kGemmNvfp4, codes, scales, nullptr, tscale, M, K, X, N, Y, stream);
    if (gemv_tokens_multi_fits(M, K, N))
        return launch_gemv_tokens_multi(kGemmNvfp4, codes, scales, nullptr, tscale, M, K, X, N, Y, stream);
    return launch_matrix_core<kGemmNvfp4>(codes, scales, nullptr, tscale, M, K, X, N, Y, stream);
}

}  // namespace q4
