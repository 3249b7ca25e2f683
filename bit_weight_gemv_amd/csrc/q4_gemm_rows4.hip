// q4_gemm_rows4.hip -- the prefill product Y[n][m] = sum_k What[m,k] * X[n][k]
// for chunks of 2..8 tokens on rows of at most 2048 weights, one 4-row tile
// per wave, in the three weight formats.
//
// What is computed: the same product as q4_gemm_smalln (the prefill form of
// the deep-fold "Decode V2" page, section 0; accel/tensor func Int4MatMul's
// reconstruction What = level[code] * s per 64-block), for the smallest
// chunks; likewise q4_gemm_smalln_affine ((code - z) * s per 64-block:
// the table holds code - 8, from which z - 8 is subtracted in fp16, exact for
// the packer's integer zero points) and q4_gemm_smalln_nvfp4 (E2M1 level
// times an E4M3 scale per 16 weights, times the tensor scale: the two
// 16-blocks of a 32-weight chunk accumulate apart and take their own scales).
//
// gfx950 design:
//  * Tiles.  A chunk of a few tokens has as few rows per CU as the GEMV
//    (11008 rows: 43 a CU), too few for 16-row matrix-core tiles to keep a
//    CU's waves busy without splitting K between waves.  The 16-block
//    v_mfma_f32_4x4x4_16b_f16 works on 4 x 4 blocks instead: block q (lanes
//    4q .. 4q+3) multiplies 4 tokens by the 4 weight rows of the tile over
//    4 k of its own, lane 4q + i supplying token i's activations (operand A)
//    and row i's weights (operand B), and lane 4q + j receiving the 4
//    tokens' sums of row j.  So each wave takes one tile of 4 rows and all
//    of K, as the GEMV does, and the 16 blocks' sums are added across lanes
//    at the end.  Chunks of 5..8 tokens take two groups of 4 tokens: two
//    MFMAs per step on the same dequantised weights.
//  * Loads.  Load p of a tile gives lane l row l % 4, bytes 16 (16p + l / 4)
//    of the row: 16 lanes read 256 contiguous bytes of each of the 4 rows
//    (measured at the speed of the GEMV's row-by-row order on 11008 x 2048).
//    Lane group q therefore holds chunks 16p + q (32 k each) of all 4 rows.
//  * Scales.  One dword per lane (two block scales of one row), handed to the
//    lanes that need them by lane shuffles: a lane needs, per load p, the
//    scale of its row for the block of chunk 16p + l / 4.  The scale
//    multiplies the chunk's 4 x 4 fp32 sums (one per load p and lane).
//  * Activations.  The workgroup converts the chunk's tokens once into an
//    fp16 copy in LDS: one wave per (token, 512-k range), that range scaled
//    by the power of two that puts its largest bf16 magnitude in
//    [2^14, 2^15); the inverse joins the block scale of the chunks of that
//    range.  A wave issues loads only for the pairs it converts: a load
//    through a range that reads nothing still costs the CU's address unit
//    as much as one that reads (on 11008 x 2048, issuing every wave the
//    same number of loads, most reading nothing, took 5.8-6.0 us against
//    5.1-5.3 us for 2..4 tokens).  The conversion is integer arithmetic on
//    the bf16 bits (exponent rebased, mantissa widened), exact while every
//    nonzero value of a range lies at most 2^28 below its largest (fp16
//    normal numbers; tested per lane, decided per wave).  All waves convert
//    at once before the barrier, so the conversion's instruction count is on
//    the critical path: against an fp32 multiply and round per value it took
//    2 / 4 / 8 tokens from 5.1 / 5.3 / 7.2 to 4.9 / 5.1 / 6.7 us.  If any
//    range of the chunk fails the test the
//    whole workgroup takes the exact loop instead: raw bf16 activations read
//    per lane and widened to fp32, the fp16 levels widened likewise, and
//    v_mfma_f32_4x4x1_16b_f32 (products exact, sums fp32).
//  * Dequantisation.  The LDS byte -> fp16-pair table shared with the GEMV
//    (64 bank-private copies; one ds_read_b32 per two weights).
//  * Measured (11008 x 2048, A/B in one process against the kernels it
//    replaces): 2 tokens 4.9 us (shared-lookup GEMV 6.3), 4 tokens 5.1
//    (16-row matrix-core kernel 7.2), 6 tokens 6.4, 8 tokens 6.7 (7.5); the
//    GEMV takes 4.9 us for one.  Affine format 2 / 4 / 8 tokens 5.3 / 5.5 /
//    7.1 us (matrix-core kernel 7.7 / 7.8 / 7.9), NVFP4-style 5.1 / 5.2 /
//    7.1 (7.5 / 7.6 / 7.8).  A third and fourth token group
//    (9..16 tokens) measured slower than the 16-row kernel (10.7 against
//    7.8 us at 16): every wave reads all of the chunk's activations from
//    LDS and runs 8 MFMAs per 32 k and group, and the conversion grows with
//    the chunk.
#include "q4_device.h"
#include "q4_internal.h"
#include "q4_lut.h"

namespace q4 {

namespace {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));

constexpr int kR4MaxK = 2048;
constexpr int kR4Ranges = kR4MaxK / 512;  // 512-k ranges: one activation scale per token and range
// Bytes per token of the fp16 copy: 16 bytes of padding put the four tokens
// of a lane group's reads in different banks.
constexpr int kR4Pitch = 2 * kR4MaxK + 16;
constexpr int kR4MaxWaves = 12;
constexpr int kR4MaxTokens = 8;

// Pairs a wave converts at most: the launch gives NTG token groups at least
// 4 NTG waves (at most 12).
constexpr int rows4_min_waves(int ntg) { return 4 * ntg < kR4MaxWaves ? 4 * ntg : kR4MaxWaves; }
constexpr int rows4_pairs_per_wave(int ntg) {
    return (16 * ntg + rows4_min_waves(ntg) - 1) / rows4_min_waves(ntg);
}

// A byte of the exponent table meaning "this range is not held exactly".
constexpr int kR4Inexact = -128;

// Lane l of the reduction receives from lane l - 2^L of its row of 16.
template <int L>
__device__ __forceinline__ float ror_lanes(float v) {
    return dpp_f<dpp_row_ror(1 << L)>(v);
}

}  // namespace

// NTG groups of 4 tokens (chunks of up to 4 NTG tokens), NTG = 1 or 2;
// FMT: the NF4 codebook, the affine format (zeros: its zero points) or the
// NVFP4-style format (scales: E4M3 bytes, tscale: the tensor scale).
template <int NTG, int FMT>
__global__ __attribute__((amdgpu_flat_work_group_size(64, 64 * kR4MaxWaves))) void gemm_rows4_kernel(
    const uint8_t *__restrict__ codes, const void *__restrict__ scales, const uint16_t *__restrict__ zeros,
    const float *__restrict__ tscale, int64_t M, int K, const uint16_t *__restrict__ X, int N,
    float *__restrict__ Y) {
    constexpr int NTOK = 4 * NTG;             // tokens the kernel holds
    constexpr int kPairs = NTOK * kR4Ranges;  // (token, range) pairs at most
    constexpr int kPPW = rows4_pairs_per_wave(NTG);
    // The activation copy first: its reads' constant offsets (token group,
    // load p, 16-byte step) then fit the DS instructions' 16-bit offset field
    // instead of costing an address add each; the table's lookups take its
    // base in that field instead.
    struct Smem {
        uint4 xh[NTOK * kR4Pitch / 16];
        uint32_t meta[kPairs / 4];
        uint32_t lut[kLutDwords];
    };
    __shared__ Smem sm;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nw = blockDim.x >> 6;
    const int64_t tile = (int64_t)blockIdx.x * nw + wave;
    const int64_t tiles = (M + 3) >> 2;
    const int row_bytes = K >> 1;
    const int nsb = K >> 6;       // 64-blocks (scales) a row
    const int nch = K >> 5;       // 32-weight chunks a row
    const int row = lane & 3;     // weight row (operand B) and token within a group (operand A) of this lane
    const int grp = lane >> 2;    // lane group: chunk 16p + grp of load p

    // Activations of the wave's (token, range) pairs: pair P = 4 t + r is
    // token t, k = 512 r + 8 lane .. +7 for this lane, for P = wave + nw i
    // below 4 N.  k past K reads zeros (an offset past the buffer).  The
    // rows of tokens N .. 4 NTG - 1 of the last group are never written:
    // they only reach the sums of those tokens, which are not stored.
    const __amdgpu_buffer_rsrc_t xrs = buffer_rsrc(X, (uint32_t)N * (uint32_t)K * 2u);
    const int npairs = 4 * N;
    u32x4_t xraw[kPPW];
#pragma unroll
    for (int i = 0; i < kPPW; ++i) {
        const int P = wave + nw * i;
        const int t = P >> 2, k0 = 512 * (P & 3) + 8 * lane;
        // (A wave with fewer pairs issues fewer loads: every load costs the
        // CU's address unit time, whether or not it reads memory.)
        if (P < npairs)
            xraw[i] = __builtin_amdgcn_raw_buffer_load_b128(xrs, k0 < K ? (t * K + k0) * 2 : 0x7FFFFFF0, 0, 0);
        else
            xraw[i] = u32x4_t{0u, 0u, 0u, 0u};
    }

    // The tile's scales, then its codes (rows past M and chunks past the
    // row's end read zeros).  Scales: lane L reads dword L % 16 of row L / 16
    // (the scales of blocks 2 (L % 16) and 2 (L % 16) + 1); issued first, so
    // that waiting for them does not wait for the codes.
    const bool live = tile < tiles;
    const int64_t row0 = uniform64(live ? tile * 4 : 0);
    const int rows = live ? (int)(M - row0 < 4 ? M - row0 : 4) : 0;
    // (NVFP4: a row's E4M3 scales are K / 16 bytes; lane L reads bytes
    // 8 (L % 16) .. +7 of row L / 16, the scales of chunks 4 (L % 16) .. +3.
    // Affine: the zero points like the scales.)
    const int sdw = lane & 15;
    uint32_t sdword = 0, zdword = 0;
    u32x2_t sq = {0u, 0u};
    if constexpr (FMT == kGemmNvfp4) {
        const int sst = K >> 4;
        const __amdgpu_buffer_rsrc_t srs =
            buffer_rsrc(static_cast<const uint8_t *>(scales) + row0 * sst, (uint32_t)(rows * sst));
        sq = __builtin_amdgcn_raw_buffer_load_b64(srs, 8 * sdw < sst ? (lane >> 4) * sst + 8 * sdw : 0x7FFFFFF0, 0,
                                                  kLoadNonTemporal);
    } else {
        const int soff = 2 * sdw < nsb ? (lane >> 4) * nsb * 2 + 4 * sdw : 0x7FFFFFF0;
        sdword = __builtin_amdgcn_raw_buffer_load_b32(
            buffer_rsrc(static_cast<const uint16_t *>(scales) + row0 * nsb, (uint32_t)(rows * nsb * 2)), soff, 0,
            kLoadNonTemporal);
        if constexpr (FMT == kGemmAffine)
            zdword = __builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(zeros + row0 * nsb, (uint32_t)(rows * nsb * 2)),
                                                          soff, 0, kLoadNonTemporal);
    }
    const __amdgpu_buffer_rsrc_t crs = buffer_rsrc(codes + row0 * row_bytes, (uint32_t)(rows * row_bytes));
    u32x4_t q[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int c = 16 * p + grp;
        q[p] = __builtin_amdgcn_raw_buffer_load_b128(crs, c < nch ? row * row_bytes + 16 * c : 0x7FFFFFF0, 0,
                                                     kLoadNonTemporal);
    }

    if constexpr (FMT == kGemmAffine)
        fill_lut_from(sm.lut, kAffinePairTable);
    else if constexpr (FMT == kGemmNvfp4)
        fill_lut_from(sm.lut, kE2m1PairTable);
    else
        fill_lut(sm.lut);

    // Convert the wave's pairs: the range's largest magnitude (over the
    // wave), of biased exponent Emax, fixes its power of two 2^e with
    // e = 141 - Emax, which puts that magnitude in [2^14, 2^15).  A bf16
    // value of exponent E then has the fp16 exponent E - Emax + 29, so the
    // conversion is integer arithmetic on the bits: subtract (Emax - 29) << 7
    // from the magnitude (saturating: zero stays zero), shift left by 3 (7 to
    // 10 mantissa bits), put the sign back -- three operations per two
    // values.  It is exact when every nonzero value of the range gives a
    // normal fp16 number, i.e. has E >= Emax - 28 (each lane tests its own
    // smallest nonzero magnitude; one ballot decides), and Emax is in
    // 29 .. 254 (a range of zeros counts as exact); otherwise the range is
    // marked inexact.
#pragma unroll
    for (int i = 0; i < kPPW; ++i) {
        const int P = wave + nw * i;
        if (P >= npairs) break;
        const u32x4_t v = xraw[i];
        u16x2_t mag[4];
        u16x2_t mx = {0, 0}, mn = {0xFFFF, 0xFFFF};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            mag[c] = __builtin_bit_cast(u16x2_t, v[c] & 0x7FFF7FFFu);
            mx = __builtin_elementwise_max(mx, mag[c]);
            mn = __builtin_elementwise_min(mn, mag[c] - u16x2_t{1, 1});
        }
        // (A range of zeros -- past K, or zero activations -- is held
        // exactly by any scale: Emax 29 stands in.)
        const int amax = (int)wave_max_u32(mx.x > mx.y ? mx.x : mx.y);
        const int Emax = amax == 0 ? 29 : amax >> 7;
        const uint32_t lo = mn.x < mn.y ? mn.x : mn.y;  // smallest nonzero magnitude - 1, or 0xFFFF
        const bool in_range = Emax >= 29 && Emax <= 254;
        const int eb = in_range ? Emax - 29 : 0;
        const bool ok = lo == 0xFFFFu || lo + 1u >= ((uint32_t)(eb + 1) << 7);
        const bool exact = in_range && __builtin_amdgcn_ballot_w64(!ok) == 0;
        const u16x2_t sub = {(unsigned short)(eb << 7), (unsigned short)(eb << 7)};
        uint32_t h[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const u16x2_t f = __builtin_elementwise_sub_sat(mag[c], sub) << u16x2_t{3, 3};
            h[c] = (v[c] & 0x80008000u) | __builtin_bit_cast(uint32_t, f);
        }
        const int t = P >> 2, r = P & 3;
        sm.xh[(t * kR4Pitch + (512 * r + 8 * lane) * 2) / 16] = make_uint4(h[0], h[1], h[2], h[3]);
        if (lane == 0) reinterpret_cast<int8_t *>(sm.meta)[P] = (int8_t)(exact ? 141 - Emax : kR4Inexact);
    }
    __syncthreads();

    // Per (token, range): the exponent e (its inverse power of two joins the
    // block scale); any inexact range of a token in the chunk sends the
    // workgroup to the exact loop.
    int eb[NTOK];
#pragma unroll
    for (int t = 0; t < NTOK; ++t) eb[t] = __builtin_amdgcn_readfirstlane((int)sm.meta[t]);
    bool all_exact = true;
#pragma unroll
    for (int t = 0; t < NTOK; ++t)
#pragma unroll
        for (int r = 0; r < kR4Ranges; ++r)
            all_exact = all_exact && ((int)(int8_t)(eb[t] >> (8 * r)) != kR4Inexact || t >= N);

    // The scale of this lane's row for the block of chunk 16p + grp: dword
    // (8p + grp / 2) / 2 of the row, held by lane 16 row + 4p + grp / 4
    // (likewise the affine zero point: zz[p] = z - 8 in both halves).
    // NVFP4: the chunk's two E4M3 bytes (its 16-blocks) are bytes
    // 2 (grp % 4), +1 of the 8 that lane 16 row + 4p + grp / 4 holds; sc[p]
    // and sh[p] are the first and the second 16-block's scales.
    float sc[4], sh[4];
    half2_t zz[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int src = 16 * row + 4 * p + (grp >> 2);
        if constexpr (FMT == kGemmNvfp4) {
            const uint32_t d0 = (uint32_t)__shfl((int)sq.x, src), d1 = (uint32_t)__shfl((int)sq.y, src);
            const uint32_t b = ((grp & 2) ? d1 : d0) >> (16 * (grp & 1));
            sc[p] = e4m3_to_f32(b & 0xFFu);
            sh[p] = e4m3_to_f32((b >> 8) & 0xFFu);
        } else {
            const uint32_t d = (uint32_t)__shfl((int)sdword, src);
            sc[p] = f16_bits_to_f32((d >> (16 * ((grp >> 1) & 1))) & 0xFFFFu);
            if constexpr (FMT == kGemmAffine) {
                const uint32_t z = (uint32_t)__shfl((int)zdword, src);
                const _Float16 z8 = (_Float16)(f16_bits_to_f32((z >> (16 * ((grp >> 1) & 1))) & 0xFFFFu) - 8.0f);
                zz[p] = half2_t{z8, z8};
            }
        }
    }

    const uint32_t laneoff = (uint32_t)lane << 2;
    // acc[4 g + t]: token 4 g + t of row `row`, summed over this lane group's
    // chunks.
    float acc[NTOK];
#pragma unroll
    for (int t = 0; t < NTOK; ++t) acc[t] = 0.0f;
    if (__builtin_expect(all_exact, 1)) {
        // This lane's activation base (token `row` of group 0, chunk grp);
        // groups, loads p and the 16-byte steps are constant offsets from it
        // (the DS offset field holds them, so no address arithmetic per read).
        const uint4 *xbase = sm.xh + (row * kR4Pitch + 64 * grp) / 16;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const u32x4_t w = q[p];
            half4_t wb[8];  // this lane's 32 weights of chunk 16p + grp, 4 a step
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                half2_t p0 = lut_pair<0>(sm.lut, w[d], laneoff);
                half2_t p1 = lut_pair<1>(sm.lut, w[d], laneoff);
                half2_t p2 = lut_pair<2>(sm.lut, w[d], laneoff);
                half2_t p3 = lut_pair<3>(sm.lut, w[d], laneoff);
                if constexpr (FMT == kGemmAffine) {
                    // code - 8 minus z - 8: exact small integers in fp16
                    p0 -= zz[p]; p1 -= zz[p]; p2 -= zz[p]; p3 -= zz[p];
                }
                wb[2 * d] = half4_t{p0.x, p0.y, p1.x, p1.y};
                wb[2 * d + 1] = half4_t{p2.x, p2.y, p3.x, p3.y};
            }
#pragma unroll
            for (int g = 0; g < NTG; ++g) {
                // Token 4g + row's fp16 activations of chunk 16p + grp (64 bytes).
                const uint4 *xp = xbase + (4 * g * kR4Pitch + 1024 * p) / 16;
                // D: k 0..15 of the chunk, Dh: k 16..31 (one accumulator
                // for the formats with one scale per chunk).
                float4_t D = {0.0f, 0.0f, 0.0f, 0.0f}, Dh = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const uint4 xv = xp[d];
                    float4_t &T = (FMT == kGemmNvfp4 && d >= 2) ? Dh : D;
                    T = __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(half4_t, uint2{xv.x, xv.y}), wb[2 * d],
                                                           T, 0, 0, 0);
                    T = __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(half4_t, uint2{xv.z, xv.w}),
                                                           wb[2 * d + 1], T, 0, 0, 0);
                }
                // (D times the block scale first: the product stays finite,
                // and a zero sum stays zero under the largest inverse power
                // of two.)
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int e = (int)(int8_t)(eb[4 * g + t] >> (8 * p));
                    float v = D[t] * sc[p];
                    if constexpr (FMT == kGemmNvfp4) v = fmaf(Dh[t], sh[p], v);
                    acc[4 * g + t] = fmaf(v, exp2i(-e), acc[4 * g + t]);
                }
            }
        }
    } else {
        // Exact loop: raw bf16 activations of token 4g + row (zeros past N
        // and past K), one k per MFMA.
#pragma unroll 1
        for (int p = 0; p < 4; ++p) {
            const int c = 16 * p + grp;
            const u32x4_t w = q[p];
            half2_t pr[16];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                pr[4 * d] = lut_pair<0>(sm.lut, w[d], laneoff);
                pr[4 * d + 1] = lut_pair<1>(sm.lut, w[d], laneoff);
                pr[4 * d + 2] = lut_pair<2>(sm.lut, w[d], laneoff);
                pr[4 * d + 3] = lut_pair<3>(sm.lut, w[d], laneoff);
                if constexpr (FMT == kGemmAffine)
#pragma unroll
                    for (int b = 0; b < 4; ++b) pr[4 * d + b] -= zz[p];
            }
#pragma unroll 1
            for (int g = 0; g < NTG; ++g) {
                const int t = 4 * g + row;
                const bool ok = t < N && c < nch;
                u32x4_t xr[4];
#pragma unroll
                for (int d = 0; d < 4; ++d)
                    xr[d] = __builtin_amdgcn_raw_buffer_load_b128(
                        xrs, ok ? (t * K + 32 * c) * 2 + 16 * d : 0x7FFFFFF0, 0, 0);
                float4_t D = {0.0f, 0.0f, 0.0f, 0.0f}, Dh = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int d = 0; d < 4; ++d)
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        // k = 8d + 2b and 8d + 2b + 1 of the chunk
                        uint32_t xw = xr[d][b];
                        __asm__ volatile("" : "+v"(xw));
                        float4_t &T = (FMT == kGemmNvfp4 && d >= 2) ? Dh : D;
                        T = __builtin_amdgcn_mfma_f32_4x4x1f32(__builtin_bit_cast(float, xw << 16),
                                                               (float)pr[4 * d + b].x, T, 0, 0, 0);
                        T = __builtin_amdgcn_mfma_f32_4x4x1f32(__builtin_bit_cast(float, xw & 0xFFFF0000u),
                                                               (float)pr[4 * d + b].y, T, 0, 0, 0);
                    }
                // (acc is indexed at run time here; the loop over groups is
                // kept rolled to hold the exact loop's registers down.)
#pragma unroll
                for (int gg = 0; gg < NTG; ++gg)
                    if (gg == g)
#pragma unroll
                        for (int tt = 0; tt < 4; ++tt) {
                            float a = fmaf(D[tt], sc[p], acc[4 * gg + tt]);
                            if constexpr (FMT == kGemmNvfp4) a = fmaf(Dh[tt], sh[p], a);
                            acc[4 * gg + tt] = a;
                        }
            }
        }
    }

    // Sum the 16 lane groups.  Pairing levels over lane bits 2 and 3 (DPP
    // row rotations by 4 and 8) leave each lane one token of each group,
    // (l / 4) % 4, summed over its row of 16 for weight row l % 4; levels
    // over bit 4 (lanes l ^ 16) then picks the group (two groups) or adds
    // the other rows (one group), and lanes l ^ 32 are added.  Lane l ends
    // with token 4 (l / 16 % NTG) + (l / 4) % 4 of row l % 4.
    const bool b2 = (lane >> 2) & 1, b3 = (lane >> 3) & 1, b4 = (lane >> 4) & 1;
    float u[2 * NTG];
#pragma unroll
    for (int j = 0; j < 2 * NTG; ++j) {
        const float e = acc[2 * j] + ror_lanes<2>(acc[2 * j]), o = acc[2 * j + 1] + ror_lanes<2>(acc[2 * j + 1]);
        u[j] = b2 ? o : e;
    }
    float v[NTG];
#pragma unroll
    for (int j = 0; j < NTG; ++j) {
        const float e = u[2 * j] + ror_lanes<3>(u[2 * j]), o = u[2 * j + 1] + ror_lanes<3>(u[2 * j + 1]);
        v[j] = b3 ? o : e;
    }
    // (Every lane runs every cross-lane step; only the selection after it
    // depends on the lane.)
    float tot;
    if constexpr (NTG == 1) {
        tot = add_xor32(add_xor16(v[0]));
    } else {
        const float s0 = add_xor16(v[0]), s1 = add_xor16(v[1]);
        tot = add_xor32(b4 ? s1 : s0);
    }
    const int tok = 4 * ((lane >> 4) & (NTG - 1)) + ((lane >> 2) & 3);
    const int64_t m = row0 + row;
    if constexpr (FMT == kGemmNvfp4) tot *= *tscale;
    if (live && lane < 16 * NTG && tok < N && m < M) Y[(int64_t)tok * M + m] = tot;
}

namespace {

int rows4_cus() {
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

template <int FMT>
const void *rows4_kernel_for(int64_t N) {
    return N <= 4 ? reinterpret_cast<const void *>(&gemm_rows4_kernel<1, FMT>)
                  : reinterpret_cast<const void *>(&gemm_rows4_kernel<2, FMT>);
}

}  // namespace

bool gemm_rows4_fits(const void *scales, const uint16_t *zeros, int64_t M, int64_t K, int64_t N) {
    return N >= 2 && N <= kR4MaxTokens && K <= kR4MaxK && K % 128 == 0 &&
           (reinterpret_cast<uintptr_t>(scales) & 3) == 0 && (reinterpret_cast<uintptr_t>(zeros) & 3) == 0 &&
           (M + 3) / 4 <= (int64_t)kR4MaxWaves * rows4_cus();
}

// One tile per wave, G waves a workgroup (one workgroup per CU: the table
// and the activation copy take 81 KB of LDS), at least 4 so that the table
// fill is shared.
hipError_t launch_gemm_rows4(int fmt, const uint8_t *codes, const void *scales, const uint16_t *zeros,
                             const float *tscale, int64_t M, int64_t K, const uint16_t *X, int64_t N, float *Y,
                             hipStream_t stream) {
    if (!gemm_rows4_fits(scales, zeros, M, K, N) || (fmt == kGemmAffine) != (zeros != nullptr) ||
        (fmt == kGemmNvfp4) != (tscale != nullptr))
        return hipErrorInvalidValue;
    const int64_t tiles = (M + 3) / 4;
    const int64_t cus = rows4_cus();
    int64_t G = (tiles + cus - 1) / cus;
    const int ntg = N <= 4 ? 1 : 2;
    if (G < rows4_min_waves(ntg)) G = rows4_min_waves(ntg);
    if (G > kR4MaxWaves) G = kR4MaxWaves;
    const int64_t grid = (tiles + G - 1) / G;
    int k = (int)K, n = (int)N;
    void *args[] = {&codes, &scales, &zeros, &tscale, &M, &k, &X, &n, &Y};
    const void *fn = fmt == kGemmAffine ? rows4_kernel_for<kGemmAffine>(N)
                     : fmt == kGemmNvfp4 ? rows4_kernel_for<kGemmNvfp4>(N)
                                         : rows4_kernel_for<kGemmNf4>(N);
    return hipLaunchKernel(fn, dim3((unsigned)grid),
                           dim3((unsigned)(64 * G)), args, 0, stream);
}

}  // namespace q4
