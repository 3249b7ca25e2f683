/*
 * q4.h -- C ABI of libq4: 4-bit, 16-level NF4-style codebook weight-only
 * GEMV and small-N GEMM for AMD Instinct MI355X (gfx950).
 *
 * What is computed (deep-fold "Decode V2 - resident executor" page):
 *   - section 6 "Linear primitive": a weight's value is the entry of a
 *     16-float table picked by its 4-bit code, times the scale of its group,
 *     and the GEMV accumulates table x scale x activation in fp32;
 *   - section 2 "Synthetic models": groups are 64 weights along K;
 *   - section 0 "Goals": the prefill form runs chunks of up to 32 tokens
 *     (LIVE_MAX_N) through one dedicated product that reads the weights once
 *     per chunk.
 * Number formats (golang.design accel/tensor page): f32 -> f16 rounds to
 * nearest even and an out-of-range value becomes an infinity (func Cast);
 * bf16 -> f32 is exact (func Cast); products accumulate in f32 and return f32
 * (func MatMul); 4-bit codes are packed low nibble first (type Int4).
 *
 * Packed format (identical on host and device, "canonical"):
 *   codes  : uint8 [M][K/2], row-major; byte j of row m holds the code of
 *            k = 2j in bits 0..3 and of k = 2j+1 in bits 4..7.
 *   scales : IEEE binary16 bit patterns, uint16 [M][K/64], row-major; the
 *            scale of block b of row m is the fp16 round-to-nearest-even of
 *            max |W[m, 64b .. 64b+63]|.
 *   value  : What[m,k] = level[code(m,k)] * scale[m][k/64], where level is the
 *            frozen table returned by q4_codebook() (level[7] == 0 exactly).
 *
 * Conventions for every entry point:
 *   - Data pointers are DEVICE pointers owned by the caller.  The library
 *     allocates nothing and keeps no state between calls.
 *   - All argument checks run on the host before anything is launched; a
 *     call that returns an error has launched nothing and written nothing.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the legacy default
 *     stream) and the call returns without waiting.  Calls are reentrant.
 *   - The device current at call time must be a gfx950 GPU and must own the
 *     pointers.
 *   - M = 0 (or N = 0) is a valid no-op returning Q4_OK.
 */
#ifndef Q4_H
#define Q4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
typedef enum {
    Q4_OK = 0,
    Q4_ERR_NULL = 1,      /* a required pointer is NULL                       */
    Q4_ERR_SHAPE = 2,     /* M < 0, K <= 0, K % 64 != 0, K > Q4_MAX_K, N < 0,
                             N > Q4_MAX_N                                      */
    Q4_ERR_ALIGN = 3,     /* a pointer breaks the alignment stated below      */
    Q4_ERR_OVERLAP = 4,   /* an output range overlaps an input or another
                             output range                                     */
    Q4_ERR_DEVICE = 5,    /* the HIP runtime refused the launch (no gfx950
                             device current, bad stream, ...)                  */
    Q4_ERR_WORKSPACE = 6  /* scratch memory for partial sums is missing or
                             smaller than the call needs                       */
} q4_status;

/* Largest K the kernels accept (a multiple of 64). */
#define Q4_MAX_K 131072
/* Largest token count of q4_gemm_smalln (LIVE_MAX_N of the deep-fold page). */
#define Q4_MAX_N 32

/* Flags OR-ed into q4_pack's device status word. */
#define Q4_PACK_NONFINITE 1 /* some weight is NaN or infinite                  */
#define Q4_PACK_OVERFLOW 2  /* some block's absmax rounds to fp16 infinity
                               (|w| >= 65520)                                   */

/* Bytes of the packed codes / scales of an M x K matrix (0 on bad shape). */
size_t q4_codes_bytes(int64_t M, int64_t K);
size_t q4_scales_bytes(int64_t M, int64_t K);

/* Copy the 16 frozen codebook levels (fp32, ascending, level[0] = -1,
 * level[7] = 0, level[15] = +1) into host memory `out`.  These are the
 * NormalFloat-4 levels (QLoRA construction with an exact zero; the deep-fold
 * page names the format NF4 and its 16-float table without printing it). */
void q4_codebook(float out[16]);

/* Human-readable name of a q4_status value. */
const char *q4_status_string(int status);

/*
 * q4_pack -- quantise W (fp32, [M][K] row-major) into the packed format.
 *   codes: q4_codes_bytes(M,K) bytes, 16-byte aligned.
 *   scales: q4_scales_bytes(M,K) bytes, 2-byte aligned.
 *   W: 16-byte aligned.
 *   status: one int32 in device memory, 4-byte aligned.  It is cleared and
 *     then receives the OR of Q4_PACK_* flags over all blocks.  A flagged
 *     block's codes and scale are left unwritten; the rest are valid.
 * Codes (reading of the unprinted step): the level nearest to w / scale in
 * exact arithmetic, an exact midpoint taking the lower level; a block whose
 * scale is 0 gets code 7 throughout.  The result is bit-exact: one answer.
 * Ranges of W, codes, scales and status must not overlap.
 */
int q4_pack(const float *W, int64_t M, int64_t K, uint8_t *codes,
            uint16_t *scales, int32_t *status, void *stream);

/*
 * q4_unpack_canonical -- write a packed matrix in the canonical layout
 * described at the top of this file.  The library's device layout is the
 * canonical one, so this is a device-to-device copy of both arrays on
 * `stream`; it exists so that bit-exactness of q4_pack can always be judged
 * on the canonical layout.
 *   codes/scales: the packed matrix (codes 16-byte aligned, scales 2-byte).
 *   codes_out: q4_codes_bytes(M,K) bytes, 16-byte aligned.
 *   scales_out: q4_scales_bytes(M,K) bytes, 2-byte aligned.
 * No two of the four ranges may overlap.
 */
int q4_unpack_canonical(const uint8_t *codes, const uint16_t *scales,
                        int64_t M, int64_t K, uint8_t *codes_out,
                        uint16_t *scales_out, void *stream);

/*
 * q4_gemv -- y[m] = sum_k What[m,k] * x[k], m < M (the batch-1 decode
 * projection).
 *   codes/scales: a packed matrix (codes 16-byte aligned, scales 2-byte).
 *   x: bf16 bit patterns [K], 16-byte aligned.
 *   y: fp32 [M], 4-byte aligned; must not overlap codes, scales or x.
 * Accuracy: |y - y_exact| <= 1e-3 * sum_k |What[m,k] x[k]| + 1e-5 for any
 * finite x and any packed matrix, while that sum stays inside fp32's range.
 * The fp16 rounding of the table costs at most 2^-11 relative per term;
 * every activation enters its product exactly (as fp16 under a power of two,
 * or widened to fp32 where the values one wave holds span more than 2^28);
 * sums are fp32.  Non-finite x propagate into y.
 */
int q4_gemv(const uint8_t *codes, const uint16_t *scales, int64_t M, int64_t K,
            const uint16_t *x, float *y, void *stream);

/*
 * q4_gemm_smalln -- Y[n][m] = sum_k What[m,k] * X[n][k], n < N <= 32, m < M
 * (the prefill-chunk form: deep-fold "Decode V2" page, section 0 Goals, a
 * prompt runs as chunks of up to 32 tokens through one product; golang.design
 * accel/tensor, func Int4MatMul: the matrix is read once per tile of tokens.
 * Every weight is read once per call).
 *   X: bf16 bit patterns [N][K] row-major, 16-byte aligned.
 *   Y: fp32 [N][M] row-major, 4-byte aligned; must not overlap the inputs.
 * Same accuracy statement as q4_gemv, for every finite X: every activation
 * enters its products exactly, as fp16 under a power of two per token and
 * range of K (256 weights in the 16-row kernel, 512 in the 4-row kernel),
 * or as fp32 where a range's nonzero values span more than 2^28 (a slower
 * path for such inputs only).  A chunk of one token is computed by the
 * q4_gemv kernels (Y[0] is then bit-identical to q4_gemv of X[0]); chunks of
 * two to eight tokens on rows of at most 2048 weights (K % 128 == 0, a
 * dword-aligned scale plane, at most 12 four-row tiles per compute unit)
 * by one 4-row tile per wave; where those conditions fail, chunks of two
 * or three tokens on such rows by the q4_gemv kernels with each table
 * lookup serving every token; chunks of two or three tokens on rows of
 * 2080 .. 24576 weights (four tokens: 8192 .. 24576) likewise by the
 * q4_gemv kernels for rows spanning several waves (a row of Y is then
 * bit-identical to q4_gemv of its token while no wave holds values of
 * another token of the chunk that span more than 2^28: such a wave takes
 * the exact path for all the chunk's tokens); all others by 16-row
 * matrix-core tiles.
 */
int q4_gemm_smalln(const uint8_t *codes, const uint16_t *scales, int64_t M,
                   int64_t K, const uint16_t *X, int64_t N, float *Y,
                   void *stream);

/*
 * q4_gemm_smalln_ws -- the product of q4_gemm_smalln (the same passages),
 * given device scratch memory for partial sums.  On rows longer than 2048
 * weights, chunks that q4_gemm_smalln runs on 16-row matrix-core tiles
 * (2..32 tokens, except 2..4 tokens where the q4_gemv kernels take them)
 * reload and convert every 256-weight slice of X for each tile there.  Here
 * K is split instead into q4_gemm_smalln_ws_bytes / (4 N M) ranges of at
 * most 2048 weights: each workgroup keeps its range's activations in
 * registers across all of its tiles and writes its sums into that range's
 * partial plane, and a second launch adds the planes in range order (every
 * call gives the same bits).  Elsewhere the call is q4_gemm_smalln and the
 * workspace is not touched (it may then be NULL).
 *   workspace: device memory of at least q4_gemm_smalln_ws_bytes(M, K, N)
 *     bytes, 16-byte aligned, owned by the caller; nothing in it needs to
 *     start at any value, and it holds nothing once the call's work ends.
 *     Calls that may run at the same time need different workspaces.
 *   workspace_bytes: its size.
 * Accuracy: as q4_gemm_smalln (the sums of each range are fp32, then fp32
 * adds across ranges).
 * Errors: as q4_gemm_smalln; Q4_ERR_WORKSPACE if scratch is needed and the
 * workspace is NULL or smaller than asked; Q4_ERR_ALIGN for a misaligned
 * workspace; Q4_ERR_OVERLAP if it overlaps an input or Y.
 */
size_t q4_gemm_smalln_ws_bytes(int64_t M, int64_t K, int64_t N);
int q4_gemm_smalln_ws(const uint8_t *codes, const uint16_t *scales, int64_t M,
                      int64_t K, const uint16_t *X, int64_t N, float *Y,
                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * q4_gemm_smalln_noalloc -- q4_gemm_smalln_ws for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the partial planes go to a
 * scratch array of Q4_NOALLOC_SCRATCH_BYTES that the library holds on each
 * device it runs on from its first use until the process ends.  The call
 * allocates nothing.  Every call on one device shares that device's array
 * (which keeps the last call's contents; no call depends on them), so calls
 * that may overlap in time on one device race and must be ordered by the
 * caller (one stream, or events).
 * Errors: as q4_gemm_smalln; Q4_ERR_WORKSPACE (nothing launched) where
 * q4_gemm_smalln_ws_bytes(M, K, N) exceeds Q4_NOALLOC_SCRATCH_BYTES;
 * Q4_ERR_DEVICE if the array's device address cannot be found.
 */
#define Q4_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int q4_gemm_smalln_noalloc(const uint8_t *codes, const uint16_t *scales,
                           int64_t M, int64_t K, const uint16_t *X, int64_t N,
                           float *Y, void *stream);

/*
 * Fused decode projections (deep-fold "Decode V2" page, section 6 Linear primitive: one
 * grid over the q, k and v rows sharing x with the q/k/v bias added in that
 * kernel; gate/up pairs writing silu(g) * u, SiLU only after the full
 * reduction; the o/down residual added into y; golang.design accel/tensor:
 * func Linear adds its bias in the product's kernel, func SwiGLU is
 * SiLU(gate) * value).
 */
#define Q4_MAX_FUSED 4           /* matrices per q4_gemv_fused call          */
#define Q4_MAX_FUSED_K 16384     /* longest rows q4_gemv_fused accepts       */
#define Q4_FUSE_SEPARATE 0       /* one output per matrix                    */
#define Q4_FUSE_SWIGLU 1         /* two matrices (gate, up) -> one output    */

/* One packed matrix of a fused call. */
typedef struct {
    const uint8_t *codes;    /* packed codes [M][K/2], 16-byte aligned        */
    const uint16_t *scales;  /* fp16 bits [M][K/64], 2-byte aligned           */
    int64_t M;               /* rows (M >= 0)                                 */
    const float *bias;       /* fp32 [M], 4-byte aligned, or NULL             */
} q4_operand;

/*
 * q4_gemv_fused -- several products of one activation vector in one launch.
 *   ops[0..count-1]: the matrices, all with K columns (K <= Q4_MAX_FUSED_K);
 *     t_i = W_i . x + bias_i (fp32 accumulation, bias added to the sum).
 *   mode Q4_FUSE_SEPARATE (1 <= count <= Q4_MAX_FUSED):
 *     y[i][m] = t_i[m] + residual[i][m],  m < ops[i].M.
 *   mode Q4_FUSE_SWIGLU (count == 2, ops[0].M == ops[1].M, gate then up):
 *     y[0][m] = silu(t_0[m]) * t_1[m] + residual[0][m],  silu(z) = z / (1 + e^-z).
 *   x: bf16 bits [K], 16-byte aligned.
 *   y: host array of device pointers (count of them, or 1 for SWIGLU), each
 *     fp32 and 4-byte aligned.
 *   residual: NULL, or a host array like y whose entries are NULL or fp32
 *     device vectors; residual[i] may be exactly y[i] (an in-place add) but
 *     must not otherwise overlap an output.
 * An output must not overlap any input or another output.  Matrices with
 * M == 0 are skipped.  Accuracy: t_i as q4_gemv; the epilogue is fp32.
 * Errors (nothing is launched): Q4_ERR_SHAPE for an unknown mode, a count
 * out of range, SWIGLU with count != 2 or unequal M, K not a positive
 * multiple of 64 or above Q4_MAX_FUSED_K, or M < 0; Q4_ERR_NULL for a missing
 * ops, x, y or y[i], codes or scales of a non-empty matrix; Q4_ERR_ALIGN;
 * Q4_ERR_OVERLAP; Q4_ERR_DEVICE if the launch fails.  With every M == 0 the
 * call returns Q4_OK without looking at x, y or residual.
 */
int q4_gemv_fused(const q4_operand *ops, int count, int64_t K,
                  const uint16_t *x, int mode, float *const *y,
                  const float *const *residual, void *stream);

/*
 * Affine 4-bit format (golang.design accel/tensor page: type Int4 stores
 * 4-bit codes, low nibble first, with an f16 scale and an f16 zero point per
 * group; func Int4MatVec reconstructs What = (code - z) * s, and states the
 * error as at most a group's range over 30).  Here a group is 64 weights
 * along K, and codes are laid out as in the NF4 format above; scales and
 * zeros are fp16 bits [M][K/64] (q4_scales_bytes each).  The page does not
 * print its quantiser; q4_pack_affine does this:
 *   - lo, hi: the block's minimum and maximum, widened to hold 0;
 *   - s = fp16 nearest-even of (hi - lo) / 15 (fp64 arithmetic, one rounding
 *     to fp16);
 *   - z = the integer nearest to -lo / s in 0..15 (a midpoint goes down);
 *   - code = the level (j - z) * s nearest to w (a midpoint goes to the lower
 *     code); with s == 0 every code and z are 0.
 * Each decision is an exact comparison, so the result is bit-exact.
 */

/*
 * q4_pack_affine -- quantise W [M][K] (fp32, 16-byte aligned) into codes,
 * scales and zeros (fp16 bits, 2-byte aligned).  *status as q4_pack
 * (Q4_PACK_NONFINITE, Q4_PACK_OVERFLOW when (hi - lo) / 15 rounds to fp16
 * infinity); a flagged block's output is unspecified.  No two of W, codes,
 * scales, zeros and status may overlap.
 */
int q4_pack_affine(const float *W, int64_t M, int64_t K, uint8_t *codes,
                   uint16_t *scales, uint16_t *zeros, int32_t *status,
                   void *stream);

/*
 * q4_gemv_affine -- y[m] = sum_k (code(m,k) - z[m][k/64]) * s[m][k/64] * x[k],
 * fp32 accumulation; x bf16 bits [K] (16-byte aligned), y fp32 [M]
 * (4-byte aligned, overlapping no input).  Accuracy as q4_gemv: within
 * 1e-3 * sum_k |What x| + 1e-5 of the exact value.  Errors as q4_gemv.
 */
int q4_gemv_affine(const uint8_t *codes, const uint16_t *scales,
                   const uint16_t *zeros, int64_t M, int64_t K,
                   const uint16_t *x, float *y, void *stream);

/*
 * int8 activations for the integer-code (affine) format (deep-fold "Decode
 * V2" page, the lane's knobs: a projection's activation may be one int8
 * word, as llama.cpp does, or two int8 words of about 14 bits, the page's
 * default).  Per block of 32 activations along K:
 *   d  = the f32 rounding of the fp64 quotient max|x| / 127;
 *   q1 = the integer nearest to x / d, ties to even, within +-127;
 *   q2 = (two words) the integer nearest to 128 (x - q1 d) / d, same rule;
 * the value carried is xq = d (q1 + q2 / 128); |x - xq| <= d / 2 (one word)
 * or d / 256 (two words).  Decisions are exact comparisons: bit-exact.
 */

/*
 * q4_quantize_x8 -- x bf16 bits [K] (16-byte aligned) -> q1 int8 [K] and,
 * for words == 2, q2 int8 [K] (16-byte aligned; q2 may be NULL for one
 * word), d fp32 [K/32] (4-byte aligned).  K as the products (a positive
 * multiple of 64).  No two ranges may overlap.
 */
int q4_quantize_x8(const uint16_t *x, int64_t K, int words, int8_t *q1,
                   int8_t *q2, float *d, void *stream);

/*
 * q4_gemv_affine_x8 -- the affine format's GEMV on int8 activations:
 * y[m] = sum_k (code - z) * s * xq[k], with xq from q4_quantize_x8 (q2 NULL:
 * one word).  The dot products are exact integer sums (v_dot4_i32_i8), then
 * one fp32 scaling per 32 weights: within 1e-3 * sum_k |What xq| + 1e-5 of
 * the exact value (the bound restated on xq).  Errors as q4_gemv_affine.
 */
int q4_gemv_affine_x8(const uint8_t *codes, const uint16_t *scales,
                      const uint16_t *zeros, int64_t M, int64_t K,
                      const int8_t *q1, const int8_t *q2, const float *d,
                      float *y, void *stream);

/*
 * NVFP4-style format (gizai tensor/lazy page, fp4Blocks: E2M1 codes, two to a
 * byte with the first in the low half; one E4M3 scale per 16 values along K;
 * an f32 tensor scale s = max|W| / (6 * 448); a weight is its E2M1 value
 * times its block's E4M3 scale times s).  Codes are laid out as the NF4
 * format; scales are E4M3 bytes [M][K/16], row-major (the page interleaves
 * them for NVIDIA tensor-core tiles; a row-per-wave GEMV wants one row's
 * scales contiguous).  The page leaves the rounding steps open;
 * q4_pack_nvfp4 does this:
 *   - s = the f32 rounding of the fp64 quotient max|W| / 2688;
 *   - a block's scale: the E4M3 value nearest to amax_block / (6 s), ties to
 *     the even pattern, at most 448 (s == 0: 0);
 *   - a code: the E2M1 magnitude nearest to |w| / (scale * s), ties to the
 *     even pattern, at most 6, with w's sign bit; a block of scale 0 is all
 *     code 0.
 * Every decision is an exact comparison, so the result is bit-exact.
 */

/*
 * q4_pack_nvfp4 -- quantise W [M][K] (fp32, 16-byte aligned): codes
 * (16-byte aligned), scales (2-byte aligned), the tensor scale (one float,
 * 4-byte aligned) and *status (Q4_PACK_NONFINITE if W holds a NaN or an
 * infinity: the blocks holding one are unspecified, s is taken over the
 * finite values).  Four launches on `stream`.  No two buffers may overlap.
 */
int q4_pack_nvfp4(const float *W, int64_t M, int64_t K, uint8_t *codes,
                  uint8_t *scales, float *tscale, int32_t *status, void *stream);

/*
 * q4_gemv_nvfp4 -- y[m] = s * sum_k E2M1(code(m,k)) * E4M3(scale[m][k/16])
 * * x[k], fp32 accumulation; the tensor scale is read from device memory
 * (tscale) when the kernel runs.  Accuracy and errors as q4_gemv.
 */
int q4_gemv_nvfp4(const uint8_t *codes, const uint8_t *scales,
                  const float *tscale, int64_t M, int64_t K,
                  const uint16_t *x, float *y, void *stream);

/*
 * The fused decode projections of q4_gemv_fused in the two formats above
 * (the epilogues of the deep-fold "Decode V2" page, section 6 Linear
 * primitive, and accel/tensor func Linear / func SwiGLU, on the affine
 * format of accel/tensor type Int4 and the NVFP4-style format of gizai
 * fp4Blocks).  One operand per matrix:
 *   affine: codes, scales and zeros as q4_gemv_affine;
 *   NVFP4-style: codes, E4M3 scales (2-byte aligned) and the device tensor
 *   scale as q4_gemv_nvfp4.  In the SWIGLU mode the gate and the up matrix
 *   keep their own tensor scales, each applied to its finished sum before
 *   SiLU.
 * Modes, x, y, residual, accuracy and errors as q4_gemv_fused; a missing
 * zeros (affine) or tscale (NVFP4-style) of a non-empty matrix is
 * Q4_ERR_NULL, and they count as inputs for Q4_ERR_OVERLAP.
 */
typedef struct {
    const uint8_t *codes;    /* packed codes [M][K/2], 16-byte aligned        */
    const uint16_t *scales;  /* fp16 bits [M][K/64], 2-byte aligned           */
    const uint16_t *zeros;   /* fp16 zero points [M][K/64], 2-byte aligned    */
    int64_t M;               /* rows (M >= 0)                                 */
    const float *bias;       /* fp32 [M], 4-byte aligned, or NULL             */
} q4_operand_affine;

typedef struct {
    const uint8_t *codes;    /* packed E2M1 codes [M][K/2], 16-byte aligned   */
    const uint8_t *scales;   /* E4M3 bytes [M][K/16], 2-byte aligned          */
    const float *tscale;     /* the f32 tensor scale (device), 4-byte aligned */
    int64_t M;               /* rows (M >= 0)                                 */
    const float *bias;       /* fp32 [M], 4-byte aligned, or NULL             */
} q4_operand_nvfp4;

int q4_gemv_fused_affine(const q4_operand_affine *ops, int count, int64_t K,
                         const uint16_t *x, int mode, float *const *y,
                         const float *const *residual, void *stream);
int q4_gemv_fused_nvfp4(const q4_operand_nvfp4 *ops, int count, int64_t K,
                        const uint16_t *x, int mode, float *const *y,
                        const float *const *residual, void *stream);

/*
 * The prefill-chunk forms of the two formats above (as q4_gemm_smalln: the
 * deep-fold "Decode V2" page, section 0 Goals, runs a prompt as chunks of up
 * to 32 tokens through one product; accel/tensor func Int4MatMul reads the
 * matrix once per tile of tokens).  Every weight is read once per call.
 *   X: bf16 bits [N][K] row-major, 16-byte aligned; 0 <= N <= Q4_MAX_N.
 *   Y: fp32 [N][M] row-major, 4-byte aligned; must not overlap the inputs.
 * N == 1 runs the format's GEMV (Y[0] is bit-identical to it); N == 0 is a
 * no-op.  Accuracy as q4_gemv, for every finite X: each token's activations
 * enter exactly (fp16 under a power of two per 256-weight slice, or as fp32
 * where a slice spans more than 2^28).  Errors as q4_gemm_smalln.
 *
 * q4_gemm_smalln_affine -- Y[n][m] = sum_k (code(m,k) - z[m][k/64])
 * * s[m][k/64] * X[n][k]; codes, scales and zeros as q4_gemv_affine.
 * Chunks of two to eight tokens take the 4-row tiles under the conditions
 * of q4_gemm_smalln, the zero-point plane also dword-aligned.
 */
int q4_gemm_smalln_affine(const uint8_t *codes, const uint16_t *scales,
                          const uint16_t *zeros, int64_t M, int64_t K,
                          const uint16_t *X, int64_t N, float *Y,
                          void *stream);

/*
 * q4_gemm_smalln_nvfp4 -- Y[n][m] = s * sum_k E2M1(code(m,k))
 * * E4M3(scale[m][k/16]) * X[n][k]; codes, scales and tscale as
 * q4_gemv_nvfp4, except that scales must be 4-byte aligned (the four scale
 * bytes of a 64-block are read as one dword).  Chunks of two to eight
 * tokens take the 4-row tiles under the conditions of q4_gemm_smalln.
 */
int q4_gemm_smalln_nvfp4(const uint8_t *codes, const uint8_t *scales,
                         const float *tscale, int64_t M, int64_t K,
                         const uint16_t *X, int64_t N, float *Y,
                         void *stream);

/*
 * q4_gemm_smalln_affine_ws, q4_gemm_smalln_nvfp4_ws -- the prefill products
 * of the two extra formats (the same passages as q4_gemm_smalln_affine and
 * q4_gemm_smalln_nvfp4) with scratch for partial sums, as q4_gemm_smalln_ws
 * is for the NF4 codebook format, and on the same chunks: on rows longer
 * than 2048 weights, chunks that the 16-row kernel would take split K into
 * ranges of at most 2048 weights whose partial planes a second launch adds
 * in range order.  Elsewhere the call is the format's q4_gemm_smalln_*
 * entry point (the workspace may then be NULL).
 *   workspace: at least q4_gemm_smalln_ws_bytes(M, K, N) bytes of device
 *     memory, 16-byte aligned, as for q4_gemm_smalln_ws.
 * Errors: as the format's q4_gemm_smalln_* entry point, and those of
 * q4_gemm_smalln_ws for the workspace.
 */
int q4_gemm_smalln_affine_ws(const uint8_t *codes, const uint16_t *scales,
                             const uint16_t *zeros, int64_t M, int64_t K,
                             const uint16_t *X, int64_t N, float *Y,
                             void *workspace, size_t workspace_bytes,
                             void *stream);
int q4_gemm_smalln_nvfp4_ws(const uint8_t *codes, const uint8_t *scales,
                            const float *tscale, int64_t M, int64_t K,
                            const uint16_t *X, int64_t N, float *Y,
                            void *workspace, size_t workspace_bytes,
                            void *stream);

/*
 * Packed row gather (deep-fold "Decode V2" page, run notes of section 6: the
 * embedding is kept as packed rows and the rows a step needs are dequantised
 * into its arena, with no dense vocabulary table; a tied embedding shares
 * the lm_head's packed matrix; golang.design accel/tensor page, func
 * QuantGatherRows: rows gathered from a quantized table).
 */
#define Q4_OUT_F32 0            /* fp32 output rows                           */
#define Q4_OUT_BF16 1           /* bf16 output rows (bit patterns, uint16)    */
#define Q4_GATHER_BAD_ID 1      /* status flag: some id outside [0, M)        */

/*
 * q4_gather_rows -- out[i][k] = What[ids[i], k] for i < n, rounded once to
 * nearest even (ties to even) from the exact What = level * scale into
 * out_type (Q4_OUT_F32 or Q4_OUT_BF16).
 *   codes, scales: the packed M x K matrix (16- and 2-byte aligned).
 *   ids: int32 [n] device array of row indices (4-byte aligned).
 *   out: [n][K] fp32 or bf16, 16-byte aligned.
 *   status: device int32 word, 4-byte aligned; set to 0, or to
 *     Q4_GATHER_BAD_ID if some ids[i] is outside [0, M).  Such an id is a
 *     caller error (accel/tensor func GatherRows): its row is written as
 *     zeros and the table is not read there.  With n == 0 the call only
 *     clears *status.
 * Errors (nothing is launched): Q4_ERR_SHAPE for a bad M, K, n < 0, an
 * unknown out_type or an output larger than the grid can cover;
 * Q4_ERR_NULL for a missing status, or ids / out with n > 0, or codes /
 * scales with n > 0 and M > 0; Q4_ERR_ALIGN; Q4_ERR_OVERLAP if out or status
 * overlaps an input or each other; Q4_ERR_DEVICE if the launch fails.
 */
int q4_gather_rows(const uint8_t *codes, const uint16_t *scales, int64_t M, int64_t K,
                   const int32_t *ids, int64_t n, int out_type, void *out,
                   int32_t *status, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* Q4_H */
