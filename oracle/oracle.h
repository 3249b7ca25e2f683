/*
 * oracle.h -- declarations of the fp64 CPU oracle for the 4-bit, 16-level
 * NF4-style codebook weight-only GEMV and its small-N GEMM form.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the slow, plain reference that the HIP
 * library is checked against.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it.  It shares no code, header,
 * table or constant with the HIP library.
 *
 * Sources (the deep-fold "Decode V2 - resident executor" page unless noted):
 *   - section 6 "Linear primitive": the GEMV dequantises with a 16-float table
 *     times a per-group scale times x, fp32 on the GPU;
 *   - section 2 "Synthetic models": quantisation groups are 64 weights long;
 *   - section 3 "CPU oracle": the NF4 matmul is decode-then-matmul,
 *     Y = What @ x;
 *   - golang.design accel/tensor page, type Int4: nibbles are packed low
 *     nibble first; func Cast: f32 -> f16 rounds to nearest-even and an
 *     out-of-range value becomes infinity; bf16 -> f32 is exact;
 *     func Argmax: ties go to the lowest index.
 */
#ifndef Q4_ORACLE_H
#define Q4_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Pack status flags (OR-ed together over every block). */
#define ORACLE_PACK_NONFINITE 1 /* some weight is NaN or +-inf            */
#define ORACLE_PACK_OVERFLOW  2 /* some block absmax rounds to fp16 +inf  */

/* The 16 levels in fp64 straight from the construction, ascending. */
void oracle_codebook_f64(double out[16]);
/* The same levels rounded once to fp32 (the frozen table). */
void oracle_codebook_f32(float out[16]);
/* Inverse standard normal CDF by bisection on erfc (exposed for pinning). */
double oracle_phi_inv(double p);

/* fp32 -> IEEE binary16 bits, round to nearest, ties to even; |v| >= 65520
 * gives +-inf; NaN gives a quiet NaN. */
uint16_t oracle_f32_to_f16_rne(float v);
/* The same rounding from a double (one rounding of the exact value). */
uint16_t oracle_f64_to_f16_rne(double v);
void oracle_f32_to_f16_rne_array(const float *v, int64_t n, uint16_t *out);
double oracle_f16_to_f64(uint16_t h);
/* bf16 bits -> value (exact widening). */
double oracle_bf16_to_f64(uint16_t b);

/* Quantise rows [row0,row1) of W[M,K] (fp32, row-major; K % 64 == 0).
 * codes: M*K/2 bytes, byte (m,j) = code(m,2j) | code(m,2j+1) << 4.
 * scales: fp16 bits, [M][K/64] row-major.
 * Returns the OR of ORACLE_PACK_* flags over the rows (0 = ok); the output of
 * a flagged block is unspecified. */
int oracle_pack_rows(const float *W, int64_t M, int64_t K, int64_t row0,
                     int64_t row1, uint8_t *codes, uint16_t *scales);
int oracle_pack(const float *W, int64_t M, int64_t K, uint8_t *codes,
                uint16_t *scales);

/* What[M,K] in fp64 (exact: level times scale). */
void oracle_dequant(const uint8_t *codes, const uint16_t *scales, int64_t M,
                    int64_t K, double *What);

/* y[m] = sum_k What[m,k] * x[k] (fp64, ascending k) and
 * S[m] = sum_k |What[m,k] * x[k]| for m in [row0,row1); x is bf16 bits.
 * y and S are indexed by m (full-length arrays). S may be NULL. */
void oracle_gemv_rows(const uint8_t *codes, const uint16_t *scales, int64_t M,
                      int64_t K, const uint16_t *x, int64_t row0, int64_t row1,
                      double *y, double *S);
void oracle_gemv(const uint8_t *codes, const uint16_t *scales, int64_t M,
                 int64_t K, const uint16_t *x, double *y, double *S);

/* Y[n,m] = sum_k What[m,k] * X[n,k] for n < N (X bf16 bits [N,K]); S alike. */
void oracle_gemm(const uint8_t *codes, const uint16_t *scales, int64_t M,
                 int64_t K, const uint16_t *X, int64_t N, double *Y, double *S);

/* SiLU(z) = z * sigmoid(z) = z / (1 + e^-z), fp64 (golang.design accel/tensor
 * page, func SiLU). */
double oracle_silu(double z);

/* The epilogue of a fused projection, fp64, for i < n (golang.design
 * accel/tensor page: func Linear adds the bias to the product, func SwiGLU is
 * SiLU(gate) * value; deep-fold "Decode V2" page, section 6 Linear primitive: q/k/v bias in
 * the projection, silu(g) * u after the full reduction, residual added into
 * y):
 *   a = t0[i] + bias0[i]                        (bias0 may be NULL)
 *   swiglu == 0: out[i] = a
 *   swiglu != 0: out[i] = silu(a) * (t1[i] + bias1[i])   (bias1 may be NULL)
 *   out[i] += residual[i]                       (residual may be NULL)
 * bias and residual are fp32 values widened exactly. */
void oracle_epilogue(const double *t0, const double *t1, const float *bias0,
                     const float *bias1, const float *residual, int64_t n,
                     int swiglu, double *out);

/* A finite double -> bfloat16 bits, one rounding to nearest, ties to even
 * (gizai tensor/lazy page, Lazy.roundedBf16: round to nearest even). */
uint16_t oracle_f64_to_bf16_rne(double v);

/* Packed row gather (deep-fold "Decode V2" page, section 6 run notes: the
 * embedding is kept as packed rows dequantised into the arena, and a tied
 * embedding reads the lm_head's packed matrix; golang.design accel/tensor
 * page, func QuantGatherRows).  For i < n with 0 <= ids[i] < M:
 *   out[i][k] = What[ids[i], k] rounded once to fp32 (bf16 == 0) or to bf16
 *               bits (bf16 != 0), nearest-even; What = c * s is exact.
 * An id outside [0, M) is a caller error (accel/tensor func GatherRows): its
 * row is written as zeros and ORACLE_GATHER_BAD_ID is returned in the flags. */
#define ORACLE_GATHER_BAD_ID 1
int32_t oracle_gather_rows(const uint8_t *codes, const uint16_t *scales, int64_t M,
                           int64_t K, const int32_t *ids, int64_t n, int bf16, void *out);

/* Affine 4-bit format (golang.design accel/tensor page: type Int4, func
 * Int4MatVec: What = (code - z) * s with an f16 scale and an f16 zero point
 * per group; the error is at most the group's range over 30).  Groups of 64
 * along K; codes laid out as the NF4 format; scales and zeros fp16 bits
 * [M][K/64].  The quantiser's steps are in oracle.c.  Returns the OR of
 * ORACLE_PACK_* flags; a flagged block's output is unspecified. */
int oracle_pack_affine_rows(const float *W, int64_t M, int64_t K, int64_t row0, int64_t row1,
                            uint8_t *codes, uint16_t *scales, uint16_t *zeros);
void oracle_dequant_affine(const uint8_t *codes, const uint16_t *scales, const uint16_t *zeros,
                           int64_t M, int64_t K, double *What);
void oracle_gemv_affine_rows(const uint8_t *codes, const uint16_t *scales, const uint16_t *zeros,
                             int64_t M, int64_t K, const uint16_t *x, int64_t row0, int64_t row1,
                             double *y, double *S);

/* NVFP4-style format (gizai tensor/lazy page, fp4Blocks): E2M1 codes (low
 * half first), one E4M3 scale per 16 values along K (row-major [M][K/16]
 * here), an f32 tensor scale s = max|W| / (6 * 448).  What = E2M1 * E4M3 * s.
 * The rounding steps the page leaves open are in oracle.c. */
double oracle_e4m3_to_f64(uint8_t b);
double oracle_e2m1_to_f64(uint8_t c);
/* s of W[0..n) (non-finite values are skipped and flagged in *status). */
float oracle_nvfp4_tensor_scale(const float *W, int64_t n, int *status);
int oracle_pack_nvfp4_rows(const float *W, int64_t M, int64_t K, int64_t row0, int64_t row1,
                           float s, uint8_t *codes, uint8_t *scales);
void oracle_dequant_nvfp4(const uint8_t *codes, const uint8_t *scales, float s, int64_t M,
                          int64_t K, double *What);
void oracle_gemv_nvfp4_rows(const uint8_t *codes, const uint8_t *scales, float s, int64_t M,
                            int64_t K, const uint16_t *x, int64_t row0, int64_t row1,
                            double *y, double *S);

/* int8 activations (deep-fold page, "The lane": one int8 word per
 * activation, or two of about 14 bits): per 32-block of x (bf16 bits [K]),
 * d = f32(max|x| / 127), q1 = nearest(x / d), q2 = nearest(128 (x - q1 d) / d)
 * (two words; q2 may be NULL for one), ties to even, within +-127.  The
 * carried value is xq = d (q1 + q2 / 128). */
void oracle_quantize_x8(const uint16_t *x, int64_t K, int words, int8_t *q1, int8_t *q2, float *d);
void oracle_dequantize_x8(const int8_t *q1, const int8_t *q2, const float *d, int64_t K, double *xq);
/* The affine format's GEMV on xq (q2 NULL: one word). */
void oracle_gemv_affine_x8_rows(const uint8_t *codes, const uint16_t *scales, const uint16_t *zeros,
                                int64_t M, int64_t K, const int8_t *q1, const int8_t *q2,
                                const float *d, int64_t row0, int64_t row1, double *y, double *S);

/* First index of the maximum (NaN never wins); -1 if n == 0 or all NaN. */
int64_t oracle_argmax_f64(const double *y, int64_t n);
int64_t oracle_argmax_f32(const float *y, int64_t n);

#ifdef __cplusplus
}
#endif
#endif
