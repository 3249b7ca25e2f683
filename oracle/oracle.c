/*
 * oracle.c -- plain, slow, obviously correct fp64 CPU oracle for the 4-bit
 * 16-level NF4-style codebook GEMV  y = dequant(W) . x  and its small-N GEMM
 * form  Y[n,:] = dequant(W) . X[n,:].
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call it; the
 * HIP library is checked against it.  It shares no code, header, table or
 * constant generator with the HIP library: the codebook here is computed
 * from its construction, the library carries its own frozen bit patterns.
 *
 * Build with plain gcc, no -ffast-math (every comparison below relies on
 * exact IEEE arithmetic).
 *
 * Where the pages fix a step it is cited by page and section; where they are
 * silent the reading taken is stated at the step.
 */
#include "oracle.h"

#include <math.h>
#include <string.h>

/* ------------------------------------------------------------------ *
 * Codebook.
 *
 * The deep-fold "Decode V2" page (section 6, "Linear primitive") names the
 * format NF4 and dequantises through "the 16-float table"; no page prints the
 * 16 values.  Reading taken: the NormalFloat-4 construction of the QLoRA
 * paper (Dettmers et al., 2023), asymmetric with an exact zero:
 *   - 8 positive levels: the standard-normal quantiles at 8 equally spaced
 *     probabilities running from 1 - delta down towards 1/2 (1/2 excluded);
 *   - 7 negative levels: minus the quantiles at 7 equally spaced
 *     probabilities over the same range (1/2 excluded);
 *   - one exact 0;
 *   - all divided by the largest quantile, so the extremes are -1 and +1;
 *   - delta = (1/30 + 1/32) / 2.
 * The levels are computed in fp64 and rounded once to fp32.
 * ------------------------------------------------------------------ */

/* Standard normal CDF written through erfc (no cancellation in the tails). */
static double phi(double z) { return 0.5 * erfc(-z / sqrt(2.0)); }

/* Upper tail 1 - phi(z), also through erfc. */
static double phi_upper(double z) { return 0.5 * erfc(z / sqrt(2.0)); }

double oracle_phi_inv(double p) {
    /* Bisection: phi is strictly increasing; stop when the bracket can no
     * longer shrink in fp64.  Above 1/2 the test is made on the upper tail,
     * phi(z) < p  <=>  1 - phi(z) > 1 - p, where 1 - p is exact and the tail
     * keeps full relative precision. */
    const int upper = p > 0.5;
    const double q = 1.0 - p; /* exact for p in [1/2, 1] */
    double lo = -40.0, hi = 40.0;
    for (int it = 0; it < 2000; ++it) {
        double mid = 0.5 * (lo + hi);
        if (mid <= lo || mid >= hi) break;
        int below = upper ? (phi_upper(mid) > q) : (phi(mid) < p);
        if (below)
            lo = mid;
        else
            hi = mid;
    }
    return 0.5 * (lo + hi);
}

void oracle_codebook_f64(double out[16]) {
    const double delta = 0.5 * (1.0 / 30.0 + 1.0 / 32.0);
    const double p_top = 1.0 - delta;
    const double top = oracle_phi_inv(p_top);
    /* negative levels, most negative first: out[0..6] */
    for (int j = 0; j < 7; ++j) {
        double p = p_top - (double)j * (p_top - 0.5) / 7.0;
        out[j] = -oracle_phi_inv(p) / top;
    }
    out[7] = 0.0;
    /* positive levels, smallest first: out[8..15] */
    for (int j = 0; j < 8; ++j) {
        double p = p_top - (double)(7 - j) * (p_top - 0.5) / 8.0;
        out[8 + j] = oracle_phi_inv(p) / top;
    }
    /* j == 0 on both sides divides the top quantile by itself: exactly -1
     * and +1. */
}

void oracle_codebook_f32(float out[16]) {
    double d[16];
    oracle_codebook_f64(d);
    for (int i = 0; i < 16; ++i) out[i] = (float)d[i];
}

/* ------------------------------------------------------------------ *
 * Number formats.
 *
 * golang.design accel/tensor, func Cast: f32 -> f16 rounds to nearest-even,
 * and a value outside the f16 range becomes an infinity; bf16 -> f32 is exact
 * (bf16 is the top half of f32).
 * ------------------------------------------------------------------ */

void oracle_f32_to_f16_rne_array(const float *v, int64_t n, uint16_t *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_f16_rne(v[i]);
}

double oracle_f16_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0x1f)
        v = m ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
    else
        v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) 2^(e-15) */
    return sign ? -v : v;
}

double oracle_bf16_to_f64(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

uint16_t oracle_f32_to_f16_rne(float v) { return oracle_f64_to_f16_rne((double)v); }

uint16_t oracle_f64_to_f16_rne(double v) {
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    if (isnan(v)) return (uint16_t)(sign | 0x7e00);
    double a = fabs(v);
    /* Halfway between the largest finite half (65504) and the next step
     * (65536) is 65520; ties-to-even goes up there, so >= 65520 is inf. */
    if (a >= 65520.0) return (uint16_t)(sign | 0x7c00);
    /* Spacing of representable halves around a: 2^-24 below 2^-14
     * (subnormals), else 2^(floor(log2 a) - 10). */
    double q;
    if (a < ldexp(1.0, -14)) {
        q = ldexp(1.0, -24);
    } else {
        int ex;
        frexp(a, &ex); /* a = f 2^ex, f in [0.5, 1) => floor(log2 a) = ex-1 */
        q = ldexp(1.0, ex - 1 - 10);
    }
    double n = a / q; /* exact: q is a power of two */
    double fl = floor(n);
    double frac = n - fl; /* exact */
    double r;
    if (frac > 0.5)
        r = fl + 1.0;
    else if (frac < 0.5)
        r = fl;
    else
        r = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0; /* tie: to even */
    double u = r * q; /* the rounded magnitude, exactly a half value */
    if (u == 0.0) return sign;
    if (u < ldexp(1.0, -14)) /* subnormal half: mantissa = u / 2^-24 */
        return (uint16_t)(sign | (uint16_t)(u / ldexp(1.0, -24)));
    int ex;
    double f = frexp(u, &ex);          /* u = f 2^ex, f in [0.5,1) */
    int E = ex - 1;                    /* u = (2f) 2^E, 2f in [1,2) */
    int mant = (int)((2.0 * f - 1.0) * 1024.0); /* exact */
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)mant);
}

/* ------------------------------------------------------------------ *
 * Quantisation (pack).
 *
 * Groups of 64 weights along K (deep-fold "Decode V2", section 2: hidden and
 * intermediate sizes are multiples of 64, the NF4 group).  Reading taken for
 * the unprinted steps:
 *   - scale: the block's absolute maximum, stored as fp16 (round to nearest
 *     even); blocks whose absmax rounds to fp16 infinity, and blocks holding
 *     a non-finite weight, are refused (accel/tensor, func Cast: an
 *     out-of-range value becomes infinity, and a silently clamped weight is
 *     not allowed);
 *   - the codes are chosen against the stored fp16 scale s: the level nearest
 *     to w / s in exact arithmetic, an exact midpoint going to the lower
 *     level; written without division as
 *         code = #{ i in 0..14 : w > m_i * s },  m_i = (c_i + c_{i+1}) / 2,
 *     every product and comparison exact in fp64 (m_i has at most 25
 *     significant bits, s at most 11);
 *   - a block whose scale is 0 gets code 7 (the exact zero level) throughout;
 *   - packing: byte j of a row holds code 2j in its low nibble and code 2j+1
 *     in its high nibble (accel/tensor, type Int4: low nibble first).
 * ------------------------------------------------------------------ */

int oracle_pack_rows(const float *W, int64_t M, int64_t K, int64_t row0,
                     int64_t row1, uint8_t *codes, uint16_t *scales) {
    (void)M;
    float cb[16];
    oracle_codebook_f32(cb);
    double mid[15];
    for (int i = 0; i < 15; ++i) mid[i] = ((double)cb[i] + (double)cb[i + 1]) / 2.0;

    const int64_t nblk = K / 64;
    int status = 0;
    for (int64_t m = row0; m < row1; ++m) {
        for (int64_t b = 0; b < nblk; ++b) {
            const float *w = W + m * K + b * 64;
            float amax = 0.0f;
            int bad = 0;
            for (int k = 0; k < 64; ++k) {
                if (!isfinite(w[k])) bad = 1;
                float aw = fabsf(w[k]);
                if (aw > amax) amax = aw;
            }
            if (bad) {
                status |= ORACLE_PACK_NONFINITE;
                continue;
            }
            uint16_t s16 = oracle_f32_to_f16_rne(amax);
            if (s16 == 0x7c00) {
                status |= ORACLE_PACK_OVERFLOW;
                continue;
            }
            scales[m * nblk + b] = s16;
            double s = oracle_f16_to_f64(s16);
            uint8_t code[64];
            for (int k = 0; k < 64; ++k) {
                if (s == 0.0) {
                    code[k] = 7;
                    continue;
                }
                int c = 0;
                for (int i = 0; i < 15; ++i)
                    if ((double)w[k] > mid[i] * s) ++c;
                code[k] = (uint8_t)c;
            }
            uint8_t *dst = codes + m * (K / 2) + b * 32;
            for (int j = 0; j < 32; ++j)
                dst[j] = (uint8_t)(code[2 * j] | (code[2 * j + 1] << 4));
        }
    }
    return status;
}

int oracle_pack(const float *W, int64_t M, int64_t K, uint8_t *codes,
                uint16_t *scales) {
    return oracle_pack_rows(W, M, K, 0, M, codes, scales);
}

/* ------------------------------------------------------------------ *
 * Dequantisation and products.
 *
 * deep-fold "Decode V2", section 3 (CPU oracle): the NF4 linear is decode
 * then matmul, Y = What @ x; section 6: the value of a weight is the table
 * entry of its code times its group's scale.  Here every What = c * s is
 * exact in fp64 (24 + 11 significant bits), x is bf16 widened exactly, every
 * product What * x is exact (at most 43 bits), and the sum runs over
 * ascending k in fp64.  S is the sum of |What * x|, the scale of the
 * acceptance bound.
 * ------------------------------------------------------------------ */

static int code_at(const uint8_t *codes, int64_t K, int64_t m, int64_t k) {
    uint8_t byte = codes[m * (K / 2) + k / 2];
    return (k % 2 == 0) ? (byte & 0xf) : (byte >> 4);
}

void oracle_dequant(const uint8_t *codes, const uint16_t *scales, int64_t M,
                    int64_t K, double *What) {
    float cb[16];
    oracle_codebook_f32(cb);
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k) {
            double s = oracle_f16_to_f64(scales[m * (K / 64) + k / 64]);
            What[m * K + k] = (double)cb[code_at(codes, K, m, k)] * s;
        }
}

void oracle_gemv_rows(const uint8_t *codes, const uint16_t *scales, int64_t M,
                      int64_t K, const uint16_t *x, int64_t row0, int64_t row1,
                      double *y, double *S) {
    (void)M;
    float cb[16];
    oracle_codebook_f32(cb);
    for (int64_t m = row0; m < row1; ++m) {
        double acc = 0.0, mag = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double s = oracle_f16_to_f64(scales[m * (K / 64) + k / 64]);
            double w = (double)cb[code_at(codes, K, m, k)] * s;
            double t = w * oracle_bf16_to_f64(x[k]);
            acc += t;
            mag += fabs(t);
        }
        y[m] = acc;
        if (S) S[m] = mag;
    }
}

void oracle_gemv(const uint8_t *codes, const uint16_t *scales, int64_t M,
                 int64_t K, const uint16_t *x, double *y, double *S) {
    oracle_gemv_rows(codes, scales, M, K, x, 0, M, y, S);
}

void oracle_gemm(const uint8_t *codes, const uint16_t *scales, int64_t M,
                 int64_t K, const uint16_t *X, int64_t N, double *Y, double *S) {
    /* The prefill form is the same product for each of the N rows of X
     * (accel/tensor, func Int4MatMul: the same representation and
     * reconstruction as the vector form). */
    for (int64_t n = 0; n < N; ++n)
        oracle_gemv_rows(codes, scales, M, K, X + n * K, 0, M, Y + n * M,
                         S ? S + n * M : (double *)0);
}

/* accel/tensor, func Argmax: the index of the largest value, ties to the
 * lowest index. */
int64_t oracle_argmax_f64(const double *y, int64_t n) {
    int64_t best = -1;
    for (int64_t i = 0; i < n; ++i)
        if (!isnan(y[i]) && (best < 0 || y[i] > y[best])) best = i;
    return best;
}

int64_t oracle_argmax_f32(const float *y, int64_t n) {
    int64_t best = -1;
    for (int64_t i = 0; i < n; ++i)
        if (!isnan(y[i]) && (best < 0 || y[i] > y[best])) best = i;
    return best;
}

/* ------------------------------------------------------------------------ */
/* Fused-projection epilogue (accel/tensor func Linear, func SiLU,           */
/* func SwiGLU; deep-fold "Decode V2", section 6 Linear primitive).                          */
/* ------------------------------------------------------------------------ */

double oracle_silu(double z) { return z / (1.0 + exp(-z)); }

void oracle_epilogue(const double *t0, const double *t1, const float *bias0, const float *bias1,
                     const float *residual, int64_t n, int swiglu, double *out) {
    for (int64_t i = 0; i < n; ++i) {
        double a = t0[i];
        if (bias0) a += (double)bias0[i];
        double v = a;
        if (swiglu) {
            double b = t1[i];
            if (bias1) b += (double)bias1[i];
            v = oracle_silu(a) * b;
        }
        if (residual) v += (double)residual[i];
        out[i] = v;
    }
}

/* ------------------------------------------------------------------------ */
/* Packed row gather (deep-fold "Decode V2" page, run notes of section 6:    */
/* the embedding stays packed, its rows are dequantised into the arena, and  */
/* a tied embedding shares the lm_head's packed matrix; golang.design        */
/* accel/tensor, func QuantGatherRows: rows gathered from a quantized table). */
/* ------------------------------------------------------------------------ */

/* A finite double -> bfloat16 bits, rounded once to nearest, ties to even.
 * bf16 keeps 8 significant bits and the fp32 exponent range: the spacing of
 * representable values around a normal a is 2^(floor(log2 a) - 7), and
 * 2^-133 below 2^-126.  Magnitudes that round past the largest finite bf16
 * become infinity. */
uint16_t oracle_f64_to_bf16_rne(double v) {
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    if (isnan(v)) return (uint16_t)(sign | 0x7fc0);
    double a = fabs(v);
    if (a == 0.0) return sign;
    double q;
    if (a < ldexp(1.0, -126)) {
        q = ldexp(1.0, -133);
    } else {
        int ex;
        frexp(a, &ex); /* floor(log2 a) = ex - 1 */
        q = ldexp(1.0, ex - 1 - 7);
    }
    double n = a / q; /* exact: q is a power of two */
    double fl = floor(n);
    double frac = n - fl;
    double r;
    if (frac > 0.5)
        r = fl + 1.0;
    else if (frac < 0.5)
        r = fl;
    else
        r = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
    double u = r * q; /* the rounded magnitude */
    if (u >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7f80);
    float f = (float)u; /* exact: u has at most 8 significant bits */
    uint32_t bits;
    memcpy(&bits, &f, sizeof bits);
    return (uint16_t)(sign | (uint16_t)(bits >> 16));
}

int32_t oracle_gather_rows(const uint8_t *codes, const uint16_t *scales, int64_t M, int64_t K,
                           const int32_t *ids, int64_t n, int bf16, void *out) {
    float cb[16];
    oracle_codebook_f32(cb);
    int32_t flags = 0;
    for (int64_t i = 0; i < n; ++i) {
        const int64_t m = ids[i];
        if (m < 0 || m >= M) {
            /* accel/tensor func GatherRows: an out-of-range id is a caller
             * error and its row comes out as zeros, never read from outside
             * the table; the flag is the diagnostic. */
            flags |= ORACLE_GATHER_BAD_ID;
            for (int64_t k = 0; k < K; ++k) {
                if (bf16)
                    ((uint16_t *)out)[i * K + k] = 0;
                else
                    ((float *)out)[i * K + k] = 0.0f;
            }
            continue;
        }
        for (int64_t k = 0; k < K; ++k) {
            const double sc = oracle_f16_to_f64(scales[m * (K / 64) + k / 64]);
            const double w = (double)cb[code_at(codes, K, m, k)] * sc; /* exact */
            if (bf16)
                ((uint16_t *)out)[i * K + k] = oracle_f64_to_bf16_rne(w);
            else
                ((float *)out)[i * K + k] = (float)w; /* one rounding, nearest-even */
        }
    }
    return flags;
}

/* ------------------------------------------------------------------------ */
/* Affine 4-bit format (golang.design accel/tensor: type Int4 holds 4-bit    */
/* codes, low nibble first, with an f16 scale and an f16 zero point per      */
/* group; func Int4MatVec reconstructs a weight as (code - z) * s; the       */
/* accuracy stated there is a group's range over 30).  Reading taken for the */
/* quantiser, which the page does not print:                                 */
/*   - groups of 64 weights along K, as the NF4 format;                      */
/*   - the group's range [lo, hi] is widened to hold 0 (so the zero point is */
/*     a code and an all-zero group is exact); s = fp16 RNE of              */
/*     (hi - lo) / 15 (fp64 subtraction and division, one rounding each),    */
/*     so the spacing of the levels is the range over 15 and the error at    */
/*     most half of it: the range over 30;                                   */
/*   - z = the integer nearest to -lo / s in 0..15, an exact midpoint going  */
/*     down, written as #{ j in 0..14 : -lo > (j + 1/2) s }; stored as f16   */
/*     (exact);                                                              */
/*   - code = the level (j - z) s nearest to w, an exact midpoint going to   */
/*     the lower code: #{ j in 0..14 : w > (j - z + 1/2) s }.  Every product */
/*     and comparison is exact (a half-integer of at most 5 bits times an    */
/*     11-bit s, against an fp32 w);                                         */
/*   - s == 0 (the widened range is 0 or below the fp16 range): codes 0 and  */
/*     z = 0, every weight reconstructs to 0;                                */
/*   - refusals as the NF4 pack: a non-finite weight, or s rounding to       */
/*     infinity.                                                             */
/* ------------------------------------------------------------------------ */

int oracle_pack_affine_rows(const float *W, int64_t M, int64_t K, int64_t row0, int64_t row1,
                            uint8_t *codes, uint16_t *scales, uint16_t *zeros) {
    (void)M;
    const int64_t nblk = K / 64;
    int status = 0;
    for (int64_t m = row0; m < row1; ++m) {
        for (int64_t b = 0; b < nblk; ++b) {
            const float *w = W + m * K + b * 64;
            float lo = 0.0f, hi = 0.0f;
            int bad = 0;
            for (int k = 0; k < 64; ++k) {
                if (!isfinite(w[k])) bad = 1;
                if (w[k] < lo) lo = w[k];
                if (w[k] > hi) hi = w[k];
            }
            if (bad) {
                status |= ORACLE_PACK_NONFINITE;
                continue;
            }
            const uint16_t s16 = oracle_f64_to_f16_rne(((double)hi - (double)lo) / 15.0);
            if (s16 == 0x7c00) {
                status |= ORACLE_PACK_OVERFLOW;
                continue;
            }
            const double s = oracle_f16_to_f64(s16);
            int z = 0;
            if (s > 0.0)
                for (int j = 0; j < 15; ++j)
                    if (-(double)lo > ((double)j + 0.5) * s) ++z;
            scales[m * nblk + b] = s16;
            zeros[m * nblk + b] = oracle_f64_to_f16_rne((double)z);
            uint8_t code[64];
            for (int k = 0; k < 64; ++k) {
                int c = 0;
                if (s > 0.0)
                    for (int j = 0; j < 15; ++j)
                        if ((double)w[k] > ((double)(j - z) + 0.5) * s) ++c;
                code[k] = (uint8_t)c;
            }
            uint8_t *out = codes + m * (K / 2) + b * 32;
            for (int j = 0; j < 32; ++j)
                out[j] = (uint8_t)((code[2 * j + 1] << 4) | code[2 * j]); /* low nibble first */
        }
    }
    return status;
}

void oracle_dequant_affine(const uint8_t *codes, const uint16_t *scales, const uint16_t *zeros, int64_t M,
                           int64_t K, double *What) {
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k) {
            const int64_t g = m * (K / 64) + k / 64;
            What[m * K + k] = ((double)code_at(codes, K, m, k) - oracle_f16_to_f64(zeros[g])) *
                              oracle_f16_to_f64(scales[g]); /* exact */
        }
}

/* y[m] = sum_k What[m,k] x[k] in fp64 over ascending k (each term exact), and
 * S[m] = sum_k |What[m,k] x[k]|, for m in [row0, row1). */
void oracle_gemv_affine_rows(const uint8_t *codes, const uint16_t *scales, const uint16_t *zeros, int64_t M,
                             int64_t K, const uint16_t *x, int64_t row0, int64_t row1, double *y, double *S) {
    (void)M;
    for (int64_t m = row0; m < row1; ++m) {
        double acc = 0.0, mag = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const int64_t g = m * (K / 64) + k / 64;
            const double w = ((double)code_at(codes, K, m, k) - oracle_f16_to_f64(zeros[g])) *
                             oracle_f16_to_f64(scales[g]);
            const double term = w * oracle_bf16_to_f64(x[k]);
            acc += term;
            mag += fabs(term);
        }
        y[m] = acc;
        if (S) S[m] = mag;
    }
}

/* ------------------------------------------------------------------------ */
/* NVFP4-style format (gizai tensor/lazy page, fp4Blocks: E2M1 codes, two to */
/* a byte with the first in the low half; one E4M3 scale per 16 values along */
/* k; a tensor scale s = max |t| / (6 * 448) in f32; a value is its E2M1    */
/* times its block's scale times s).  Reading taken for the steps the page   */
/* leaves open:                                                              */
/*   - s = the f32 rounding of the fp64 quotient max|W| / 2688;             */
/*   - a block's scale is the E4M3 value nearest to amax_b / (6 s), ties to  */
/*     the even pattern, at most 448 (s == 0: scale 0);                      */
/*   - a weight's code is the E2M1 magnitude nearest to |w| / (scale * s),   */
/*     ties to the even pattern, at most 6, with w's sign bit; a block whose */
/*     scale is 0 is all code 0;                                             */
/*   - every decision compares against a midpoint times 6 s or scale * s:    */
/*     midpoints of at most 5 significant bits, 6 of 2, an E4M3 of 4 and s   */
/*     of 24, so each product and comparison is exact in fp64;               */
/*   - scales are stored row-major, [M][K/16] (not the page's tensor-core   */
/*     interleave).                                                          */
/* ------------------------------------------------------------------------ */

/* The value of an E4M3 (OCP E4M3FN: bias 7, no infinities, 0x7F NaN) byte. */
double oracle_e4m3_to_f64(uint8_t b) {
    const int sign = b >> 7, e = (b >> 3) & 15, m = b & 7;
    double v;
    if (e == 15 && m == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)m, -9); /* (m / 8) 2^-6 */
    else
        v = ldexp(8.0 + m, e - 10); /* (1 + m / 8) 2^(e - 7) */
    return sign ? -v : v;
}

/* The value of an E2M1 code (sign bit 3): 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
double oracle_e2m1_to_f64(uint8_t c) {
    static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    const double v = mag[c & 7];
    return (c & 8) ? -v : v;
}

/* Nearest of the ascending grid g[0..n-1] to a >= 0 scaled by u (a against
 * g[i] * u), ties to the even index; a above the grid saturates. */
static int nearest_on_grid(double a, const double *g, int n, double u) {
    int i = 0;
    while (i + 1 < n) {
        const double mid = (g[i] + g[i + 1]) / 2.0 * u; /* exact */
        if (a > mid || (a == mid && (i & 1))) {
            ++i;
            continue;
        }
        break;
    }
    return i;
}

float oracle_nvfp4_tensor_scale(const float *W, int64_t n, int *status) {
    double amax = 0.0;
    *status = 0;
    for (int64_t i = 0; i < n; ++i) {
        if (!isfinite(W[i])) {
            *status |= ORACLE_PACK_NONFINITE;
            continue;
        }
        if (fabs((double)W[i]) > amax) amax = fabs((double)W[i]);
    }
    return (float)(amax / 2688.0);
}

int oracle_pack_nvfp4_rows(const float *W, int64_t M, int64_t K, int64_t row0, int64_t row1, float s,
                           uint8_t *codes, uint8_t *scales) {
    (void)M;
    static double e4m3[127]; /* positive E4M3 values, ascending (0x00 .. 0x7E) */
    static const double e2m1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    for (int b = 0; b < 127; ++b) e4m3[b] = oracle_e4m3_to_f64((uint8_t)b);
    int status = 0;
    const int64_t nblk = K / 16;
    for (int64_t m = row0; m < row1; ++m) {
        for (int64_t b = 0; b < nblk; ++b) {
            const float *w = W + m * K + b * 16;
            double amax = 0.0;
            int bad = 0;
            for (int k = 0; k < 16; ++k) {
                if (!isfinite(w[k])) bad = 1;
                else if (fabs((double)w[k]) > amax) amax = fabs((double)w[k]);
            }
            if (bad) {
                status |= ORACLE_PACK_NONFINITE;
                continue;
            }
            const int sb = (s > 0.0f) ? nearest_on_grid(amax, e4m3, 127, 6.0 * (double)s) : 0;
            scales[m * nblk + b] = (uint8_t)sb;
            const double unit = e4m3[sb] * (double)s; /* exact */
            for (int k = 0; k < 16; k += 2) {
                uint8_t c[2];
                for (int h = 0; h < 2; ++h) {
                    const double wv = (double)w[k + h];
                    if (unit == 0.0) {
                        c[h] = 0;
                        continue;
                    }
                    const int mag = nearest_on_grid(fabs(wv), e2m1, 8, unit);
                    c[h] = (uint8_t)(mag | (signbit(wv) ? 8 : 0));
                }
                codes[m * (K / 2) + b * 8 + k / 2] = (uint8_t)(c[0] | (c[1] << 4));
            }
        }
    }
    return status;
}

/* What[m,k] = E2M1(code) * E4M3(scale) * s, exact in fp64. */
void oracle_dequant_nvfp4(const uint8_t *codes, const uint8_t *scales, float s, int64_t M, int64_t K,
                          double *What) {
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k)
            What[m * K + k] = oracle_e2m1_to_f64((uint8_t)code_at(codes, K, m, k)) *
                              oracle_e4m3_to_f64(scales[m * (K / 16) + k / 16]) * (double)s;
}

void oracle_gemv_nvfp4_rows(const uint8_t *codes, const uint8_t *scales, float s, int64_t M, int64_t K,
                            const uint16_t *x, int64_t row0, int64_t row1, double *y, double *S) {
    (void)M;
    for (int64_t m = row0; m < row1; ++m) {
        double sum = 0.0, absum = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double wq = oracle_e2m1_to_f64((uint8_t)code_at(codes, K, m, k)) *
                              oracle_e4m3_to_f64(scales[m * (K / 16) + k / 16]) * (double)s;
            const double prod = wq * oracle_bf16_to_f64(x[k]); /* exact */
            sum += prod;
            absum += fabs(prod);
        }
        y[m] = sum;
        if (S) S[m] = absum;
    }
}

/* ------------------------------------------------------------------------ */
/* int8 activations for the integer-code (affine) format (deep-fold page's  */
/* lane knobs, section "The lane": a projection's activation may be one     */
/* int8 word, as llama.cpp does, or two int8 words of about 14 bits, the    */
/* default).  Reading taken:                                                 */
/*   - blocks of 32 activations along K (one 16-byte code chunk);           */
/*   - d = the f32 rounding of the fp64 quotient max|x_block| / 127;        */
/*   - q1 = the integer nearest to x / d, ties to even, within +-127;       */
/*   - two words: r = x - q1 d (exact) and q2 = the integer nearest to      */
/*     128 r / d, ties to even, within +-127 (|r| <= d/2 keeps it in +-64);   */
/*   - the value carried is xq = d (q1 + q2 / 128) (q2 = 0 for one word);   */
/*   - every decision compares |x| (or |r|) with (j + 1/2) d (or / 128),    */
/*     exact in fp64, so any implementation decides alike.                  */
/* The product then uses xq in place of x: the GEMV tolerance applies to    */
/* sum What xq, and |x - xq| <= d / 2 (one word) or d / 256 (two words).    */
/* ------------------------------------------------------------------------ */

/* Nearest integer to a / u (a >= 0, u > 0) in 0..127, ties to even, by
 * comparisons with (j + 1/2) u. */
static int nearest_int_127(double a, double u) {
    int j = 0;
    while (j < 127) {
        const double mid = ((double)j + 0.5) * u;
        if (a > mid || (a == mid && (j & 1))) ++j;
        else break;
    }
    return j;
}

void oracle_quantize_x8(const uint16_t *x, int64_t K, int words, int8_t *q1, int8_t *q2, float *d) {
    for (int64_t b = 0; b < K / 32; ++b) {
        double amax = 0.0;
        for (int k = 0; k < 32; ++k) {
            const double v = fabs(oracle_bf16_to_f64(x[b * 32 + k]));
            if (v > amax) amax = v;
        }
        const float db = (float)(amax / 127.0);
        d[b] = db;
        for (int k = 0; k < 32; ++k) {
            const int64_t i = b * 32 + k;
            const double v = oracle_bf16_to_f64(x[i]);
            int a1 = 0, a2 = 0;
            if (db > 0.0f) {
                a1 = nearest_int_127(fabs(v), (double)db);
                if (v < 0) a1 = -a1;
                if (words == 2) {
                    const double r = v - (double)a1 * (double)db; /* exact */
                    a2 = nearest_int_127(fabs(r), (double)db / 128.0);
                    if (r < 0) a2 = -a2;
                }
            }
            q1[i] = (int8_t)a1;
            if (words == 2) q2[i] = (int8_t)a2;
        }
    }
}

/* xq[k] = d (q1 + q2 / 128), exact in fp64 (q2 NULL: one word). */
void oracle_dequantize_x8(const int8_t *q1, const int8_t *q2, const float *d, int64_t K, double *xq) {
    for (int64_t k = 0; k < K; ++k)
        xq[k] = (double)d[k / 32] * ((double)q1[k] + (q2 ? (double)q2[k] / 128.0 : 0.0));
}

/* The affine format's GEMV on int8 activations: y[m] = sum_k What[m,k] xq[k]
 * (each term exact in fp64, ascending k), S[m] = sum_k |What[m,k] xq[k]|. */
void oracle_gemv_affine_x8_rows(const uint8_t *codes, const uint16_t *scales, const uint16_t *zeros, int64_t M,
                                int64_t K, const int8_t *q1, const int8_t *q2, const float *d, int64_t row0,
                                int64_t row1, double *y, double *S) {
    (void)M;
    for (int64_t m = row0; m < row1; ++m) {
        double total = 0.0, size = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const int64_t g = m * (K / 64) + k / 64;
            const double wv = ((double)code_at(codes, K, m, k) - oracle_f16_to_f64(zeros[g])) *
                              oracle_f16_to_f64(scales[g]);
            const double xv = (double)d[k / 32] * ((double)q1[k] + (q2 ? (double)q2[k] / 128.0 : 0.0));
            total += wv * xv;
            size += fabs(wv * xv);
        }
        y[m] = total;
        if (S) S[m] = size;
    }
}
