/*
 * oracle.c -- CPU reference for row-wise RMSNorm forward, its backward (dX and
 * the weight gradient dW) and the fused residual-add + RMSNorm + FP8 e4m3
 * 1x128 block-quant producer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the independent checker of the HIP
 * library.  Only the test suite, the smoke check and the benchmark's CPU
 * baseline may load it; the product path never calls it and shares no code,
 * header, table or helper with it.
 *
 * Everything is plain, sequential C in FP64 (built without fast-math and with
 * floating-point contraction off).  Inputs are decoded exactly to double with
 * this file's own bf16 / fp32 decoders; results that the method defines in FP64
 * are returned unrounded, so a test can state its tolerance against the exact
 * value.  The two places where the method itself fixes fp32 arithmetic (the
 * per-block scale and the quotient that is quantised) are computed in fp32
 * exactly as the method states them.
 *
 * Sources (the method is defined on these pages; no code was taken from them):
 *  - FlashInfer commit #5741 "cake_rmsnorm_train" (quoted on the FlashInfer
 *    PR #4480 page), sections Summary, Design (Forward / Backward) and
 *    Accuracy: y = x*rstd*w with the fp32 reciprocal RMS saved for the
 *    backward; dx = rstd*(g*w - mean(g*w*xhat)*xhat); dw the column sum of
 *    g*x*rstd over rows; h_new = bf16(x + residual) is what gets normalised.
 *  - FlashInfer PR #4480 "Add FusedAddRMSNormFP8BlockQuant", description
 *    (Kernel, API) and the review thread: residual updated in place with the
 *    pre-norm sum, bf16 normed output, fp32 scale = amax/448 per 1x128 block
 *    in the column-major (H/128, round_up(T,4)) layout, e4m3 codes quantised
 *    from the bf16-rounded normed values.
 *  - FlashInfer PR #6332 (QKV projection + QK-RMSNorm + RoPE overlapped with
 *    the Ulysses head exchange), Description, operator math: per-head fp32
 *    RMSNorm over head_dim with one shared weight per Q or K.
 *
 * Readings taken where the pages are silent (each is also listed in the
 * design notes of the repository):
 *  R1  rstd = 1/sqrt(mean(x^2) + eps): eps is added to the mean inside the
 *      square root; the weight multiplies as plain w (not 1+w).
 *  R2  eps is the fp32 value passed by the caller, widened exactly to double.
 *  R3  the backward uses the forward's stored rstd (an input), not a
 *      recomputation from x.
 *  R4  the fused producer normalises the bf16-rounded sum h = bf16(x + r).
 *  R5  scale = fp32(amax) / 448.0f as one IEEE fp32 division (round to
 *      nearest even); an all-zero block has scale 0 and all codes 0x00.
 *  R6  code = e4m3fn(fp32(n) / scale): IEEE fp32 division, then round to
 *      nearest even onto the E4M3FN grid, saturating to +-448, sign kept
 *      (a negative value that rounds to zero is 0x80).
 *  R7  scale layout: element (row m, block k) lives at scale[k*scale_ld + m];
 *      padding rows m in [T, scale_ld) are not written.
 *  R11 the training forward with a residual stores h_new = x + u rounded once
 *      into the dtype of x (bf16 or fp32) and normalises that rounded h_new.
 *  R12 the training backward with a residual-stream gradient returns
 *      dx_total = dx + g_residual, the sum taken before the one rounding
 *      into the output dtype; dw is unchanged by g_residual.
 *  R13 per-head RMSNorm treats every (token, head) slice of head_dim
 *      contiguous values as one row, with the same [head_dim] weight for all
 *      heads; rstd is indexed token-major, rstd[t*heads + h].
 *  R14 producer variants: fp16 rows work as bf16 rows do (h, normed rounded
 *      to fp16); an e5m2 output uses MAX = 57344 in place of 448 (scale =
 *      amax / MAX); with a given per-tensor scale s every block uses s, and
 *      codes = satfinite(n / s) (IEEE fp32 quotient, nearest-even, clamped
 *      to +-MAX).
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <stdint.h>
#include <string.h>

#define RNO_F32 0
#define RNO_BF16 1
#define RNO_F16 2
#define RNO_E4M3 0
#define RNO_E5M2 1

/* ------------------------------------------------------------------------ */
/* bf16 codec (bf16 = the upper 16 bits of an IEEE binary32).                */
/* ------------------------------------------------------------------------ */

/* Exact decode: a bf16 pattern is a binary32 whose low 16 bits are zero. */
double rno_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a double to the nearest bf16 value, ties to even, in one rounding.
 * bf16 has 8 significant bits, the binary32 exponent range and subnormals
 * down to 2^-133.  Values at or beyond the overflow threshold become +-inf
 * (never produced by the workloads here). */
uint16_t rno_double_to_bf16(double v)
{
    if (isnan(v)) return 0x7FC0;
    int neg = signbit(v) ? 1 : 0;
    double a = fabs(v);
    uint16_t sign = neg ? 0x8000 : 0;
    if (a == 0.0) return sign;
    int e;
    (void)frexp(a, &e);               /* a = f * 2^e, 0.5 <= f < 1 */
    int qexp = e - 8;                 /* quantum of an 8-significant-bit value */
    if (qexp < -133) qexp = -133;     /* bf16 subnormal quantum */
    double quantum = ldexp(1.0, qexp);
    double k = a / quantum;           /* exact: division by a power of two */
    double fl = floor(k);
    double frac = k - fl;
    if (frac > 0.5 || (frac == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;
    double r = fl * quantum;          /* exactly representable in bf16 */
    if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80);
    float rf = (float)r;              /* exact: bf16 values are binary32 values */
    uint32_t u;
    memcpy(&u, &rf, sizeof u);
    return (uint16_t)(sign | ((u >> 16) & 0x7FFF));
}

/* ------------------------------------------------------------------------ */
/* E4M3FN codec: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinity;  */
/* S.1111.111 is NaN; largest finite 1.75 * 2^8 = 448; subnormals k * 2^-9.  */
/* ------------------------------------------------------------------------ */

double rno_e4m3_to_double(uint8_t c)
{
    int neg = (c >> 7) & 1;
    int ex = (c >> 3) & 0xF;
    int m = c & 7;
    double v;
    if (ex == 0xF && m == 7) return NAN;
    if (ex == 0)
        v = ldexp((double)m, -9);                 /* m/8 * 2^-6 */
    else
        v = ldexp(1.0 + m / 8.0, ex - 7);
    return neg ? -v : v;
}

/* Encode an exactly representable non-negative E4M3 magnitude into 7 bits. */
static uint8_t encode_e4m3_magnitude(double r)
{
    if (r == 0.0) return 0;
    if (r < ldexp(1.0, -6))                        /* subnormal: r = m * 2^-9 */
        return (uint8_t)(r / ldexp(1.0, -9));
    int e;
    double f = frexp(r, &e);                       /* r = f * 2^e, f in [0.5,1) */
    int ex = e - 1 + 7;                            /* r = (2f) * 2^(e-1) */
    int m = (int)((2.0 * f - 1.0) * 8.0);          /* exact for grid values */
    return (uint8_t)((ex << 3) | m);
}

/* Round a binary32 value to E4M3FN, nearest-even, saturating to +-448. */
uint8_t rno_float_to_e4m3(float v)
{
    if (isnan(v)) return 0x7F;
    uint8_t sign = signbit(v) ? 0x80 : 0;
    double a = fabs((double)v);
    if (a >= 448.0) return (uint8_t)(sign | 0x7E);
    int qexp;
    if (a < ldexp(1.0, -6)) {
        qexp = -9;                                 /* subnormal spacing */
    } else {
        int e;
        (void)frexp(a, &e);                        /* a in [2^(e-1), 2^e) */
        qexp = (e - 1) - 3;                        /* 3 mantissa bits */
    }
    double quantum = ldexp(1.0, qexp);
    double k = a / quantum;                        /* exact */
    double fl = floor(k);
    double frac = k - fl;
    if (frac > 0.5 || (frac == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;
    double r = fl * quantum;                       /* may carry into next binade */
    if (r > 448.0) r = 448.0;
    return (uint8_t)(sign | encode_e4m3_magnitude(r));
}

/* ------------------------------------------------------------------------ */
/* Element access.                                                           */
/* ------------------------------------------------------------------------ */

static double load_elem(const void* base, int dtype, int64_t idx)
{
    if (dtype == RNO_BF16) return rno_bf16_to_double(((const uint16_t*)base)[idx]);
    return (double)((const float*)base)[idx];
}

/* ------------------------------------------------------------------------ */
/* RMSNorm forward.                                                          */
/* Cake commit #5741, Design: Forward -- per row an fp32 sum of squares, the */
/* reciprocal RMS rstd, y = x*rstd*w.  Here every step is FP64 and y is      */
/* returned unrounded (readings R1, R2).                                     */
/* ------------------------------------------------------------------------ */

int rno_rmsnorm_fwd(const void* x, int64_t ldx, int x_dtype,
                    const void* w, int w_dtype,
                    int64_t T, int64_t H, float eps,
                    double* y, int64_t ldy,      /* may be NULL */
                    double* rstd)                /* may be NULL */
{
    if (T < 0 || H <= 0) return 1;
    for (int64_t r = 0; r < T; ++r) {
        double ss = 0.0;
        for (int64_t j = 0; j < H; ++j) {
            double v = load_elem(x, x_dtype, r * ldx + j);
            ss += v * v;
        }
        double ms = ss / (double)H;
        double rs = 1.0 / sqrt(ms + (double)eps);
        if (rstd) rstd[r] = rs;
        if (y) {
            for (int64_t j = 0; j < H; ++j) {
                double v = load_elem(x, x_dtype, r * ldx + j);
                y[r * ldy + j] = v * rs * load_elem(w, w_dtype, j);
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* RMSNorm backward.                                                         */
/* Cake commit #5741, Design: Backward -- xhat = x*rstd,                     */
/* dx = rstd*(g*w - mean_j(g*w*xhat)*xhat); dw_j = sum over rows of          */
/* g*x*rstd (the eager form quoted in its Accuracy section).  rstd is the    */
/* forward's stored value, passed in (reading R3).  dW is accumulated over   */
/* rows 0..T-1 in order, in FP64, and written (not added to) into dw.        */
/* ------------------------------------------------------------------------ */

int rno_rmsnorm_bwd(const void* dy, int64_t lddy,
                    const void* x, int64_t ldx, int x_dtype,
                    const void* w, int w_dtype,
                    const double* rstd,
                    int64_t T, int64_t H,
                    double* dx, int64_t lddx,    /* may be NULL */
                    double* dw)                  /* may be NULL; H entries */
{
    if (T < 0 || H <= 0) return 1;
    if (dw)
        for (int64_t j = 0; j < H; ++j) dw[j] = 0.0;
    for (int64_t r = 0; r < T; ++r) {
        double rs = rstd[r];
        if (dx) {
            double dot = 0.0;                    /* sum_j g*w*xhat */
            for (int64_t j = 0; j < H; ++j) {
                double g = load_elem(dy, x_dtype, r * lddy + j);
                double xv = load_elem(x, x_dtype, r * ldx + j);
                double wv = load_elem(w, w_dtype, j);
                dot += g * wv * (xv * rs);
            }
            double c = dot / (double)H;
            for (int64_t j = 0; j < H; ++j) {
                double g = load_elem(dy, x_dtype, r * lddy + j);
                double xv = load_elem(x, x_dtype, r * ldx + j);
                double wv = load_elem(w, w_dtype, j);
                double xhat = xv * rs;
                dx[r * lddx + j] = rs * (g * wv - c * xhat);
            }
        }
        if (dw) {
            for (int64_t j = 0; j < H; ++j) {
                double g = load_elem(dy, x_dtype, r * lddy + j);
                double xv = load_elem(x, x_dtype, r * ldx + j);
                dw[j] += g * xv * rs;
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* 1x128 block quantisation of bf16 normed values to E4M3FN.                 */
/* FlashInfer PR #4480, description (Kernel) and the review thread:          */
/* per row and per 128-column block, scale = amax/448 in fp32; the codes are */
/* the e4m3 rounding of normed/scale; scales stored column-major with the    */
/* row index fastest (readings R5, R6, R7).                                  */
/* ------------------------------------------------------------------------ */

int rno_block_quant_e4m3(const uint16_t* normed, int64_t ldn,
                         int64_t T, int64_t H,
                         float* scale, int64_t scale_ld,
                         uint8_t* codes, int64_t ldq)
{
    if (T < 0 || H <= 0 || H % 128 != 0 || scale_ld < T) return 1;
    int64_t nblk = H / 128;
    for (int64_t r = 0; r < T; ++r) {
        for (int64_t k = 0; k < nblk; ++k) {
            float amax = 0.0f;
            for (int64_t j = 128 * k; j < 128 * k + 128; ++j) {
                float a = (float)fabs(rno_bf16_to_double(normed[r * ldn + j]));
                if (a > amax) amax = a;
            }
            float s = amax / 448.0f;                       /* IEEE fp32 division */
            if (scale) scale[k * scale_ld + r] = s;
            if (codes) {
                for (int64_t j = 128 * k; j < 128 * k + 128; ++j) {
                    float n = (float)rno_bf16_to_double(normed[r * ldn + j]);
                    uint8_t q;
                    if (s == 0.0f)
                        q = 0x00;                          /* all-zero block */
                    else
                        q = rno_float_to_e4m3(n / s);      /* IEEE fp32 division */
                    codes[r * ldq + j] = q;
                }
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Fused residual add + RMSNorm + 1x128 FP8 block quant.                     */
/* FlashInfer PR #4480 description: one pass emits the residual sum (in      */
/* place), the bf16 normed output, the fp32 block scales and the e4m3 codes; */
/* the codes are quantised from the bf16-rounded normed values.  h is the    */
/* bf16 rounding of the exact sum x + r (reading R4); rstd and the normed    */
/* value n = h*rstd*w are FP64, n_bf16 is n rounded once to bf16.            */
/* Any output pointer may be NULL.                                           */
/* ------------------------------------------------------------------------ */

int rno_add_rmsnorm_fp8(const uint16_t* x, int64_t ldx,
                        const uint16_t* res, int64_t ldr,
                        const uint16_t* w,
                        int64_t T, int64_t H, float eps,
                        uint16_t* h_out, int64_t ldh,
                        double* rstd,
                        double* normed, int64_t ldn,
                        uint16_t* normed_bf16, int64_t ldnb,
                        float* scale, int64_t scale_ld,
                        uint8_t* codes, int64_t ldq)
{
    if (T < 0 || H <= 0 || H % 128 != 0 || scale_ld < T) return 1;
    for (int64_t r = 0; r < T; ++r) {
        double ss = 0.0;
        for (int64_t j = 0; j < H; ++j) {
            double s = rno_bf16_to_double(x[r * ldx + j]) + rno_bf16_to_double(res[r * ldr + j]);
            uint16_t hb = rno_double_to_bf16(s);
            if (h_out) h_out[r * ldh + j] = hb;
            double hv = rno_bf16_to_double(hb);
            ss += hv * hv;
        }
        double rs = 1.0 / sqrt(ss / (double)H + (double)eps);
        if (rstd) rstd[r] = rs;
        for (int64_t j = 0; j < H; ++j) {
            double s = rno_bf16_to_double(x[r * ldx + j]) + rno_bf16_to_double(res[r * ldr + j]);
            double hv = rno_bf16_to_double(rno_double_to_bf16(s));
            double n = hv * rs * rno_bf16_to_double(w[j]);
            if (normed) normed[r * ldn + j] = n;
            if (normed_bf16) normed_bf16[r * ldnb + j] = rno_double_to_bf16(n);
        }
        if (scale || codes) {
            /* quantise this row from its own bf16 normed values */
            uint16_t* row = (uint16_t*)malloc((size_t)H * sizeof(uint16_t));
            if (!row) return 2;
            for (int64_t j = 0; j < H; ++j) {
                double s = rno_bf16_to_double(x[r * ldx + j]) + rno_bf16_to_double(res[r * ldr + j]);
                double hv = rno_bf16_to_double(rno_double_to_bf16(s));
                row[j] = rno_double_to_bf16(hv * rs * rno_bf16_to_double(w[j]));
            }
            int rc = rno_block_quant_e4m3(row, H, 1, H,
                                          scale ? scale + r : NULL, scale_ld,
                                          codes ? codes + r * ldq : NULL, ldq);
            free(row);
            if (rc) return rc;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Training pair with a residual stream.                                     */
/* Cake commit #5741, API and Design: the forward optionally takes a         */
/* residual u, returns h_new = bf16(x + u) and normalises it; the backward   */
/* of that forward adds the gradient arriving along the residual stream,     */
/* g_residual, into the dx it returns (dx_total), so both inputs of the add  */
/* receive the same gradient.  Readings R11, R12 (fp32 inputs: the same with */
/* fp32 in place of bf16).                                                   */
/* ------------------------------------------------------------------------ */

/* h = x + u, the exact sum rounded once into x's dtype. */
int rno_residual_add(const void* x, int64_t ldx, const void* u, int64_t ldu, int dtype,
                     int64_t T, int64_t H, void* h, int64_t ldh)
{
    if (T < 0 || H <= 0) return 1;
    for (int64_t r = 0; r < T; ++r) {
        for (int64_t j = 0; j < H; ++j) {
            double s = load_elem(x, dtype, r * ldx + j) + load_elem(u, dtype, r * ldu + j);
            if (dtype == RNO_BF16)
                ((uint16_t*)h)[r * ldh + j] = rno_double_to_bf16(s);
            else
                ((float*)h)[r * ldh + j] = (float)s;      /* one round-to-nearest-even */
        }
    }
    return 0;
}

/* y, rstd of RMSNorm applied to h_new = round(x + u); h_new is written to h
 * (required, x's dtype, row stride ldh). */
int rno_rmsnorm_fwd_residual(const void* x, int64_t ldx, const void* u, int64_t ldu, int x_dtype,
                             const void* w, int w_dtype,
                             int64_t T, int64_t H, float eps,
                             void* h, int64_t ldh,
                             double* y, int64_t ldy,      /* may be NULL */
                             double* rstd)                /* may be NULL */
{
    if (!h) return 1;
    int rc = rno_residual_add(x, ldx, u, ldu, x_dtype, T, H, h, ldh);
    if (rc) return rc;
    return rno_rmsnorm_fwd(h, ldh, x_dtype, w, w_dtype, T, H, eps, y, ldy, rstd);
}

/* dx_total = dx + g_residual (unrounded) and dw, at the forward's h_new and
 * stored rstd. */
int rno_rmsnorm_bwd_residual(const void* dy, int64_t lddy,
                             const void* h, int64_t ldh, int x_dtype,
                             const void* w, int w_dtype,
                             const double* rstd,
                             const void* g_res, int64_t ldgr,
                             int64_t T, int64_t H,
                             double* dx, int64_t lddx,    /* may be NULL */
                             double* dw)                  /* may be NULL */
{
    int rc = rno_rmsnorm_bwd(dy, lddy, h, ldh, x_dtype, w, w_dtype, rstd, T, H, dx, lddx, dw);
    if (rc) return rc;
    if (dx)
        for (int64_t r = 0; r < T; ++r)
            for (int64_t j = 0; j < H; ++j)
                dx[r * lddx + j] += load_elem(g_res, x_dtype, r * ldgr + j);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Per-head RMSNorm (QK-norm).                                               */
/* FlashInfer PR #6332 (QKV projection + QK-RMSNorm + RoPE overlapped with  */
/* the Ulysses head exchange), Description, operator math: an fp32 RMSNorm with */
/* eps 1e-6 over each head's head_dim values, one shared [head_dim] weight   */
/* per Q or K.  Row (t, h) starts at element t*ld_token + h*ld_head of x.    */
/* y is returned unrounded and dense, y[(t*heads + h)*D + j] (reading R13).  */
/* ------------------------------------------------------------------------ */

int rno_rmsnorm_fwd_heads(const void* x, int64_t ld_token, int64_t ld_head, int x_dtype,
                          const void* w, int w_dtype,
                          int64_t T, int64_t heads, int64_t D, float eps,
                          double* y,                   /* may be NULL; [T*heads, D] */
                          double* rstd)                /* may be NULL; [T*heads] */
{
    if (T < 0 || heads <= 0 || D <= 0) return 1;
    size_t es = x_dtype == RNO_BF16 ? 2 : 4;
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t h = 0; h < heads; ++h) {
            int64_t r = t * heads + h;
            const char* row = (const char*)x + (size_t)(t * ld_token + h * ld_head) * es;
            int rc = rno_rmsnorm_fwd(row, D, x_dtype, w, w_dtype, 1, D, eps,
                                     y ? y + r * D : NULL, D, rstd ? rstd + r : NULL);
            if (rc) return rc;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* IEEE binary16 codec: 1 sign, 5 exponent (bias 15), 10 fraction bits;      */
/* largest finite 65504; subnormals k * 2^-24.                               */
/* ------------------------------------------------------------------------ */

double rno_f16_to_double(uint16_t b)
{
    int neg = (b >> 15) & 1;
    int ex = (b >> 10) & 0x1F;
    int m = b & 0x3FF;
    double v;
    if (ex == 0x1F) return m ? NAN : (neg ? -INFINITY : INFINITY);
    if (ex == 0)
        v = ldexp((double)m, -24);
    else
        v = ldexp(1.0 + m / 1024.0, ex - 15);
    return neg ? -v : v;
}

/* Round a double to the nearest binary16 value, ties to even, in one
 * rounding; at or beyond the overflow threshold (65520) the result is +-inf. */
uint16_t rno_double_to_f16(double v)
{
    if (isnan(v)) return 0x7E00;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0) return sign;
    int e;
    (void)frexp(a, &e);               /* a in [2^(e-1), 2^e) */
    int qexp = e - 11;                /* quantum of an 11-significant-bit value */
    if (qexp < -24) qexp = -24;       /* subnormal quantum */
    double quantum = ldexp(1.0, qexp);
    double k = a / quantum;
    double fl = floor(k);
    double frac = k - fl;
    if (frac > 0.5 || (frac == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;
    double r = fl * quantum;
    if (r >= 65536.0) return (uint16_t)(sign | 0x7C00);
    if (r < ldexp(1.0, -14))          /* subnormal: r = m * 2^-24 */
        return (uint16_t)(sign | (uint16_t)(r / ldexp(1.0, -24)));
    int er;
    double f = frexp(r, &er);         /* r = (2f) * 2^(er-1), 2f in [1,2) */
    int m = (int)((2.0 * f - 1.0) * 1024.0);
    return (uint16_t)(sign | ((er - 1 + 15) << 10) | m);
}

/* ------------------------------------------------------------------------ */
/* E5M2 codec: 1 sign, 5 exponent (bias 15), 2 mantissa bits; S.11111.00 is  */
/* infinity, S.11111.xx (xx != 0) NaN; largest finite 1.75 * 2^15 = 57344;   */
/* subnormals k * 2^-16.                                                     */
/* ------------------------------------------------------------------------ */

double rno_e5m2_to_double(uint8_t c)
{
    int neg = (c >> 7) & 1;
    int ex = (c >> 2) & 0x1F;
    int m = c & 3;
    double v;
    if (ex == 0x1F) return m ? NAN : (neg ? -INFINITY : INFINITY);
    if (ex == 0)
        v = ldexp((double)m, -16);
    else
        v = ldexp(1.0 + m / 4.0, ex - 15);
    return neg ? -v : v;
}

/* Round a binary32 value to E5M2, nearest-even, saturating to +-57344 (also
 * for infinities); NaN gives 0x7F. */
uint8_t rno_float_to_e5m2(float v)
{
    if (isnan(v)) return 0x7F;
    uint8_t sign = signbit(v) ? 0x80 : 0;
    double a = fabs((double)v);
    if (a >= 57344.0) return (uint8_t)(sign | 0x7B);
    int qexp;
    if (a < ldexp(1.0, -14)) {
        qexp = -16;                                /* subnormal spacing */
    } else {
        int e;
        (void)frexp(a, &e);                        /* a in [2^(e-1), 2^e) */
        qexp = e - 3;                              /* 3 significant bits */
    }
    double quantum = ldexp(1.0, qexp);
    double k = a / quantum;
    double fl = floor(k);
    double frac = k - fl;
    if (frac > 0.5 || (frac == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;
    double r = fl * quantum;
    if (r > 57344.0) r = 57344.0;
    if (r == 0.0) return sign;
    if (r < ldexp(1.0, -14)) return (uint8_t)(sign | (uint8_t)(r / ldexp(1.0, -16)));
    int er;
    double f = frexp(r, &er);
    int m = (int)((2.0 * f - 1.0) * 4.0);
    return (uint8_t)(sign | ((er - 1 + 15) << 2) | m);
}

/* ------------------------------------------------------------------------ */
/* Producer variants (reading R14): bf16 or fp16 rows, e4m3 or e5m2 codes,   */
/* a dynamic scale per 1x128 block or one given per-tensor scale.            */
/* FlashInfer PR #4480: description (the block-scaled sibling of the         */
/* per-tensor FusedAddRMSNormQuant), its test matrix over fp16 and bf16      */
/* inputs, and the review thread (the bound 448 tied to the output type,     */
/* i.e. 57344 for e5m2).                                                     */
/* ------------------------------------------------------------------------ */

static double lp_decode(uint16_t b, int dtype)
{
    return dtype == RNO_F16 ? rno_f16_to_double(b) : rno_bf16_to_double(b);
}

static uint16_t lp_encode(double v, int dtype)
{
    return dtype == RNO_F16 ? rno_double_to_f16(v) : rno_double_to_bf16(v);
}

static uint8_t fp8_encode(float v, int fmt)
{
    return fmt == RNO_E5M2 ? rno_float_to_e5m2(v) : rno_float_to_e4m3(v);
}

static float fp8_max(int fmt) { return fmt == RNO_E5M2 ? 57344.0f : 448.0f; }

/* Codes (and, with block scales, the scales) of low-precision normed values.
 * tensor_scale > 0: one given scale for every element, no scales written;
 * tensor_scale == 0: per row and 128-column block, s = amax / MAX. */
int rno_quant_lp(const uint16_t* normed, int64_t ldn, int dtype, int fmt,
                 int64_t T, int64_t H, float tensor_scale,
                 float* scale, int64_t scale_ld,
                 uint8_t* codes, int64_t ldq)
{
    if (T < 0 || H <= 0 || H % 128 != 0 || (tensor_scale == 0.0f && scale && scale_ld < T)) return 1;
    if (tensor_scale < 0.0f || isnan(tensor_scale) || isinf(tensor_scale)) return 1;
    float mx = fp8_max(fmt);
    for (int64_t r = 0; r < T; ++r) {
        for (int64_t k = 0; k < H / 128; ++k) {
            float s = tensor_scale;
            if (tensor_scale == 0.0f) {
                float amax = 0.0f;
                for (int64_t j = 128 * k; j < 128 * k + 128; ++j) {
                    float a = (float)fabs(lp_decode(normed[r * ldn + j], dtype));
                    if (a > amax) amax = a;
                }
                s = amax / mx;                              /* IEEE fp32 division */
                if (scale) scale[k * scale_ld + r] = s;
            }
            if (!codes) continue;
            for (int64_t j = 128 * k; j < 128 * k + 128; ++j) {
                float n = (float)lp_decode(normed[r * ldn + j], dtype);
                codes[r * ldq + j] = (s == 0.0f) ? 0x00 : fp8_encode(n / s, fmt);   /* IEEE fp32 division */
            }
        }
    }
    return 0;
}

/* The producer: h = round_lp(x + res) (written to h_out), rstd from h,
 * n = h*rstd*w (FP64, unrounded to `normed`, rounded once to the row dtype
 * in `normed_lp`), then rno_quant_lp of normed_lp.  Any output may be NULL. */
int rno_add_rmsnorm_quant(const uint16_t* x, int64_t ldx, const uint16_t* res, int64_t ldr,
                          const uint16_t* w, int dtype, int fmt,
                          int64_t T, int64_t H, float eps, float tensor_scale,
                          uint16_t* h_out, int64_t ldh, double* rstd,
                          double* normed, int64_t ldn, uint16_t* normed_lp, int64_t ldnl,
                          float* scale, int64_t scale_ld, uint8_t* codes, int64_t ldq)
{
    if (T < 0 || H <= 0 || H % 128 != 0) return 1;
    if (dtype != RNO_BF16 && dtype != RNO_F16) return 1;
    uint16_t* row = (uint16_t*)malloc((size_t)H * sizeof(uint16_t));
    if (!row) return 2;
    for (int64_t r = 0; r < T; ++r) {
        double ss = 0.0;
        for (int64_t j = 0; j < H; ++j) {
            uint16_t hb = lp_encode(lp_decode(x[r * ldx + j], dtype) + lp_decode(res[r * ldr + j], dtype), dtype);
            if (h_out) h_out[r * ldh + j] = hb;
            double hv = lp_decode(hb, dtype);
            ss += hv * hv;
        }
        double rs = 1.0 / sqrt(ss / (double)H + (double)eps);
        if (rstd) rstd[r] = rs;
        for (int64_t j = 0; j < H; ++j) {
            double hv = lp_decode(lp_encode(lp_decode(x[r * ldx + j], dtype) + lp_decode(res[r * ldr + j], dtype),
                                            dtype), dtype);
            double n = hv * rs * lp_decode(w[j], dtype);
            if (normed) normed[r * ldn + j] = n;
            row[j] = lp_encode(n, dtype);
            if (normed_lp) normed_lp[r * ldnl + j] = row[j];
        }
        if (scale || codes) {
            int rc = rno_quant_lp(row, H, dtype, fmt, 1, H, tensor_scale,
                                  scale ? scale + r : NULL, scale_ld, codes ? codes + r * ldq : NULL, ldq);
            if (rc) { free(row); return rc; }
        }
    }
    free(row);
    return 0;
}
