/*
 * mp3d_oracle.c -- plain, slow CPU oracle for 3-D max pooling over NCDHW
 * tensors: the forward window maximum with its per-plane argmax, and the
 * backward pass that routes each output gradient to that argmax.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header, table or
 * helper with the HIP library; the only thing both sides see is the seeded
 * input tensors.
 *
 * What is computed, and where it is defined:
 *  - Fixed windows ("Struct Maxpool3dForward", teenygrad API docs, the
 *    description under the struct: no padding, and the output extent on each
 *    axis is (X - K) / STRIDE + 1 with integer division).  Window o on an
 *    axis covers [o*stride, o*stride + K).
 *  - Adaptive windows ("Add adaptive_max_pool3d_backward Moore Threads
 *    specialized operator", FlagGems-Experimental PR #308, Summary).  The
 *    page says that when every axis divides evenly the windows tile the
 *    input disjointly and otherwise they overlap, but it prints no bound
 *    formula.  Reading taken: window o of O over an axis of length X covers
 *    [floor(o*X/O), ceil((o+1)*X/O)), which tiles [0,X) into blocks of X/O
 *    when O divides X and overlaps otherwise, as the page describes.
 *  - Backward (same PR #308 page, Summary): every output gradient is sent to
 *    the input position of its window's argmax; where windows overlap,
 *    several outputs may land on one input and their contributions add.
 *    Accumulation is in binary32 starting from +0, in ascending output
 *    order, then rounded once to the storage type.  Alongside, the exact
 *    binary64 sum, the sum of magnitudes and the contribution count per
 *    input are returned so that tests can bound any other summation order.
 *
 * Readings where the pages are silent:
 *  - Scan order and ties: a window is scanned d, then h, then w, ascending;
 *    an element replaces the running best only if it is strictly greater,
 *    so among equal maxima the first in scan order wins.  -0 and +0 compare
 *    equal (IEEE), so they tie.
 *  - NaN ranks above every number: a NaN replaces a non-NaN best, and the
 *    first NaN in scan order wins among NaNs.  y carries that element's bits.
 *  - The argmax is stored as int32 (d*H + h)*W + w, flat within one D*H*W
 *    plane.
 *  - idx values outside [0, D*H*W) are ignored by the backward.
 *
 * Floating point: comparisons are made on exact binary64 widenings of the
 * stored values.  The 16-bit formats are decoded and rounded here from
 * their IEEE 754 definitions (round to nearest, ties to even), without any
 * library conversion routine.  Build with -ffp-contract=off and without
 * -ffast-math.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

enum { ORACLE_F32 = 0, ORACLE_F16 = 1, ORACLE_BF16 = 2, ORACLE_F64 = 3 };

/* ---------------------------------------------------------------------- */
/* 16-bit formats, from the IEEE 754 binary16 and the bfloat16 layouts.    */
/* ---------------------------------------------------------------------- */

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                 /* zero or subnormal */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);     /* (1.m) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16: the upper half of a binary32 (8 exponent bits, 7 fraction). */
double oracle_bf16_to_f64(uint16_t b)
{
    int sign = (b >> 15) & 1;
    int e = (b >> 7) & 0xff;
    int m = b & 0x7f;
    double v;
    if (e == 0)
        v = ldexp((double)m, -133);                /* zero or subnormal */
    else if (e == 255)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + m), e - 134);     /* (1.m) * 2^(e-127) */
    return sign ? -v : v;
}

static uint32_t f32_bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}

/* Round a binary32 to binary16, nearest-even.  NaN keeps its sign and the
 * top fraction bits and is made quiet. */
uint16_t oracle_f32_to_f16(float f)
{
    uint32_t u = f32_bits(f);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000);
    double a = fabs((double)f);
    if (isnan(f))
        return (uint16_t)(sign | 0x7e00 | ((u & 0x7fffff) >> 13));
    if (a == 0.0)
        return sign;
    if (isinf(f))
        return (uint16_t)(sign | 0x7c00);
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: units of 2^-24; rint rounds ties to even */
        double q = rint(ldexp(a, 24));
        return (uint16_t)(sign | (uint16_t)q);     /* q == 1024 is 2^-14 */
    }
    int ex;
    frexp(a, &ex);                                 /* a in [2^(ex-1), 2^ex) */
    int E = ex - 1;
    double mant = rint(ldexp(a, 10 - E));          /* in [1024, 2048] */
    if (mant == 2048.0) { mant = 1024.0; E += 1; }
    if (E + 15 >= 31)
        return (uint16_t)(sign | 0x7c00);          /* overflow to infinity */
    return (uint16_t)(sign | ((E + 15) << 10) | ((int)mant - 1024));
}

/* Round a binary32 to bfloat16, nearest-even.  NaN keeps its sign and the
 * top fraction bits and is made quiet. */
uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t u = f32_bits(f);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000);
    double a = fabs((double)f);
    if (isnan(f))
        return (uint16_t)(sign | 0x7fc0 | ((u & 0x7fffff) >> 16));
    if (a == 0.0)
        return sign;
    if (isinf(f))
        return (uint16_t)(sign | 0x7f80);
    if (a < ldexp(1.0, -126)) {
        double q = rint(ldexp(a, 133));            /* units of 2^-133 */
        return (uint16_t)(sign | (uint16_t)q);     /* q == 128 is 2^-126 */
    }
    int ex;
    frexp(a, &ex);
    int E = ex - 1;
    double mant = rint(ldexp(a, 7 - E));           /* in [128, 256] */
    if (mant == 256.0) { mant = 128.0; E += 1; }
    if (E + 127 >= 255)
        return (uint16_t)(sign | 0x7f80);
    return (uint16_t)(sign | ((E + 127) << 7) | ((int)mant - 128));
}

/* Value of element i of a buffer of the given storage type, widened
 * exactly to binary64. */
static double load_f64(const void *buf, int dtype, int64_t i)
{
    if (dtype == ORACLE_F64)
        return ((const double *)buf)[i];
    if (dtype == ORACLE_F32)
        return (double)((const float *)buf)[i];
    if (dtype == ORACLE_F16)
        return oracle_f16_to_f64(((const uint16_t *)buf)[i]);
    return oracle_bf16_to_f64(((const uint16_t *)buf)[i]);
}

static int dtype_size(int dtype)
{
    return dtype == ORACLE_F64 ? 8 : dtype == ORACLE_F32 ? 4 : 2;
}

/* ---------------------------------------------------------------------- */
/* Windows                                                                 */
/* ---------------------------------------------------------------------- */

/* Bounds [*start, *end) of window o on one axis of length X split into O
 * windows.  k > 0 selects fixed windows of width k and stride s (the
 * teenygrad forward's rule); k == 0 selects adaptive windows. */
void oracle_window(int64_t X, int64_t O, int64_t k, int64_t s, int64_t o,
                   int64_t *start, int64_t *end)
{
    if (k > 0) {
        *start = o * s;
        *end = o * s + k;
    } else {
        *start = (o * X) / O;                      /* floor(o*X/O)     */
        *end = ((o + 1) * X + O - 1) / O;          /* ceil((o+1)*X/O)  */
    }
}

/* Output extent of a fixed-window axis, or -1 if the window does not fit. */
int64_t oracle_fixed_out(int64_t X, int64_t k, int64_t s)
{
    if (k <= 0 || s <= 0 || X < k)
        return -1;
    return (X - k) / s + 1;
}

/* ---------------------------------------------------------------------- */
/* Forward                                                                 */
/* ---------------------------------------------------------------------- */

/* x: P planes of D*H*W elements of `dtype`; y: P planes of OD*OH*OW of
 * `dtype`; idx: P planes of OD*OH*OW int32.  k[3]/s[3] per axis (d, h, w);
 * k[a] == 0 means the axis uses adaptive windows and O[a] is taken as
 * given.  For fixed axes O[a] must equal (X - k)/s + 1. */
void oracle_forward(const void *x, void *y, int32_t *idx, int dtype,
                    int64_t P, int64_t D, int64_t H, int64_t W,
                    int64_t OD, int64_t OH, int64_t OW,
                    const int64_t *k, const int64_t *s)
{
    const int64_t plane_in = D * H * W;
    const int64_t plane_out = OD * OH * OW;
    const int es = dtype_size(dtype);
    for (int64_t p = 0; p < P; ++p) {
        for (int64_t od = 0; od < OD; ++od) {
            int64_t d0, d1;
            oracle_window(D, OD, k[0], s[0], od, &d0, &d1);
            for (int64_t oh = 0; oh < OH; ++oh) {
                int64_t h0, h1;
                oracle_window(H, OH, k[1], s[1], oh, &h0, &h1);
                for (int64_t ow = 0; ow < OW; ++ow) {
                    int64_t w0, w1;
                    oracle_window(W, OW, k[2], s[2], ow, &w0, &w1);
                    int64_t best_i = -1;
                    double best = 0.0;
                    for (int64_t d = d0; d < d1; ++d)
                        for (int64_t h = h0; h < h1; ++h)
                            for (int64_t w = w0; w < w1; ++w) {
                                int64_t i = (d * H + h) * W + w;
                                double v = load_f64(x, dtype, p * plane_in + i);
                                int take;
                                if (best_i < 0)
                                    take = 1;
                                else if (v > best)
                                    take = 1;
                                else if (isnan(v) && !isnan(best))
                                    take = 1;
                                else
                                    take = 0;
                                if (take) {
                                    best = v;
                                    best_i = i;
                                }
                            }
                    int64_t o = p * plane_out + (od * OH + oh) * OW + ow;
                    memcpy((char *)y + o * es,
                           (const char *)x + (p * plane_in + best_i) * es, es);
                    idx[o] = (int32_t)best_i;
                }
            }
        }
    }
}

/* ---------------------------------------------------------------------- */
/* Forward with padding and dilation                                       */
/* ---------------------------------------------------------------------- */

/* The pages define fixed windows without padding only.  Reading taken for
 * the wider surface: window o takes the k taps o*s - pad + j*dil, j = 0..k-1
 * (they span (k-1)*dil + 1 positions, the effective kernel of the FlagGems
 * conv_transpose2d PR page, Implementation); taps outside [0, X) are
 * padding and are skipped.  Output extent: floor mode counts the spans
 * that fit X + 2*pad; ceil mode rounds the count up and then drops a last
 * window that would start at or beyond X + pad.  -1 if no span fits. */
int64_t oracle_fixed_out_ex(int64_t X, int64_t k, int64_t s, int64_t pad, int64_t dil,
                            int ceil_mode)
{
    if (k <= 0 || s <= 0 || pad < 0 || dil <= 0)
        return -1;
    int64_t span = (k - 1) * dil + 1;
    int64_t room = X + 2 * pad - span;
    if (room < 0)
        return -1;
    int64_t n = room / s;
    if (ceil_mode && n * s < room)
        n += 1;                                    /* one more, partial, window */
    int64_t O = n + 1;
    if (ceil_mode && (O - 1) * s >= X + pad)
        O -= 1;
    return O;
}

/* Position of tap j of window o on one axis, or -1 if it is padding or past
 * the window.  k == 0: adaptive windows (contiguous, no padding). */
static int64_t tap_position(int64_t X, int64_t O, int64_t k, int64_t s, int64_t pad,
                            int64_t dil, int64_t o, int64_t j)
{
    int64_t q;
    if (k > 0) {
        if (j >= k)
            return -1;
        q = o * s - pad + j * dil;
    } else {
        int64_t a, b;
        oracle_window(X, O, 0, 0, o, &a, &b);
        if (j >= b - a)
            return -1;
        q = a + j;
    }
    return (q >= 0 && q < X) ? q : -1;
}

/* Forward over the taps of each window, in d, h, w scan order of the tap
 * numbers (the same order as the positions, which grow with j).  idx is
 * int64; a window with no tap inside the input gives y = -inf, idx = -1.
 * k/s/pad/dil are arrays of 3; k[a] == 0 selects adaptive windows. */
void oracle_forward_ex(const void *x, void *y, int64_t *idx, int dtype,
                       int64_t P, int64_t D, int64_t H, int64_t W,
                       int64_t OD, int64_t OH, int64_t OW,
                       const int64_t *k, const int64_t *s,
                       const int64_t *pad, const int64_t *dil)
{
    const int64_t plane_in = D * H * W;
    const int64_t plane_out = OD * OH * OW;
    const int es = dtype_size(dtype);
    /* most taps any window can have on an axis */
    int64_t nt[3];
    const int64_t X[3] = {D, H, W};
    const int64_t O[3] = {OD, OH, OW};
    for (int a = 0; a < 3; ++a) {
        if (k[a] > 0) {
            nt[a] = k[a];
        } else {
            nt[a] = 0;
            for (int64_t o = 0; o < O[a]; ++o) {
                int64_t lo, hi;
                oracle_window(X[a], O[a], 0, 0, o, &lo, &hi);
                if (hi - lo > nt[a])
                    nt[a] = hi - lo;
            }
        }
    }
    for (int64_t p = 0; p < P; ++p)
        for (int64_t od = 0; od < OD; ++od)
            for (int64_t oh = 0; oh < OH; ++oh)
                for (int64_t ow = 0; ow < OW; ++ow) {
                    int64_t best_i = -1;
                    double best = 0.0;
                    for (int64_t jd = 0; jd < nt[0]; ++jd) {
                        int64_t d = tap_position(D, OD, k[0], s[0], pad[0], dil[0], od, jd);
                        if (d < 0)
                            continue;
                        for (int64_t jh = 0; jh < nt[1]; ++jh) {
                            int64_t h = tap_position(H, OH, k[1], s[1], pad[1], dil[1], oh, jh);
                            if (h < 0)
                                continue;
                            for (int64_t jw = 0; jw < nt[2]; ++jw) {
                                int64_t w = tap_position(W, OW, k[2], s[2], pad[2], dil[2], ow, jw);
                                if (w < 0)
                                    continue;
                                int64_t i = (d * H + h) * W + w;
                                double v = load_f64(x, dtype, p * plane_in + i);
                                int take = best_i < 0 || v > best || (isnan(v) && !isnan(best));
                                if (take) {
                                    best = v;
                                    best_i = i;
                                }
                            }
                        }
                    }
                    int64_t o = p * plane_out + (od * OH + oh) * OW + ow;
                    if (best_i >= 0) {
                        memcpy((char *)y + o * es,
                               (const char *)x + (p * plane_in + best_i) * es, es);
                    } else if (dtype == ORACLE_F64) {
                        ((double *)y)[o] = -INFINITY;
                    } else if (dtype == ORACLE_F32) {
                        ((float *)y)[o] = -INFINITY;
                    } else {
                        ((uint16_t *)y)[o] = dtype == ORACLE_F16 ? 0xfc00 : 0xff80;
                    }
                    idx[o] = best_i;
                }
}

/* The argmax recovered from the forward's output, for a backward that is
 * given x and y instead of idx (the teenygrad backward receives the
 * forward's inputs and output, "Struct Maxpool3dForward", RuntimeOp).
 * Reading taken: the first tap of window o in d, h, w scan order whose
 * element equals y[o] -- equal as numbers, so -0 matches +0 -- or, when
 * y[o] is a NaN, the first NaN tap; -1 when no tap matches.  Geometry as in
 * oracle_forward_ex. */
void oracle_argmax_from_output(const void *x, const void *y, int64_t *idx, int dtype,
                               int64_t P, int64_t D, int64_t H, int64_t W,
                               int64_t OD, int64_t OH, int64_t OW,
                               const int64_t *k, const int64_t *s,
                               const int64_t *pad, const int64_t *dil)
{
    const int64_t plane_in = D * H * W;
    const int64_t plane_out = OD * OH * OW;
    const int64_t X[3] = {D, H, W};
    const int64_t O[3] = {OD, OH, OW};
    int64_t nt[3];
    for (int a = 0; a < 3; ++a) {
        if (k[a] > 0) {
            nt[a] = k[a];
        } else {
            nt[a] = 0;
            for (int64_t o = 0; o < O[a]; ++o) {
                int64_t lo, hi;
                oracle_window(X[a], O[a], 0, 0, o, &lo, &hi);
                if (hi - lo > nt[a])
                    nt[a] = hi - lo;
            }
        }
    }
    for (int64_t p = 0; p < P; ++p)
        for (int64_t od = 0; od < OD; ++od)
            for (int64_t oh = 0; oh < OH; ++oh)
                for (int64_t ow = 0; ow < OW; ++ow) {
                    int64_t o = p * plane_out + (od * OH + oh) * OW + ow;
                    double want = load_f64(y, dtype, o);
                    int64_t found = -1;
                    for (int64_t jd = 0; jd < nt[0] && found < 0; ++jd) {
                        int64_t d = tap_position(D, OD, k[0], s[0], pad[0], dil[0], od, jd);
                        if (d < 0)
                            continue;
                        for (int64_t jh = 0; jh < nt[1] && found < 0; ++jh) {
                            int64_t h = tap_position(H, OH, k[1], s[1], pad[1], dil[1], oh, jh);
                            if (h < 0)
                                continue;
                            for (int64_t jw = 0; jw < nt[2] && found < 0; ++jw) {
                                int64_t w = tap_position(W, OW, k[2], s[2], pad[2], dil[2], ow, jw);
                                if (w < 0)
                                    continue;
                                int64_t i = (d * H + h) * W + w;
                                double v = load_f64(x, dtype, p * plane_in + i);
                                if (isnan(want) ? isnan(v) : v == want)
                                    found = i;
                            }
                        }
                    }
                    idx[o] = found;
                }
}

/* ---------------------------------------------------------------------- */
/* Backward                                                                */
/* ---------------------------------------------------------------------- */

/* gy, idx: P planes of OD*OH*OW; gx: P planes of D*H*W, all of `dtype`
 * except idx (int32).  acc32 is a caller-provided binary32 scratch of
 * P*D*H*W that holds the accumulator before rounding on return.  ref64,
 * abs64 (binary64) and count (int32) are optional per-input side outputs
 * (NULL to skip): the binary64 sum, the sum of magnitudes and the number of
 * contributions.  float64 gradients (PR #308 page, Testing, leaves float64
 * to a generic path; reading taken: the same ordered sum, in binary64) are
 * added in binary64 from +0 in ascending output order straight into gx;
 * acc32 then holds their binary32 roundings. */
void oracle_backward(const void *gy, const int32_t *idx, void *gx, int dtype,
                     int64_t P, int64_t D, int64_t H, int64_t W,
                     int64_t OD, int64_t OH, int64_t OW,
                     float *acc32, double *ref64, double *abs64,
                     int32_t *count)
{
    const int64_t plane_in = D * H * W;
    const int64_t plane_out = OD * OH * OW;
    const int64_t n = P * plane_in;
    for (int64_t t = 0; t < n; ++t) {
        acc32[t] = 0.0f;
        if (dtype == ORACLE_F64) ((double *)gx)[t] = 0.0;
        if (ref64) ref64[t] = 0.0;
        if (abs64) abs64[t] = 0.0;
        if (count) count[t] = 0;
    }
    for (int64_t p = 0; p < P; ++p) {
        for (int64_t o = 0; o < plane_out; ++o) {
            int64_t i = idx[p * plane_out + o];
            if (i < 0 || i >= plane_in)
                continue;
            double gv = load_f64(gy, dtype, p * plane_out + o);
            int64_t t = p * plane_in + i;
            if (dtype == ORACLE_F64) {
                double *g64 = (double *)gx;
                g64[t] = g64[t] + gv;              /* one binary64 add, RNE */
            } else {
                float g = (float)gv;               /* exact: gy is <= 32 bit */
                float sum = acc32[t] + g;          /* one binary32 add, RNE */
                acc32[t] = sum;
            }
            if (ref64) ref64[t] += gv;
            if (abs64) abs64[t] += fabs(gv);
            if (count) count[t] += 1;
        }
    }
    for (int64_t t = 0; t < n; ++t) {
        if (dtype == ORACLE_F64)
            acc32[t] = (float)((double *)gx)[t];
        else if (dtype == ORACLE_F32)
            ((float *)gx)[t] = acc32[t];
        else if (dtype == ORACLE_F16)
            ((uint16_t *)gx)[t] = oracle_f32_to_f16(acc32[t]);
        else
            ((uint16_t *)gx)[t] = oracle_f32_to_bf16(acc32[t]);
    }
}

/* ---------------------------------------------------------------------- */
/* Array forms of the conversions, for exhaustive checks.                  */
/* ---------------------------------------------------------------------- */

void oracle_widen_array(const void *src, int dtype, int64_t n, double *dst)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = load_f64(src, dtype, i);
}

void oracle_round_array(const float *src, int dtype, int64_t n, uint16_t *dst)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = dtype == ORACLE_F16 ? oracle_f32_to_f16(src[i])
                                     : oracle_f32_to_bf16(src[i]);
}
