/*
 * kvq_oracle.c -- plain, slow, single-threaded fp64 CPU oracle for the fused
 * per-vector KV-cache quantizer (sign-randomized Walsh-Hadamard rotation with a
 * per-(head, channel) smooth scale, per-group abs-max int4 with nibble packing,
 * its inverse, and the product-VQ encode/decode variant).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library's product path includes,
 * links or calls this file.  It is used by the test-suite, by the smoke check
 * and by the CPU-baseline leg of the benchmark, and it shares no code, header,
 * table or constant with the HIP kernels.
 *
 * Every value is computed in IEEE binary64.  The Hadamard product is the dense
 * O(D^2) definition, not a butterfly; the binary16 codec is written from the
 * IEEE 754 binary16 format definition; rounding to integers uses nearbyint()
 * under the default round-to-nearest-even mode.  Built with
 * -ffp-contract=off so that no multiply-add is fused behind our back.
 *
 * Sources (cited by page title and section):
 *  [VQ-blog]  "The Kernel That Finally Did Something -- And Didn't Quite Agree
 *             With Itself" (VeloxQuant-MLX blog, tag vecinfer), sections
 *             "What VecInfer does" and "The numbers".
 *  [README]   VeloxQuant-MLX 0.52.0 package description, section
 *             "Metal kernels" (quantize_vq: nearest centroid, argmin kept in
 *             registers).
 *  [ABSTRACT] "When Quantization Is Free: An int4 KV Cache That Outruns fp16
 *             on Apple Silicon" (arXiv 2605.05699), abstract.
 *  [GIST]     gist.science explanation of arXiv 2605.05699, "Technische
 *             Samenvatting" -> "Methodologie" sections 1 (sign-randomized
 *             transform), 2 (fused kernel step list), 3 (per-channel plus
 *             per-group scaling).
 *  [POLAR]    PolarQuant / block-FP4 abstract (Apple M5 Max): names block-scaled
 *             E2M1 FP4 as a KV-cache format; the format is taken as the OCP
 *             Microscaling (MX) v1.0 MXFP4 definition (32-element blocks,
 *             E8M0 power-of-two scale, E2M1 elements).
 *  [SCALAR-ATTEND] VeloxQuant-MLX 0.52.0 package description, section
 *             "Fused group-affine (KIVI-style) attention": single-query decode
 *             attention straight from group-quantized codes, online softmax
 *             accumulated in fp32, no dequantized cache in memory.
 *
 * Readings of points the pages leave open (each one is listed, with its
 * reasoning, in the design notes of the repository):
 *  - lambda multiplies x before the rotation, and divides after the inverse
 *    rotation ("smooth scale ... then rotation"; "unscale" last) [VQ-blog].
 *  - Hadamard in Sylvester (natural) order, H[i][j] = (-1)^popcount(i & j),
 *    normalised by D^-1/2 in both directions (the transform is described as
 *    unitary) [GIST s.1].
 *  - groups are contiguous runs of G rotated coordinates [GIST s.2, s.3].
 *  - symmetric int4: scale = amax / 7 stored as binary16 (round to nearest
 *    even), codes = clamp(round_half_even(y / stored_scale), -7, 7); an
 *    all-zero group gets scale 0 and codes 0 [ABSTRACT; GIST s.2].
 *  - nibble format: two's complement 4-bit, element 2k in the low nibble of
 *    byte k [GIST s.2 "two int4 values in one byte"].
 *  - VQ: contiguous sub-vectors, squared Euclidean distance on the unrounded
 *    rotated key, lowest index on ties [README "Metal kernels"; VQ-blog].
 *  - SRFT (the Fourier alternative to the Hadamard rotation) [GIST s.1, s.2]:
 *    unitary DFT of s * lambda * x, real-packed as [X_0, X_{D/2}, sqrt2 Re X_1,
 *    sqrt2 Im X_1, ...], an orthonormal map; D any even number.
 *  - codebook training is Lloyd's k-means on the rotated sub-vectors of
 *    synthetic samples: assign each to its nearest centroid (the encode
 *    above), then move each centroid to the mean of its samples; a centroid
 *    with no samples stays where it was; the result is stored as binary16
 *    like the codebook it replaces [VQ-blog, calibration caveat].
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary16 codec, from the format definition:                       */
/*   1 sign bit, 5 exponent bits (bias 15), 10 fraction bits;                 */
/*   exponent 0 = subnormal (fraction * 2^-24), exponent 31 = inf / NaN.      */
/* ------------------------------------------------------------------------ */

double kvqo_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24);
    } else if (e == 31) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp(1.0 + (double)f / 1024.0, e - 15);
    }
    return sign ? -v : v;
}

/* Round a binary64 value to the nearest binary16, ties to even. */
uint16_t kvqo_f64_to_f16(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v)) return (uint16_t)(sign | 0x7e00);
    /* 65504 is the largest finite value; half-way to 2^16 is 65520, and the
       tie goes to the even neighbour 2^16, which overflows to infinity. */
    if (a >= 65520.0) return (uint16_t)(sign | 0x7c00);
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: integer multiple of 2^-24 (a carry to 1024 lands
           exactly on the smallest normal encoding 0x0400) */
        double n = nearbyint(ldexp(a, 24));
        return (uint16_t)(sign | (uint16_t)n);
    }
    int k;
    double m = frexp(a, &k);      /* a = m * 2^k, m in [0.5, 1) */
    int E = k - 1;                /* a = (2m) * 2^E, 2m in [1, 2) */
    double n = nearbyint((2.0 * m - 1.0) * 1024.0);
    if (n == 1024.0) { n = 0.0; E += 1; }
    if (E + 15 >= 31) return (uint16_t)(sign | 0x7c00);
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)n);
}

void kvqo_f16_decode(int64_t n, const uint16_t* h, double* out)
{
    for (int64_t i = 0; i < n; i++) out[i] = kvqo_f16_to_f64(h[i]);
}

void kvqo_f16_encode(int64_t n, const double* v, uint16_t* out)
{
    for (int64_t i = 0; i < n; i++) out[i] = kvqo_f64_to_f16(v[i]);
}

/* ------------------------------------------------------------------------ */
/* Walsh-Hadamard matrix, Sylvester order                                      */
/* ------------------------------------------------------------------------ */

/* Entry (i, j) of the unnormalised D x D Sylvester Hadamard matrix. */
int kvqo_hadamard_entry(int i, int j)
{
    return (__builtin_popcount((unsigned)(i & j)) & 1) ? -1 : 1;
}

static int is_pow2(int d) { return d > 0 && (d & (d - 1)) == 0; }

/* Rotation of one vector [GIST s.1; VQ-blog "What VecInfer does"]:
     y_i = D^-1/2 * sum_j H[i][j] * s_j * lambda_j * x_j
   x is binary16 (decoded exactly), lambda binary32, s in {-1, +1}. */
static void rotate_one(int D, const uint16_t* x, const float* lam,
                       const int8_t* s, double* v, double* y)
{
    for (int j = 0; j < D; j++)
        v[j] = (double)s[j] * (double)lam[j] * kvqo_f16_to_f64(x[j]);
    double norm = 1.0 / sqrt((double)D);
    for (int i = 0; i < D; i++) {
        double acc = 0.0;
        for (int j = 0; j < D; j++) acc += kvqo_hadamard_entry(i, j) * v[j];
        y[i] = acc * norm;
    }
}

/* Inverse rotation [VQ-blog "The kernel toggle": inverse transform, then
   unscale]:  xhat_j = (s_j / lambda_j) * D^-1/2 * sum_i H[i][j] * yhat_i.
   H is symmetric and H*H = D*I, so this inverts rotate_one exactly. */
static void unrotate_one(int D, const double* yhat, const float* lam,
                         const int8_t* s, double* xhat)
{
    double norm = 1.0 / sqrt((double)D);
    for (int j = 0; j < D; j++) {
        double acc = 0.0;
        for (int i = 0; i < D; i++) acc += kvqo_hadamard_entry(i, j) * yhat[i];
        xhat[j] = ((double)s[j] / (double)lam[j]) * (acc * norm);
    }
}

/* n vectors of length D; x [n, D] binary16 bits; lam [n, D] (the lambda row
   that belongs to each vector's layer and head); s [D]; y [n, D]. */
int kvqo_rotate_rows(int64_t n, int D, const uint16_t* x, const float* lam,
                     const int8_t* s, double* y)
{
    if (!is_pow2(D)) return -1;
    double* v = (double*)malloc(sizeof(double) * (size_t)D);
    if (!v) return -2;
    for (int64_t r = 0; r < n; r++)
        rotate_one(D, x + r * D, lam + r * D, s, v, y + r * D);
    free(v);
    return 0;
}

/* yhat [n, D] fp64 rotated-domain values -> xhat64 [n, D], and optionally the
   binary16 rounding of it (xhat16 may be NULL). */
int kvqo_unrotate_rows(int64_t n, int D, const double* yhat, const float* lam,
                       const int8_t* s, double* xhat64, uint16_t* xhat16)
{
    if (!is_pow2(D)) return -1;
    for (int64_t r = 0; r < n; r++) {
        unrotate_one(D, yhat + r * D, lam + r * D, s, xhat64 + r * D);
        if (xhat16)
            for (int j = 0; j < D; j++)
                xhat16[r * D + j] = kvqo_f64_to_f16(xhat64[r * D + j]);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Sign-randomized real Fourier rotation (SRFT) [GIST s.1, s.2]               */
/* ------------------------------------------------------------------------ */

/* cos and sin of 2*pi*t/D for t = 0 .. D-1 (the phase j*k is reduced modulo
   D before the lookup, so no large argument reaches cos or sin). */
static void dft_table(int D, double* c, double* sn)
{
    const double pi = 3.14159265358979323846;
    for (int t = 0; t < D; t++) {
        double a = 2.0 * pi * (double)t / (double)D;
        c[t] = cos(a);
        sn[t] = sin(a);
    }
}

/* Forward SRFT of one vector, D even:
     v_j = s_j * lambda_j * x_j;
     X_k = D^-1/2 * sum_j v_j * exp(-2 pi i j k / D)    (unitary DFT);
   v is real, so X_{D-k} = conj(X_k) and X_0, X_{D/2} are real.  The real
   packing keeps one copy of each conjugate pair, scaled so that the map is
   orthonormal:
     y_0 = X_0,  y_1 = X_{D/2},
     y_{2k} = sqrt(2) Re X_k,  y_{2k+1} = sqrt(2) Im X_k   (0 < k < D/2). */
static void srft_one(int D, const uint16_t* x, const float* lam, const int8_t* s,
                     double* v, double* y, const double* c, const double* sn)
{
    for (int j = 0; j < D; j++)
        v[j] = (double)s[j] * (double)lam[j] * kvqo_f16_to_f64(x[j]);
    double norm = 1.0 / sqrt((double)D);
    for (int k = 0; k <= D / 2; k++) {
        double re = 0.0, im = 0.0;
        for (int j = 0; j < D; j++) {
            int t = (int)(((int64_t)j * k) % D);
            re += v[j] * c[t];
            im -= v[j] * sn[t];
        }
        re *= norm;
        im *= norm;
        if (k == 0) y[0] = re;
        else if (k == D / 2) y[1] = re;
        else { y[2 * k] = sqrt(2.0) * re; y[2 * k + 1] = sqrt(2.0) * im; }
    }
}

/* Inverse: rebuild X from the packing (X_k = (y_{2k} + i y_{2k+1}) / sqrt 2)
   and take the unitary inverse DFT, whose result is real:
     v_j = D^-1/2 [ y_0 + (-1)^j y_1
                    + sqrt(2) sum_{0<k<D/2} (y_{2k} cos(2 pi jk/D) - y_{2k+1} sin(2 pi jk/D)) ];
   then unscale: xhat_j = (s_j / lambda_j) v_j. */
static void isrft_one(int D, const double* yhat, const float* lam, const int8_t* s,
                      double* xhat, const double* c, const double* sn)
{
    double norm = 1.0 / sqrt((double)D);
    for (int j = 0; j < D; j++) {
        double acc = yhat[0] + ((j & 1) ? -yhat[1] : yhat[1]);
        for (int k = 1; k < D / 2; k++) {
            int t = (int)(((int64_t)j * k) % D);
            acc += sqrt(2.0) * (yhat[2 * k] * c[t] - yhat[2 * k + 1] * sn[t]);
        }
        xhat[j] = ((double)s[j] / (double)lam[j]) * (acc * norm);
    }
}

int kvqo_srft_rows(int64_t n, int D, const uint16_t* x, const float* lam,
                   const int8_t* s, double* y)
{
    if (D < 2 || (D & 1)) return -1;
    double* v = (double*)malloc(sizeof(double) * (size_t)D * 3);
    double* c = v + D;
    double* sn = c + D;
    dft_table(D, c, sn);
    for (int64_t r = 0; r < n; r++)
        srft_one(D, x + r * D, lam + r * D, s, v, y + r * D, c, sn);
    free(v);
    return 0;
}

int kvqo_isrft_rows(int64_t n, int D, const double* yhat, const float* lam,
                    const int8_t* s, double* xhat64, uint16_t* xhat16)
{
    if (D < 2 || (D & 1)) return -1;
    double* c = (double*)malloc(sizeof(double) * (size_t)D * 2);
    double* sn = c + D;
    dft_table(D, c, sn);
    for (int64_t r = 0; r < n; r++) {
        isrft_one(D, yhat + r * D, lam + r * D, s, xhat64 + r * D, c, sn);
        if (xhat16)
            for (int j = 0; j < D; j++)
                xhat16[r * D + j] = kvqo_f64_to_f16(xhat64[r * D + j]);
    }
    free(c);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Group quantizer and nibble format [ABSTRACT; GIST s.2, s.3]                 */
/* ------------------------------------------------------------------------ */

/* Code of one rotated value given the stored (binary16-decoded) scale of its
   group: 0 for a zero scale, else round-half-even of y/scale clamped to
   [-7, 7]. */
static int code_of(double y, double scale)
{
    if (scale == 0.0) return 0;
    double r = nearbyint(y / scale);
    if (r > 7.0) r = 7.0;
    if (r < -7.0) r = -7.0;
    return (int)r;
}

/* Byte k holds element 2k in bits 0..3 and element 2k+1 in bits 4..7, each
   as 4-bit two's complement. */
void kvqo_pack_nibbles(int64_t n_codes, const int8_t* q, uint8_t* bytes)
{
    for (int64_t k = 0; k < n_codes / 2; k++)
        bytes[k] = (uint8_t)(((unsigned)q[2 * k] & 0xfu) |
                             (((unsigned)q[2 * k + 1] & 0xfu) << 4));
}

void kvqo_unpack_nibbles(int64_t n_bytes, const uint8_t* bytes, int8_t* q)
{
    for (int64_t k = 0; k < n_bytes; k++) {
        int lo = bytes[k] & 0xf, hi = (bytes[k] >> 4) & 0xf;
        q[2 * k] = (int8_t)(lo >= 8 ? lo - 16 : lo);
        q[2 * k + 1] = (int8_t)(hi >= 8 ? hi - 16 : hi);
    }
}

/* Codes of rotated vectors y [n, D] under given binary16 scales [n, D/G]
   (unpacked, one int8 per coordinate). Used both by the quantizer and to
   condition a comparison on another implementation's stored scale. */
int kvqo_codes_given_scales(int64_t n, int D, int G, const double* y,
                            const uint16_t* scales, int8_t* q)
{
    if (G <= 0 || D % G) return -1;
    int ng = D / G;
    for (int64_t r = 0; r < n; r++)
        for (int i = 0; i < D; i++)
            q[r * D + i] = (int8_t)code_of(y[r * D + i],
                                           kvqo_f16_to_f64(scales[r * ng + i / G]));
    return 0;
}

/* Quantize n vectors.  x [n, D] binary16, lam [n, D], s [D];
   codes [n, D/2] packed bytes, scales [n, D/G] binary16 bits; y_out [n, D]
   (may be NULL) receives the fp64 rotated values.
   Per group g (coordinates gG .. gG+G-1):
     amax = max |y_i|;  scale = binary16_rne(amax / 7);
     q_i = clamp(rne(y_i / scale), -7, 7)  (0 when scale == 0).
   Returns the number of vectors outside the domain (a non-finite input or a
   scale that overflows binary16); their outputs are set to zero. */
static int64_t quantize_rows_with(int fourier, int64_t n, int D, int G, const uint16_t* x,
                                  const float* lam, const int8_t* s, uint8_t* codes,
                                  uint16_t* scales, double* y_out)
{
    if (fourier ? (D < 2 || (D & 1)) : !is_pow2(D)) return -1;
    if (G <= 0 || D % G || (G & 1)) return -1;
    int ng = D / G;
    double* v = (double*)malloc(sizeof(double) * (size_t)D);
    double* y = (double*)malloc(sizeof(double) * (size_t)D);
    double* c = (double*)malloc(sizeof(double) * (size_t)D * 2);
    double* sn = c + D;
    int8_t* q = (int8_t*)malloc((size_t)D);
    if (fourier) dft_table(D, c, sn);
    int64_t bad = 0;
    for (int64_t r = 0; r < n; r++) {
        int ok = 1;
        for (int j = 0; j < D; j++)
            if (!isfinite(kvqo_f16_to_f64(x[r * D + j]))) ok = 0;
        if (ok && fourier) srft_one(D, x + r * D, lam + r * D, s, v, y, c, sn);
        else if (ok) rotate_one(D, x + r * D, lam + r * D, s, v, y);
        for (int g = 0; ok && g < ng; g++) {
            double amax = 0.0;
            for (int i = g * G; i < (g + 1) * G; i++)
                if (fabs(y[i]) > amax) amax = fabs(y[i]);
            uint16_t sc = kvqo_f64_to_f16(amax / 7.0);
            if ((sc & 0x7c00) == 0x7c00) { ok = 0; break; }
            scales[r * ng + g] = sc;
            double sbar = kvqo_f16_to_f64(sc);
            for (int i = g * G; i < (g + 1) * G; i++) q[i] = (int8_t)code_of(y[i], sbar);
        }
        if (!ok) {
            bad++;
            memset(codes + r * (D / 2), 0, (size_t)(D / 2));
            memset(scales + r * ng, 0, sizeof(uint16_t) * (size_t)ng);
            if (y_out) for (int i = 0; i < D; i++) y_out[r * D + i] = NAN;
            continue;
        }
        kvqo_pack_nibbles(D, q, codes + r * (D / 2));
        if (y_out) memcpy(y_out + r * D, y, sizeof(double) * (size_t)D);
    }
    free(v); free(y); free(c); free(q);
    return bad;
}

int64_t kvqo_quantize_rows(int64_t n, int D, int G, const uint16_t* x,
                           const float* lam, const int8_t* s, uint8_t* codes,
                           uint16_t* scales, double* y_out)
{
    return quantize_rows_with(0, n, D, G, x, lam, s, codes, scales, y_out);
}

/* The same group quantizer on the SRFT rotation (D even). */
int64_t kvqo_quantize_srft_rows(int64_t n, int D, int G, const uint16_t* x,
                                const float* lam, const int8_t* s, uint8_t* codes,
                                uint16_t* scales, double* y_out)
{
    return quantize_rows_with(1, n, D, G, x, lam, s, codes, scales, y_out);
}

/* Dequantize n vectors from packed codes [n, D/2] and binary16 scales
   [n, D/G] [VQ-blog: dequantize -> inverse transform -> unscale]:
     yhat_i = q_i * scale_g;  xhat = unrotate(yhat);
   xhat64 [n, D] receives the exact fp64 result and xhat16 [n, D] (may be
   NULL) its binary16 rounding. */
static int dequantize_rows_with(int fourier, int64_t n, int D, int G, const uint8_t* codes,
                                const uint16_t* scales, const float* lam,
                                const int8_t* s, double* xhat64, uint16_t* xhat16)
{
    if (fourier ? (D < 2 || (D & 1)) : !is_pow2(D)) return -1;
    if (G <= 0 || D % G || (G & 1)) return -1;
    int ng = D / G;
    int8_t* q = (int8_t*)malloc((size_t)D);
    double* yh = (double*)malloc(sizeof(double) * (size_t)D);
    double* c = (double*)malloc(sizeof(double) * (size_t)D * 2);
    double* sn = c + D;
    if (fourier) dft_table(D, c, sn);
    for (int64_t r = 0; r < n; r++) {
        kvqo_unpack_nibbles(D / 2, codes + r * (D / 2), q);
        for (int i = 0; i < D; i++)
            yh[i] = (double)q[i] * kvqo_f16_to_f64(scales[r * ng + i / G]);
        if (fourier) isrft_one(D, yh, lam + r * D, s, xhat64 + r * D, c, sn);
        else unrotate_one(D, yh, lam + r * D, s, xhat64 + r * D);
        if (xhat16)
            for (int j = 0; j < D; j++)
                xhat16[r * D + j] = kvqo_f64_to_f16(xhat64[r * D + j]);
    }
    free(q); free(yh); free(c);
    return 0;
}

int kvqo_dequantize_rows(int64_t n, int D, int G, const uint8_t* codes,
                         const uint16_t* scales, const float* lam,
                         const int8_t* s, double* xhat64, uint16_t* xhat16)
{
    return dequantize_rows_with(0, n, D, G, codes, scales, lam, s, xhat64, xhat16);
}

/* Mirror of kvqo_quantize_srft_rows: yhat_i = q_i * scale_g, then the inverse
   SRFT and unscale. */
int kvqo_dequantize_srft_rows(int64_t n, int D, int G, const uint8_t* codes,
                              const uint16_t* scales, const float* lam,
                              const int8_t* s, double* xhat64, uint16_t* xhat16)
{
    return dequantize_rows_with(1, n, D, G, codes, scales, lam, s, xhat64, xhat16);
}

/* ------------------------------------------------------------------------ */
/* int8 variant [GIST s.2: the fused kernel rounds to signed int4 or int8]    */
/* ------------------------------------------------------------------------ */

/* Same rotation and groups as the int4 quantizer, with 127 levels each side:
     scale = binary16_rne(amax / 127);
     q_i = clamp(rne(y_i / scale), -127, 127)  (0 when scale == 0),
   one two's-complement byte per coordinate (element i in byte i). */
static int code8_of(double y, double scale)
{
    if (scale == 0.0) return 0;
    double r = nearbyint(y / scale);
    if (r > 127.0) r = 127.0;
    if (r < -127.0) r = -127.0;
    return (int)r;
}

int kvqo_codes8_given_scales(int64_t n, int D, int G, const double* y,
                             const uint16_t* scales, int8_t* q)
{
    if (G <= 0 || D % G) return -1;
    int ng = D / G;
    for (int64_t r = 0; r < n; r++)
        for (int i = 0; i < D; i++)
            q[r * D + i] = (int8_t)code8_of(y[r * D + i],
                                            kvqo_f16_to_f64(scales[r * ng + i / G]));
    return 0;
}

/* Quantize n vectors to int8 codes [n, D] and binary16 scales [n, D/G];
   y_out [n, D] (may be NULL) receives the fp64 rotated values.  Returns the
   number of vectors outside the domain (zeroed), as kvqo_quantize_rows. */
int64_t kvqo_quantize8_rows(int64_t n, int D, int G, const uint16_t* x,
                            const float* lam, const int8_t* s, int8_t* codes,
                            uint16_t* scales, double* y_out)
{
    if (!is_pow2(D) || G <= 0 || D % G || (G & 1)) return -1;
    int ng = D / G;
    double* v = (double*)malloc(sizeof(double) * (size_t)D);
    double* y = (double*)malloc(sizeof(double) * (size_t)D);
    int64_t bad = 0;
    for (int64_t r = 0; r < n; r++) {
        int ok = 1;
        for (int j = 0; j < D; j++)
            if (!isfinite(kvqo_f16_to_f64(x[r * D + j]))) ok = 0;
        if (ok) rotate_one(D, x + r * D, lam + r * D, s, v, y);
        for (int g = 0; ok && g < ng; g++) {
            double amax = 0.0;
            for (int i = g * G; i < (g + 1) * G; i++)
                if (fabs(y[i]) > amax) amax = fabs(y[i]);
            uint16_t sc = kvqo_f64_to_f16(amax / 127.0);
            if ((sc & 0x7c00) == 0x7c00) { ok = 0; break; }
            scales[r * ng + g] = sc;
            double sbar = kvqo_f16_to_f64(sc);
            for (int i = g * G; i < (g + 1) * G; i++) codes[r * D + i] = (int8_t)code8_of(y[i], sbar);
        }
        if (!ok) {
            bad++;
            memset(codes + r * D, 0, (size_t)D);
            memset(scales + r * ng, 0, sizeof(uint16_t) * (size_t)ng);
            if (y_out) for (int i = 0; i < D; i++) y_out[r * D + i] = NAN;
            continue;
        }
        if (y_out) memcpy(y_out + r * D, y, sizeof(double) * (size_t)D);
    }
    free(v); free(y);
    return bad;
}

/* Dequantize n int8 vectors: yhat_i = q_i * scale_g, xhat = unrotate(yhat). */
int kvqo_dequantize8_rows(int64_t n, int D, int G, const int8_t* codes,
                          const uint16_t* scales, const float* lam,
                          const int8_t* s, double* xhat64, uint16_t* xhat16)
{
    if (!is_pow2(D) || G <= 0 || D % G || (G & 1)) return -1;
    int ng = D / G;
    double* yh = (double*)malloc(sizeof(double) * (size_t)D);
    for (int64_t r = 0; r < n; r++) {
        for (int i = 0; i < D; i++)
            yh[i] = (double)codes[r * D + i] * kvqo_f16_to_f64(scales[r * ng + i / G]);
        unrotate_one(D, yh, lam + r * D, s, xhat64 + r * D);
        if (xhat16)
            for (int j = 0; j < D; j++)
                xhat16[r * D + j] = kvqo_f64_to_f16(xhat64[r * D + j]);
    }
    free(yh);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Block-scaled E2M1 (MXFP4) variant [POLAR: "block-scaled E2M1 FP4";         */
/* the format itself as the OCP Microscaling (MX) v1.0 definition]            */
/* ------------------------------------------------------------------------ */

/* E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0; exponent 0
   is subnormal (mantissa * 0.5).  Magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6. */
double kvqo_e2m1_value(int code)
{
    int e = (code >> 1) & 3, m = code & 1;
    double mag = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return (code & 8) ? -mag : mag;
}

/* Nearest E2M1 code of v, ties to the even code (mantissa bit 0), magnitudes
   above 6 saturating to 6; the sign bit is v's sign bit (so -0 -> 0x8). */
static int e2m1_code(double v)
{
    double a = fabs(v);
    int mag;
    if (a >= 6.0) {
        mag = 7;
    } else {
        mag = 0;
        while (mag < 7 && kvqo_e2m1_value(mag + 1) <= a) mag++;
        double lo = kvqo_e2m1_value(mag), hi = kvqo_e2m1_value(mag + 1);
        if (a - lo > hi - a || (a - lo == hi - a && (mag & 1))) mag++;
    }
    return (signbit(v) ? 8 : 0) | mag;
}

/* Shared block exponent of a 32-element block with abs-max amax:
   floor(log2(amax)) - 2 (the largest E2M1 exponent), clamped to
   [-127, 127]; -127 for an all-zero block.  Stored as E8M0: e + 127. */
static int mx_exponent(double amax)
{
    if (amax == 0.0) return -127;
    int E;
    frexp(amax, &E);                 /* amax = f * 2^E, f in [0.5, 1) */
    int e = (E - 1) - 2;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

/* Quantize n vectors: same rotation as the int4 quantizer, then blocks of 32
   rotated coordinates: X = 2^e with e = mx_exponent(amax), code_i =
   e2m1_code(y_i / X).  codes [n, D/2] packed like the int4 nibbles (element
   2k in the low nibble of byte k); scales [n, D/32] E8M0 bytes (e + 127).
   Returns the number of vectors outside the domain (non-finite input),
   zeroed. */
int64_t kvqo_quantize_mxfp4_rows(int64_t n, int D, const uint16_t* x, const float* lam,
                                 const int8_t* s, uint8_t* codes, uint8_t* scales, double* y_out)
{
    if (!is_pow2(D) || D < 32) return -1;
    int nb = D / 32;
    double* v = (double*)malloc(sizeof(double) * (size_t)D);
    double* y = (double*)malloc(sizeof(double) * (size_t)D);
    int8_t* q = (int8_t*)malloc((size_t)D);
    int64_t bad = 0;
    for (int64_t r = 0; r < n; r++) {
        int ok = 1;
        for (int j = 0; j < D; j++)
            if (!isfinite(kvqo_f16_to_f64(x[r * D + j]))) ok = 0;
        if (!ok) {
            bad++;
            memset(codes + r * (D / 2), 0, (size_t)(D / 2));
            memset(scales + r * nb, 0, (size_t)nb);
            if (y_out) for (int i = 0; i < D; i++) y_out[r * D + i] = NAN;
            continue;
        }
        rotate_one(D, x + r * D, lam + r * D, s, v, y);
        for (int b = 0; b < nb; b++) {
            double amax = 0.0;
            for (int i = 32 * b; i < 32 * (b + 1); i++)
                if (fabs(y[i]) > amax) amax = fabs(y[i]);
            int e = mx_exponent(amax);
            scales[r * nb + b] = (uint8_t)(e + 127);
            for (int i = 32 * b; i < 32 * (b + 1); i++) q[i] = (int8_t)e2m1_code(ldexp(y[i], -e));
        }
        for (int k = 0; k < D / 2; k++)
            codes[r * (D / 2) + k] = (uint8_t)((q[2 * k] & 0xf) | ((q[2 * k + 1] & 0xf) << 4));
        if (y_out) memcpy(y_out + r * D, y, sizeof(double) * (size_t)D);
    }
    free(v); free(y); free(q);
    return bad;
}

/* E2M1 codes [n, D] (one per byte, low nibble) of rotated values y [n, D]
   under given E8M0 block scales [n, D/32]. */
int kvqo_mxfp4_codes_given_scales(int64_t n, int D, const double* y, const uint8_t* scales, uint8_t* q)
{
    if (D % 32) return -1;
    int nb = D / 32;
    for (int64_t r = 0; r < n; r++)
        for (int i = 0; i < D; i++)
            q[r * D + i] = (uint8_t)e2m1_code(ldexp(y[r * D + i], -((int)scales[r * nb + i / 32] - 127)));
    return 0;
}

/* Dequantize: yhat_i = 2^(scale_b - 127) * value(code_i), then unrotate. */
int kvqo_dequantize_mxfp4_rows(int64_t n, int D, const uint8_t* codes, const uint8_t* scales,
                               const float* lam, const int8_t* s, double* xhat64, uint16_t* xhat16)
{
    if (!is_pow2(D) || D < 32) return -1;
    int nb = D / 32;
    double* yh = (double*)malloc(sizeof(double) * (size_t)D);
    for (int64_t r = 0; r < n; r++) {
        for (int i = 0; i < D; i++) {
            int byte = codes[r * (D / 2) + i / 2];
            int c = (i & 1) ? (byte >> 4) & 0xf : byte & 0xf;
            yh[i] = ldexp(kvqo_e2m1_value(c), (int)scales[r * nb + i / 32] - 127);
        }
        unrotate_one(D, yh, lam + r * D, s, xhat64 + r * D);
        if (xhat16)
            for (int j = 0; j < D; j++)
                xhat16[r * D + j] = kvqo_f64_to_f16(xhat64[r * D + j]);
    }
    free(yh);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Product VQ [README "Metal kernels"; VQ-blog "What VecInfer does"]           */
/* ------------------------------------------------------------------------ */

/* Squared distance between sub-vector ysub[0..sub) and centroid k of a
   [K, sub] binary16 codebook, in fp64 (direct form). */
static double subdist(int sub, const double* ysub, const uint16_t* cb, int k)
{
    double d = 0.0;
    for (int t = 0; t < sub; t++) {
        double diff = ysub[t] - kvqo_f16_to_f64(cb[(int64_t)k * sub + t]);
        d += diff * diff;
    }
    return d;
}

/* Encode n vectors: rotate each (same rotation as the scalar quantizer, no
   group quantizer), split into D/sub contiguous sub-vectors, and give each the
   lowest index k attaining the minimum squared distance to centroid k.
   codebooks [n_books, K, sub] binary16; book [n] picks each vector's codebook
   (the vector's KV head); idx [n, D/sub]; y_out (may be NULL) [n, D]. */
int kvqo_vq_encode_rows(int64_t n, int D, int sub, int K, const uint16_t* x,
                        const float* lam, const int8_t* s,
                        const uint16_t* codebooks, const int32_t* book,
                        uint16_t* idx, double* y_out)
{
    if (!is_pow2(D) || sub <= 0 || D % sub || K <= 0 || K > 65536) return -1;
    int nsub = D / sub;
    double* v = (double*)malloc(sizeof(double) * (size_t)D);
    double* y = (double*)malloc(sizeof(double) * (size_t)D);
    for (int64_t r = 0; r < n; r++) {
        rotate_one(D, x + r * D, lam + r * D, s, v, y);
        const uint16_t* cb = codebooks + (int64_t)book[r] * K * sub;
        for (int j = 0; j < nsub; j++) {
            int best = 0;
            double bd = subdist(sub, y + j * sub, cb, 0);
            for (int k = 1; k < K; k++) {
                double d = subdist(sub, y + j * sub, cb, k);
                if (d < bd) { bd = d; best = k; }
            }
            idx[r * nsub + j] = (uint16_t)best;
        }
        if (y_out) memcpy(y_out + r * D, y, sizeof(double) * (size_t)D);
    }
    free(v); free(y);
    return 0;
}

/* Distances d[r, j] between sub-vector j of y [n, D] and the centroid that
   idx [n, D/sub] names, in fp64. */
int kvqo_vq_distances(int64_t n, int D, int sub, int K, const double* y,
                      const uint16_t* codebooks, const int32_t* book,
                      const uint16_t* idx, double* d)
{
    if (sub <= 0 || D % sub) return -1;
    int nsub = D / sub;
    for (int64_t r = 0; r < n; r++) {
        const uint16_t* cb = codebooks + (int64_t)book[r] * K * sub;
        for (int j = 0; j < nsub; j++) {
            int k = idx[r * nsub + j];
            if (k >= K) return -2;
            d[r * nsub + j] = subdist(sub, y + r * D + j * sub, cb, k);
        }
    }
    return 0;
}

/* Decode n vectors: yhat = concatenation of the named centroids, then the
   inverse rotation and unscale; xhat64 [n, D], xhat16 [n, D] (may be NULL). */
int kvqo_vq_decode_rows(int64_t n, int D, int sub, int K, const uint16_t* idx,
                        const uint16_t* codebooks, const int32_t* book,
                        const float* lam, const int8_t* s, double* xhat64,
                        uint16_t* xhat16)
{
    if (!is_pow2(D) || sub <= 0 || D % sub || K <= 0) return -1;
    int nsub = D / sub;
    double* yh = (double*)malloc(sizeof(double) * (size_t)D);
    for (int64_t r = 0; r < n; r++) {
        const uint16_t* cb = codebooks + (int64_t)book[r] * K * sub;
        for (int j = 0; j < nsub; j++) {
            int k = idx[r * nsub + j];
            if (k >= K) { free(yh); return -2; }
            for (int t = 0; t < sub; t++)
                yh[j * sub + t] = kvqo_f16_to_f64(cb[(int64_t)k * sub + t]);
        }
        unrotate_one(D, yh, lam + r * D, s, xhat64 + r * D);
        if (xhat16)
            for (int j = 0; j < D; j++)
                xhat16[r * D + j] = kvqo_f64_to_f16(xhat64[r * D + j]);
    }
    free(yh);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Codebook training: one Lloyd (k-means) step [VQ-blog "What VecInfer does,  */
/* and the calibration caveat up front"]                                       */
/* ------------------------------------------------------------------------ */

/* The update half of a Lloyd iteration, given each sample's assignment.
   ysub [n, sub] are the samples (rotated sub-vectors, fp64) and idx [n] their
   assigned centroids (the nearest one in cb_old, as kvqo_vq_encode_rows gives
   them).  For every centroid k of the [K, sub] binary16 codebook cb_old:
     counts[k]   = number of samples assigned to k;
     mean64[k]   = their mean, in fp64; a centroid with no samples keeps its
                   old value;
     cb_new[k]   = binary16 RNE of mean64[k] (cb_old[k] unchanged if empty);
     abs_mean[k] = mean of |y| per coordinate over its samples (0 if empty),
                   a scale for judging a summation in lower precision.
   Returns -2 if an assignment is out of range. */
int kvqo_kmeans_update(int64_t n, int sub, int K, const double* ysub, const uint16_t* idx,
                       const uint16_t* cb_old, double* mean64, uint16_t* cb_new,
                       uint32_t* counts, double* abs_mean)
{
    if (sub <= 0 || K <= 0 || K > 65536) return -1;
    for (int64_t k = 0; k < (int64_t)K * sub; k++) { mean64[k] = 0.0; abs_mean[k] = 0.0; }
    for (int k = 0; k < K; k++) counts[k] = 0;
    for (int64_t i = 0; i < n; i++) {
        int k = idx[i];
        if (k >= K) return -2;
        counts[k]++;
        for (int t = 0; t < sub; t++) {
            mean64[(int64_t)k * sub + t] += ysub[i * sub + t];
            abs_mean[(int64_t)k * sub + t] += fabs(ysub[i * sub + t]);
        }
    }
    for (int k = 0; k < K; k++) {
        for (int t = 0; t < sub; t++) {
            int64_t e = (int64_t)k * sub + t;
            if (counts[k] == 0) {
                mean64[e] = kvqo_f16_to_f64(cb_old[e]);
                cb_new[e] = cb_old[e];
            } else {
                mean64[e] /= (double)counts[k];
                abs_mean[e] /= (double)counts[k];
                cb_new[e] = kvqo_f64_to_f16(mean64[e]);
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Decode attention over the int4 cache [SCALAR-ATTEND]                       */
/* ------------------------------------------------------------------------ */

/* One decode step of softmax attention for R query heads per KV head (query
   head j reads KV head j / R), over the first len[l] tokens of each outer
   index l (len == NULL: all T tokens):
     khat_t = dequantize(K codes_t, K scales_t)   (exact fp64, never rounded)
     vhat_t = dequantize(V codes_t, V scales_t)
     a_t = scale * (q_j . khat_t),  p = softmax over t of a,  out_j = sum p_t vhat_t
   The softmax subtracts the largest a_t before exponentiating.  Layouts,
   all contiguous: q [L, H*R, D] binary16; codes [L, T, H, D/2]; scales
   [L, T, H, D/G] binary16; lamK, lamV [L, H, D]; out64 [L, H*R, D].  An
   outer index with len 0 gets zeros. */
int kvqo_attend_decode(int L, int T, int H, int R, int D, int G, const uint16_t* q,
                       const uint8_t* kc, const uint16_t* ks, const uint8_t* vc,
                       const uint16_t* vs, const float* lamK, const float* lamV,
                       const int8_t* s, const int32_t* len, double scale, double* out64)
{
    if (!is_pow2(D) || G <= 0 || D % G || (G & 1) || L < 0 || T < 0 || H <= 0 || R <= 0) return -1;
    int ng = D / G;
    double* kh = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1) * D);
    double* vh = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1) * D);
    double* a = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
    for (int l = 0; l < L; l++) {
        int n = len ? len[l] : T;
        if (n < 0 || n > T) { free(kh); free(vh); free(a); return -2; }
        for (int h = 0; h < H; h++) {
            const float* lk = lamK + ((int64_t)l * H + h) * D;
            const float* lv = lamV + ((int64_t)l * H + h) * D;
            for (int t = 0; t < n; t++) {
                int64_t row = ((int64_t)l * T + t) * H + h;
                kvqo_dequantize_rows(1, D, G, kc + row * (D / 2), ks + row * ng, lk, s, kh + (int64_t)t * D, NULL);
                kvqo_dequantize_rows(1, D, G, vc + row * (D / 2), vs + row * ng, lv, s, vh + (int64_t)t * D, NULL);
            }
            for (int r = 0; r < R; r++) {
                int j = h * R + r;
                const uint16_t* qj = q + ((int64_t)l * H * R + j) * D;
                double* o = out64 + ((int64_t)l * H * R + j) * D;
                for (int c = 0; c < D; c++) o[c] = 0.0;
                if (n == 0) continue;
                double amax = -INFINITY;
                for (int t = 0; t < n; t++) {
                    double dot = 0.0;
                    for (int c = 0; c < D; c++) dot += kvqo_f16_to_f64(qj[c]) * kh[(int64_t)t * D + c];
                    a[t] = scale * dot;
                    if (a[t] > amax) amax = a[t];
                }
                double z = 0.0;
                for (int t = 0; t < n; t++) {
                    double w = exp(a[t] - amax);
                    z += w;
                    for (int c = 0; c < D; c++) o[c] += w * vh[(int64_t)t * D + c];
                }
                for (int c = 0; c < D; c++) o[c] /= z;
            }
        }
    }
    free(kh); free(vh); free(a);
    return 0;
}
